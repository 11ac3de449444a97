"""CPU oracle of the frame-step glue around the Talker.  TEST INFRASTRUCTURE
ONLY (imported by the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg; never by the HIP library or its binding).

Two plain definitions from the pages:

* the step embedding of a frame slot: the codebook-0 token's row of the codec
  embedding table, plus, for each further codebook g, its token's row of
  acoustic table g, plus the slot's overlay row (the trailing text row)
  ("qwentts.cpp src/talker-forward.h", the batched step graph's
  ``input_embed``: group-major ids, one gather per table, summed, plus the
  overlay; "rightkit-qts 0.2.3 src/pipeline/tts_transformer.rs",
  ``build_talker_step_embedding``).  Summed in float32 in that order (table
  0, table 1, ..., overlay), the order the HIP kernel uses, so the two agree
  bit for bit;
* the greedy codebook-0 pick: logits from ``vocab - 1024`` up are suppressed
  (set to minus infinity) except the end-of-speech id, then the argmax, the
  lowest index among equal maxima ("rightkit-qts 0.2.3
  src/pipeline/tts_transformer.rs", the suppression loop before
  ``select_token``).  ``select_token``'s body is not on the pages; with
  temperature 0 (greedy) it is read as the argmax.  A NaN logit never wins;
  a row with no finite candidate returns the lowest unsuppressed index.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def embed_sum(tables: Sequence[np.ndarray], ids: np.ndarray,
              overlay: Optional[np.ndarray] = None) -> np.ndarray:
    """``out[s] = tables[0][ids[0][s]] + ... + tables[G-1][ids[G-1][s]]
    (+ overlay[s])``, float32, summed left to right.  ``ids`` is
    group-major ``[G][n]``; an id outside its table raises."""
    ids = np.asarray(ids)
    G, n = ids.shape
    if len(tables) != G:
        raise ValueError("one table per group")
    hidden = tables[0].shape[1]
    out = np.zeros((n, hidden), dtype=np.float32)
    for s in range(n):
        acc = None
        for g in range(G):
            i = int(ids[g, s])
            if not 0 <= i < tables[g].shape[0]:
                raise IndexError(f"id {i} outside table {g}")
            row = np.asarray(tables[g][i], dtype=np.float32)
            acc = row.copy() if acc is None else np.float32(acc + row)
        if overlay is not None:
            acc = np.float32(acc + np.asarray(overlay[s], dtype=np.float32))
        out[s] = acc
    return out


def suppressed_argmax(logits: np.ndarray, suppress_begin: int,
                      keep_id: int) -> int:
    """Greedy pick over one row of logits: indices ``>= suppress_begin`` are
    excluded except ``keep_id``; NaN never wins; ties go to the lowest
    index."""
    best, best_i = None, None
    for t, v in enumerate(np.asarray(logits, dtype=np.float64)):
        if t >= suppress_begin and t != keep_id:
            continue
        if best_i is None:
            best_i, best = t, (v if v == v else -np.inf)
            continue
        if v == v and v > best:
            best, best_i = v, t
    return int(best_i)
