"""Shared helpers of the GPU tests: weight caching, comparisons, printing."""
import functools
import sys

import numpy as np

from synth import make_weights, workload


@functools.lru_cache(maxsize=2)
def weights_for(name: str, n_layers=None):
    return make_weights(workload(name), n_layers=n_layers)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(g, o) -> float:
    """max |gpu - oracle| / max |oracle| (the logit-scale relative error)."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    assert np.isfinite(g).all(), "non-finite GPU output"
    return float(np.abs(g - o).max() / max(np.abs(o).max(), 1e-30))


def _gap_bound(g, o) -> float:
    """Twice this step's measured max |gpu - oracle| over the finite logits."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    fin = np.isfinite(g) & np.isfinite(o)
    return 2.0 * float(np.abs(g[fin] - o[fin]).max()) if fin.any() else 0.0


def argmax_ok(g, o) -> bool:
    """Codebook-0 argmax: equal to the oracle's; where the two picks differ,
    the oracle's own logits at them must lie within twice this step's
    measured max |gpu - oracle| (both picks are then consistent with the
    measured error; an error at the bar would not excuse a wrong pick)."""
    g = np.asarray(g)
    o = np.asarray(o)
    ig, io = int(np.argmax(g)), int(np.argmax(o))
    if ig == io:
        return True
    return bool(o[io] - o[ig] <= _gap_bound(g, o))


def argmax_banded(g, o) -> bool:
    """True when the picks differ and argmax_ok accepted the GPU's."""
    return int(np.argmax(g)) != int(np.argmax(o)) and argmax_ok(g, o)
