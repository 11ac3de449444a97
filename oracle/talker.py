"""CPU oracle of the KV-cached Talker forward.  TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this module.  The product path (the HIP library
and its Python binding) never imports, calls or links it, and it shares no
code with that path.

What it computes is the plain definition of the Talker decoder stack as the
pages state it, written out in NumPy float64 (float32 only when asked, for
timing), one step after another in the pages' order:

* per layer: pre-norm RMSNorm; bias-free Q/K/V projections; per-head RMSNorm
  of q and k over head_dim with a shared ``[head_dim]`` gain; 1-D NEOX rotary
  embedding at the absolute cache position; write of k and v into the cache;
  causal grouped-query attention that reads the cache back; o_proj plus
  residual; post-attention RMSNorm; SwiGLU MLP plus residual
  ("qwentts.cpp src/talker-forward.h", ``talker_layer_forward``;
  "transcribe.cpp src/causal_lm/causal_lm.cpp", ``block_prefill``;
  "rightkit-qts 0.2.3 src/pipeline/tts_transformer.rs", ``forward_prefill``);
* after the stack: final RMSNorm and the codec_head projection to codebook-0
  logits of the last row ("qwentts.cpp src/talker-forward.h",
  ``talker_forward_core``);
* output heads: a model may stack several output projections (the code
  predictor's per-codebook heads); ``select_head`` picks the one that forms
  the logits of the following calls, head 0 for the code predictor's two-row
  prefill and head j at its generation step j ("rightkit-qts 0.2.3
  src/pipeline/tts_transformer.rs", ``forward_code_pred_prefill_cached``,
  ``forward_code_pred_step_cached``);
* cache bookkeeping: prefill rewinds the sequence to 0 and writes T
  positions; decode appends one position at ``cur_len`` and attends to
  ``[0, cur_len + 1)``; ``cur_len`` advances only on success
  ("qwentts.cpp src/talker-forward.h", ``talker_forward_prefill`` and
  ``talker_forward_decode``).

Readings taken where the pages leave a step open (each one is listed with its
reason in the design notes of the repository):

* RMSNorm is ``x / sqrt(mean(x^2) + eps) * g`` (gain applied as is);
* NEOX RoPE rotates the pairs ``(x_i, x_{i + hd/2})`` by ``pos * theta^(-2i/hd)``;
* the query head ``h`` reads KV head ``h // (n_heads / n_kv_heads)``;
* attention reads an f32 or f16 cache after the write, so K and V pass
  through the cache's storage type (float16 rounding for f16 caches) before
  use, in prefill and decode alike;
* float16 rounding of the cache is round-to-nearest-even of the float32 value;
* an 8-bit (Q8_0) cache stores blocks of 32 values along head_dim as int8
  codes and a float16 scale; attention reads the positions written by
  earlier calls dequantised from the cache and the call's own rows
  unquantised ("rightkit-qts 0.2.3 src/pipeline/tts_transformer.rs",
  ``forward_step_cached``: the cached prefix cast back to F32 and joined
  with the current k/v; ``forward_prefill_cached``: attention on the fresh
  k/v).  A q8 prefill therefore differs from the same rows decoded one by
  one, through the quantisation of the rows the decode reads back.

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, invariants, brute force and independent library routines.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np


# ---------------------------------------------------------------------------
# elementary steps


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis, then the gain.

    "qwentts.cpp src/talker-forward.h", ``talker_layer_forward`` (pre-norm:
    ``ggml_rms_norm`` followed by ``ggml_mul`` with the norm weight).
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gain


def rope_inv_freq(head_dim: int, theta: float, dtype=np.float64) -> np.ndarray:
    """Per-pair angular frequency ``theta^(-2i/head_dim)``, ``i < head_dim/2``."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return (float(theta) ** (-2.0 * i / head_dim)).astype(dtype)


def rope_neox(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """NEOX (rotate-half) rotary embedding of the last axis.

    ``pos`` broadcasts against ``x[..., 0]``.  The pages apply ``ggml_rope_ext``
    in NEOX mode over all ``head_dim`` dims with unit frequency scale and no
    extrapolation mix; the multimodal axes collapse to one position
    ("qwentts.cpp src/talker-forward.h", ``talker_layer_forward``, RoPE
    NEOX comment; file header on the collapsed mrope).
    """
    hd = x.shape[-1]
    half = hd // 2
    inv = rope_inv_freq(hd, theta)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c = np.cos(ang).astype(x.dtype)
    s = np.sin(ang).astype(x.dtype)
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    """``z * sigmoid(z)``, written ``z / (1 + exp(-z))``."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """``silu(gate) * up`` ("qwentts.cpp src/talker-forward.h",
    ``talker_layer_forward``, ``ggml_swiglu_split(gate, up)``)."""
    return silu(gate) * up


def q8_block_quantize(x: np.ndarray):
    """Q8_0 quantisation of float32 values in blocks of 32 along the last axis
    (the 8-bit KV storage, "rightkit-qts 0.2.3
    src/pipeline/tts_transformer.rs", ``TalkerKvStorage::TurboQuantQ8_0``,
    which stores K and V in ggml's Q8_0 type).  The pages name the type but
    not its arithmetic; the reading is the block format as that library
    documents it: per block, scale ``d = max|x| / 127`` (float32), codes
    ``q = round_half_away(x * (1 / d))`` in float32 (0 when d is 0), the
    scale stored as float16.  Returns (codes int8 [..., n/32, 32], scales
    float16 [..., n/32])."""
    x = np.asarray(x, dtype=np.float32)
    if x.shape[-1] % 32:
        raise ValueError("last axis must be a multiple of 32")
    b = x.reshape(*x.shape[:-1], x.shape[-1] // 32, 32)
    amax = np.abs(b).max(axis=-1)
    d = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(d > 0, np.float32(1.0) / d, np.float32(0.0)).astype(np.float32)
    v = (b * inv[..., None]).astype(np.float32)
    q = np.sign(v) * np.floor(np.abs(v) + np.float32(0.5))
    return q.astype(np.int8), d.astype(np.float16)


def q8_block_dequantize(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Values of Q8_0 blocks: ``code * float(scale)`` (exact in float32)."""
    v = q.astype(np.float32) * d.astype(np.float32)[..., None]
    return v.reshape(*v.shape[:-2], v.shape[-2] * 32)


def round_kv(z: np.ndarray, kv_dtype: str, dtype) -> np.ndarray:
    """Value the cache holds after storing ``z``: ``float16(float32(z))`` for an
    f16 cache, ``float32(z)`` for an f32 cache, the Q8_0 block round trip of
    ``float32(z)`` for a q8 cache; returned in ``dtype``."""
    if kv_dtype == "q8":
        return q8_block_dequantize(*q8_block_quantize(z.astype(np.float32))).astype(dtype)
    if kv_dtype == "f16":
        return z.astype(np.float32).astype(np.float16).astype(dtype)
    if kv_dtype == "f32":
        return z.astype(np.float32).astype(dtype)
    raise ValueError(kv_dtype)


def causal_gqa_attention(q: np.ndarray, k_cache: np.ndarray,
                         v_cache: np.ndarray, positions: np.ndarray,
                         scale: float) -> np.ndarray:
    """Causal grouped-query attention of T query rows over a cache.

    ``q``: ``[T][n_heads][hd]``; ``k_cache``/``v_cache``: ``[n_kv][>=max+1][hd]``;
    row ``t`` sees keys ``j <= positions[t]`` only.  Softmax subtracts the row
    maximum.  Query head ``h`` uses KV head ``h // G``.  Returns
    ``[T][n_heads][hd]``.

    "qwentts.cpp src/talker-forward.h", ``talker_attn_f32`` (scores, masked
    scaled softmax, weighted sum of V) and the causal mask built in
    ``talker_forward_core`` (zero where key <= n_past + q);
    "transcribe.cpp src/causal_lm/causal_lm.cpp", ``block_prefill`` (manual
    GQA path: each KV head repeated for its group of consecutive q heads).
    """
    T, nq, hd = q.shape
    nkv = k_cache.shape[0]
    G = nq // nkv
    n_ctx = int(positions.max()) + 1
    key_idx = np.arange(n_ctx)
    visible = key_idx[None, :] <= positions[:, None]          # [T][n_ctx]
    out = np.empty_like(q)
    for h in range(nq):
        g = h // G
        s = (q[:, h, :] @ k_cache[g, :n_ctx, :].T) * scale       # [T][n_ctx]
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v_cache[g, :n_ctx, :]
    return out


# ---------------------------------------------------------------------------
# the model


class TalkerOracle:
    """KV-cached Talker forward on the CPU, float64 by default.

    ``weights`` is ``{"layers": [dict(wq, wk, wv, wo, wg, wu, wd, g_in, g_post,
    g_q, g_k)], "g_final", "w_head"}`` with ``[out][in]`` projection matrices.
    """

    def __init__(self, shape, weights: Dict, dtype=np.float64):
        self.s = shape
        self.dtype = dtype
        cv = lambda a: np.asarray(a, dtype=dtype)
        self.layers = [{k: cv(v) for k, v in lw.items()}
                       for lw in weights["layers"]]
        self.L = len(self.layers)
        self.g_final = cv(weights["g_final"])
        heads = cv(weights["w_head"])
        self.w_heads = heads if heads.ndim == 3 else heads[None]
        self.w_head = self.w_heads[0]
        self.scale = 1.0 / np.sqrt(shape.head_dim)
        # per sequence: K and V [L][n_kv][alloc][hd], grown on demand
        self.kc: List[Optional[np.ndarray]] = [None] * shape.n_seqs
        self.vc: List[Optional[np.ndarray]] = [None] * shape.n_seqs
        self.cur_len = [0] * shape.n_seqs

    # -- cache bookkeeping ---------------------------------------------------
    def _reserve(self, seq: int, n: int) -> None:
        s = self.s
        have = 0 if self.kc[seq] is None else self.kc[seq].shape[2]
        if n <= have:
            return
        new = max(n, 2 * have, 64)
        shp = (self.L, s.n_kv_heads, new, s.head_dim)
        k = np.zeros(shp, dtype=self.dtype)
        v = np.zeros(shp, dtype=self.dtype)
        if have:
            k[:, :, :have] = self.kc[seq]
            v[:, :, :have] = self.vc[seq]
        self.kc[seq], self.vc[seq] = k, v

    def kv_len(self, seq: int) -> int:
        return self.cur_len[seq]

    def kv_rewind(self, seq: int, n_keep: int) -> None:
        """Truncate ``seq`` to its first ``n_keep`` positions."""
        if not 0 <= n_keep <= self.cur_len[seq]:
            raise ValueError("n_keep out of range")
        self.cur_len[seq] = n_keep

    def kv(self, seq: int, layer: int, which: int) -> np.ndarray:
        """Cache content ``[n_kv][cur_len][hd]`` (0 = K, 1 = V)."""
        c = self.kc[seq] if which == 0 else self.vc[seq]
        n = self.cur_len[seq]
        if c is None:
            return np.zeros((self.s.n_kv_heads, 0, self.s.head_dim), self.dtype)
        return c[layer, :, :n, :].copy()

    # -- one layer -----------------------------------------------------------
    def layer(self, l: int, x: np.ndarray, seq: int, p0: int) -> np.ndarray:
        """Layer ``l`` on rows ``x[T][H]`` at positions ``p0 .. p0+T-1``."""
        s, w = self.s, self.layers[l]
        T = x.shape[0]
        pos = p0 + np.arange(T)
        h = rms_norm(x, w["g_in"], s.rms_eps)
        q = (h @ w["wq"].T).reshape(T, s.n_heads, s.head_dim)
        k = (h @ w["wk"].T).reshape(T, s.n_kv_heads, s.head_dim)
        v = (h @ w["wv"].T).reshape(T, s.n_kv_heads, s.head_dim)
        q = rms_norm(q, w["g_q"], s.rms_eps)
        k = rms_norm(k, w["g_k"], s.rms_eps)
        q = rope_neox(q, pos[:, None], s.rope_theta)
        k = rope_neox(k, pos[:, None], s.rope_theta)
        # write, then read back through the cache
        self.kc[seq][l, :, p0:p0 + T, :] = round_kv(
            k.transpose(1, 0, 2), s.kv_dtype, self.dtype)
        self.vc[seq][l, :, p0:p0 + T, :] = round_kv(
            v.transpose(1, 0, 2), s.kv_dtype, self.dtype)
        ka, va = self.attended_kv(l, seq, p0, k, v)
        o = causal_gqa_attention(q, ka, va, pos, self.scale)
        x = x + o.reshape(T, s.q_dim) @ w["wo"].T
        h2 = rms_norm(x, w["g_post"], s.rms_eps)
        a = swiglu(h2 @ w["wg"].T, h2 @ w["wu"].T)
        return x + a @ w["wd"].T

    def attended_kv(self, l: int, seq: int, p0: int, k: np.ndarray,
                    v: np.ndarray):
        """Keys and values ``[n_kv][p0 + T][hd]`` that the attention of the
        rows at ``p0 .. p0+T-1`` reads, once their ``k``/``v`` (``[T][n_kv][hd]``)
        are in the cache.

        f32 and f16 caches: the cache itself (read after write).  q8 cache:
        positions ``< p0`` dequantised from the cache and the call's own rows
        as computed, unquantised ("rightkit-qts 0.2.3
        src/pipeline/tts_transformer.rs", ``forward_step_cached``,
        ``TalkerKvStorage::TurboQuantQ8_0`` arm: the prefix view of the
        cache cast to F32, concatenated with ``k_cur``/``v_cur``;
        ``forward_prefill_cached`` attends to ``k_cur``/``v_cur``).  The
        pages give no chunked q8 extend; it is read the same way (prefix
        from the cache, the chunk's rows fresh), which holds decode at
        ``T = 1`` and prefill at ``p0 = 0``.
        """
        T = k.shape[0]
        kc, vc = self.kc[seq][l], self.vc[seq][l]
        if self.s.kv_dtype != "q8":
            return kc[:, :p0 + T], vc[:, :p0 + T]
        ka = kc[:, :p0 + T].copy()
        va = vc[:, :p0 + T].copy()
        ka[:, p0:] = k.transpose(1, 0, 2)
        va[:, p0:] = v.transpose(1, 0, 2)
        return ka, va

    def select_head(self, i: int) -> None:
        """Form the logits of the following calls with stacked head ``i``."""
        if not 0 <= i < self.w_heads.shape[0]:
            raise ValueError("head index out of range")
        self.w_head = self.w_heads[i]

    def head(self, x: np.ndarray):
        """Final RMSNorm and codec_head on rows ``x``: (logits, hidden)."""
        hf = rms_norm(x, self.g_final, self.s.rms_eps)
        return hf @ self.w_head.T, hf

    # -- entry points --------------------------------------------------------
    def extend(self, seq: int, emb: np.ndarray, all_rows: bool = False,
               taps: Optional[list] = None):
        """Append ``T`` rows at ``cur_len``; returns (logits, hidden) of the last
        row, or of every row with ``all_rows``.  ``taps`` collects each layer's
        output rows when given."""
        s = self.s
        emb = np.asarray(emb)
        if emb.ndim != 2 or emb.shape[1] != s.hidden or emb.shape[0] < 1:
            raise ValueError("emb must be [T>=1][hidden]")
        if not 0 <= seq < s.n_seqs:
            raise ValueError("bad sequence id")
        p0 = self.cur_len[seq]
        T = emb.shape[0]
        if p0 + T > s.cap:
            raise OverflowError("KV capacity exceeded")
        self._reserve(seq, p0 + T)
        x = emb.astype(self.dtype)
        for l in range(self.L):
            x = self.layer(l, x, seq, p0)
            if taps is not None:
                taps.append(x.copy())
        self.cur_len[seq] = p0 + T
        rows = x if all_rows else x[-1:]
        logits, hidden = self.head(rows)
        if all_rows:
            return logits, hidden
        return logits[0], hidden[0]

    def extend_rows(self, seq: int, emb: np.ndarray, rows: Sequence[int]):
        """Append ``T`` rows at ``cur_len`` like :meth:`extend`, but return
        (logits, hidden) only for the listed rows (indices into ``emb``).

        One-layer models only: there the cache a row writes depends on that
        row's embedding alone (input RMSNorm, K/V projection, QK-norm, RoPE),
        and a row's output depends on its own query and the cache up to its
        position, so the attention of the other rows never has to be formed.
        This lets the long-context workloads be checked on sampled rows
        ("qwentts.cpp src/talker-forward.h", ``talker_layer_forward``: the
        per-row attention over the cache window).
        """
        s = self.s
        if self.L != 1:
            raise ValueError("extend_rows needs a one-layer model")
        emb = np.asarray(emb)
        T = emb.shape[0]
        p0 = self.cur_len[seq]
        if p0 + T > s.cap:
            raise OverflowError("KV capacity exceeded")
        self._reserve(seq, p0 + T)
        w = self.layers[0]
        x = emb.astype(self.dtype)
        pos = p0 + np.arange(T)
        h = rms_norm(x, w["g_in"], s.rms_eps)
        k = (h @ w["wk"].T).reshape(T, s.n_kv_heads, s.head_dim)
        v = (h @ w["wv"].T).reshape(T, s.n_kv_heads, s.head_dim)
        k = rope_neox(rms_norm(k, w["g_k"], s.rms_eps), pos[:, None], s.rope_theta)
        self.kc[seq][0, :, p0:p0 + T, :] = round_kv(k.transpose(1, 0, 2), s.kv_dtype, self.dtype)
        self.vc[seq][0, :, p0:p0 + T, :] = round_kv(v.transpose(1, 0, 2), s.kv_dtype, self.dtype)
        self.cur_len[seq] = p0 + T
        ka, va = self.attended_kv(0, seq, p0, k, v)
        r = np.asarray(list(rows), dtype=np.int64)
        hr = h[r]
        q = (hr @ w["wq"].T).reshape(len(r), s.n_heads, s.head_dim)
        q = rope_neox(rms_norm(q, w["g_q"], s.rms_eps), pos[r][:, None], s.rope_theta)
        o = causal_gqa_attention(q, ka, va, pos[r], self.scale)
        xr = x[r] + o.reshape(len(r), s.q_dim) @ w["wo"].T
        h2 = rms_norm(xr, w["g_post"], s.rms_eps)
        xr = xr + swiglu(h2 @ w["wg"].T, h2 @ w["wu"].T) @ w["wd"].T
        return self.head(xr)

    def prefill(self, seq: int, emb: np.ndarray, all_rows: bool = False):
        """Rewind ``seq`` to 0, then write ``T`` positions."""
        s = self.s
        if np.asarray(emb).shape[0] > s.cap:
            raise OverflowError("KV capacity exceeded")
        self.cur_len[seq] = 0
        return self.extend(seq, emb, all_rows=all_rows)

    def prefill_batch(self, seqs: Sequence[int], embs: np.ndarray):
        """Prefill each listed sequence from ``embs[b]`` ``[T][hidden]``: B
        independent prefills of equal length, each into positions [0, T) of
        its own cache ("transcribe.cpp src/causal_lm/causal_lm.cpp",
        ``block_prefill_batched``); per-sequence (logits, hidden) stacked."""
        seqs = list(seqs)
        if len(set(seqs)) != len(seqs):
            raise ValueError("duplicate sequence id")
        embs = np.asarray(embs)
        if embs.shape[1] > self.s.cap:
            raise OverflowError("KV capacity exceeded")
        outs = [self.prefill(sq, embs[i]) for i, sq in enumerate(seqs)]
        return (np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs]))

    def decode(self, seq: int, emb_row: np.ndarray):
        """One position at ``cur_len``; attends to ``[0, cur_len + 1)``."""
        return self.extend(seq, np.asarray(emb_row).reshape(1, -1))

    def decode_batch(self, seqs: Sequence[int], embs: np.ndarray):
        """One position for each listed sequence; per-row (logits, hidden)."""
        seqs = list(seqs)
        if len(set(seqs)) != len(seqs):
            raise ValueError("duplicate sequence id")
        for sq in seqs:
            if self.cur_len[sq] + 1 > self.s.cap:
                raise OverflowError("KV capacity exceeded")
        outs = [self.decode(sq, embs[i]) for i, sq in enumerate(seqs)]
        return (np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs]))


def code_predictor_frame(orc: TalkerOracle, hidden: np.ndarray,
                         cb0_embedding: np.ndarray,
                         step_embeddings: np.ndarray, seq: int = 0):
    """One frame of the code predictor on the oracle ``orc``: a two-row
    prefill of (the Talker's last hidden state, the codebook-0 embedding)
    read through head 0, then one decode step per further codebook, step j
    (1-based) fed ``step_embeddings[j - 1]`` and read through head j.  Returns
    the list of logits, one per codebook after the first
    ("rightkit-qts 0.2.3 src/pipeline/tts_transformer.rs",
    ``predict_remaining_codebooks_kv_with_cache``).  The step inputs are the
    caller's: on the pages, the previous code's row of embedding table j - 1,
    passed through ``project_input``, taken here as the identity since the
    two hidden sizes agree.
    """
    out = []
    orc.select_head(0)
    lg, _ = orc.prefill(seq, np.stack([hidden, cb0_embedding]))
    out.append(lg)
    for j in range(1, len(step_embeddings) + 1):
        orc.select_head(j)
        lg, _ = orc.decode(seq, step_embeddings[j - 1])
        out.append(lg)
    return out
