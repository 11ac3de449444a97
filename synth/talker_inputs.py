"""Seeded synthetic inputs for the Talker forward: shapes, weights, embeddings.

Nothing in this module computes any part of the forward.  It only fixes the
shapes of the workloads and draws their random inputs, so that the CPU oracle
and the HIP path receive the very same numbers.

Shapes follow the Talker configuration defaults of "rightkit-qts 0.2.3
src/pipeline/tts_transformer.rs" (``TtsTransformerConfig::default``: hidden
1024, 28 layers, 16 query heads, 8 KV heads, head_dim 128, intermediate 3072,
rms eps 1e-6, rope theta 1e6, codec vocab 3072).

Draw recipe (every array is independent and reproducible on its own):

* each array comes from ``numpy.random.default_rng(SeedSequence(key))`` (PCG64)
  with ``key = [seed, tag, ...]``;
* projection weights are ``0.02 * N(0, 1)`` drawn as float32; for bf16-weight
  workloads they are rounded once to the nearest bf16 value (ties to even), so
  the float32 array holds exactly the bf16 numbers both sides use;
* RMSNorm gains (input, post-attention, q, k, final) are ``1 + 0.05 * N(0, 1)``
  in float32 and are never rounded;
* prefill and step embeddings are ``N(0, 1)`` float32 (for the code
  predictor they stand in for the Talker's last hidden state, the codebook-0
  embedding and the per-step table rows);
* stacked output heads (code predictor) draw head i with key
  ``[seed, final tag, 1, i]``;
* the long-context stress workload adds ``sign * 3.0e4`` to four fixed channels
  of every embedding row;
* a workload may scale the q and k norm gains by a constant (``qk_gain``):
  the query-key scores then spread ``qk_gain^2`` times wider, so the softmax
  picks out a few keys even at 32k positions instead of averaging thousands
  (used where a check has to see the attention at long context).

Weight layout is row-major ``[out][in]`` as in the pages' ``mul_mat(W, x)``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

# key tags (second element of every SeedSequence key)
_TAG_FINAL = 10_000
_TAG_PREFILL = 20_000
_TAG_STEP = 30_000
_TAG_OUTLIER = 40_000
_TAG_LENGTHS = 50_000
_TAG_TABLE = 60_000
_TAG_OVERLAY = 70_000

LAYER_TENSORS = ("wq", "wk", "wv", "wo", "wg", "wu", "wd",
                 "g_in", "g_post", "g_q", "g_k")


@dataclasses.dataclass(frozen=True)
class TalkerShape:
    """Model geometry plus cache and workload sizes of one synthetic run."""
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    rms_eps: float
    rope_theta: float
    weight_dtype: str          # "f32" or "bf16"
    kv_dtype: str              # "f32", "f16" or "q8" (Q8_0 blocks of 32)
    cap: int                   # KV capacity per sequence
    n_seqs: int                # KV sets
    seed: int                  # weight seed
    emb_seed: int              # embedding seed
    prefill_len: int = 0       # bs1 prefill length (0: per-sequence lengths)
    decode_steps: int = 0
    chunk: int = 0             # prefill chunk for extend (0: one shot)
    batch_lengths: bool = False
    outliers: bool = False
    n_out_heads: int = 1       # stacked output projections (code predictor: 15)
    qk_gain: float = 1.0       # factor on the q and k norm gains

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def layer_shapes(self) -> Dict[str, tuple]:
        H, I, Q, KV, hd = (self.hidden, self.intermediate, self.q_dim,
                           self.kv_dim, self.head_dim)
        return {"wq": (Q, H), "wk": (KV, H), "wv": (KV, H), "wo": (H, Q),
                "wg": (I, H), "wu": (I, H), "wd": (H, I),
                "g_in": (H,), "g_post": (H,), "g_q": (hd,), "g_k": (hd,)}

    def params_per_layer(self) -> int:
        return sum(int(np.prod(s)) for k, s in self.layer_shapes().items()
                   if k.startswith("w"))

    def with_(self, **kw) -> "TalkerShape":
        return dataclasses.replace(self, **kw)


_TALKER = dict(hidden=1024, n_heads=16, n_kv_heads=8, head_dim=128,
               intermediate=3072, vocab=3072, rms_eps=1e-6, rope_theta=1e6,
               weight_dtype="bf16", kv_dtype="f16")

WORKLOADS: Dict[str, TalkerShape] = {
    # tiny Qwen3-style decoder, float32 weights, activations and cache
    "tiny_f32_2l": TalkerShape(
        name="tiny_f32_2l", n_layers=2, hidden=256, n_heads=4, n_kv_heads=2,
        head_dim=64, intermediate=768, vocab=3072, rms_eps=1e-6,
        rope_theta=1e6, weight_dtype="f32", kv_dtype="f32", cap=64, n_seqs=1,
        seed=1001, emb_seed=1001, prefill_len=16, decode_steps=8),
    # one Talker layer at real shape + final norm + codec head
    "talker_1l_t128": TalkerShape(
        name="talker_1l_t128", n_layers=1, cap=2048, n_seqs=1, seed=1002,
        emb_seed=1002, prefill_len=128, decode_steps=64, **_TALKER),
    # full 28-layer Talker, batch 1, prefill 128 then 1024 steps
    "talker_28l_t128_d1024": TalkerShape(
        name="talker_28l_t128_d1024", n_layers=28, cap=2048, n_seqs=1,
        seed=1003, emb_seed=1003, prefill_len=128, decode_steps=1024,
        **_TALKER),
    # 16 ragged utterances, lengths U{512..4096}, 64 batched decode steps
    "talker_28l_batch16_ragged": TalkerShape(
        name="talker_28l_batch16_ragged", n_layers=28, cap=4160, n_seqs=16,
        seed=1004, emb_seed=1004, decode_steps=64, chunk=2048,
        batch_lengths=True, **_TALKER),
    # 32k context in 2048-row chunks, 256 steps, 3e4 outlier channels
    "talker_28l_ctx32k_outlier": TalkerShape(
        name="talker_28l_ctx32k_outlier", n_layers=28, cap=33024, n_seqs=1,
        seed=1005, emb_seed=1005, prefill_len=32768, decode_steps=256,
        chunk=2048, outliers=True, **_TALKER),
    # one layer of the 32k workload's weights with q/k norm gains x4 and
    # N(0, 1) rows (no outlier channels): sharp attention at 32k positions
    "talker_1l_ctx32k_sharp": TalkerShape(
        name="talker_1l_ctx32k_sharp", n_layers=1, cap=33024, n_seqs=1,
        seed=1005, emb_seed=1005, prefill_len=32768, decode_steps=256,
        chunk=2048, qk_gain=4.0, **_TALKER),
    # bs1 decode at context 1921..2048 on the 28-layer weights of seed 1003
    "talker_28l_kv2k": TalkerShape(
        name="talker_28l_kv2k", n_layers=28, cap=2048, n_seqs=1, seed=1003,
        emb_seed=1006, prefill_len=1920, decode_steps=128, **_TALKER),
    # code predictor: 5 layers of the Talker's block geometry, 15 heads of
    # 2048 codes; per frame a 2-row prefill, then 14 one-token steps
    "code_predictor_5l": TalkerShape(
        name="code_predictor_5l", n_layers=5, cap=16, n_seqs=1, seed=1007,
        emb_seed=1007, prefill_len=2, decode_steps=14, n_out_heads=15,
        **{**_TALKER, "vocab": 2048}),
}


def workload(name: str) -> TalkerShape:
    return WORKLOADS[name]


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of each float32, kept as float32.

    This is the storage format of the weights, applied at draw time; finite
    inputs only.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def _normal(shape, *key) -> np.ndarray:
    return _rng(*key).standard_normal(size=shape, dtype=np.float32)


def make_layer_weights(shape: TalkerShape, layer: int) -> Dict[str, np.ndarray]:
    out = {}
    for tid, (name, shp) in enumerate(shape.layer_shapes().items()):
        z = _normal(shp, shape.seed, layer, tid)
        if name.startswith("w"):
            w = np.float32(0.02) * z
            if shape.weight_dtype == "bf16":
                w = round_to_bf16(w)
            out[name] = w
        else:
            g = np.float32(1.0) + np.float32(0.05) * z
            if name in ("g_q", "g_k") and shape.qk_gain != 1.0:
                g = np.float32(shape.qk_gain) * g
            out[name] = g
    return out


def make_weights(shape: TalkerShape, n_layers: Optional[int] = None) -> Dict:
    """All weights as float32 arrays: ``{"layers": [...], "g_final", "w_head"}``."""
    L = shape.n_layers if n_layers is None else n_layers
    layers: List[Dict[str, np.ndarray]] = [make_layer_weights(shape, l)
                                           for l in range(L)]
    g_final = np.float32(1.0) + np.float32(0.05) * _normal(
        (shape.hidden,), shape.seed, _TAG_FINAL, 0)
    if shape.n_out_heads == 1:
        w_head = np.float32(0.02) * _normal((shape.vocab, shape.hidden),
                                            shape.seed, _TAG_FINAL, 1)
    else:
        w_head = np.float32(0.02) * np.stack([
            _normal((shape.vocab, shape.hidden), shape.seed, _TAG_FINAL, 1, i)
            for i in range(shape.n_out_heads)])
    if shape.weight_dtype == "bf16":
        w_head = round_to_bf16(w_head)
    return {"layers": layers, "g_final": g_final, "w_head": w_head}


def outlier_channels(shape: TalkerShape):
    """Four distinct channels and their fixed signs (+, -, +, -)."""
    ch = _rng(shape.emb_seed, _TAG_OUTLIER).choice(shape.hidden, size=4,
                                                   replace=False)
    return np.sort(ch).astype(np.int64), np.array([1.0, -1.0, 1.0, -1.0],
                                                  dtype=np.float32)


def _add_outliers(shape: TalkerShape, e: np.ndarray) -> np.ndarray:
    if shape.outliers:
        ch, sg = outlier_channels(shape)
        e[..., ch] += np.float32(3.0e4) * sg
    return e


def prefill_embeddings(shape: TalkerShape, T: int, seq: int = 0) -> np.ndarray:
    """``[T][hidden]`` float32 prefill rows of sequence ``seq``."""
    e = _normal((T, shape.hidden), shape.emb_seed, _TAG_PREFILL, seq)
    return _add_outliers(shape, e)


def step_embedding(shape: TalkerShape, step: int, seq: int = 0) -> np.ndarray:
    """``[hidden]`` float32 embedding fed to decode step ``step`` of ``seq``."""
    e = _normal((shape.hidden,), shape.emb_seed, _TAG_STEP, seq, step)
    return _add_outliers(shape, e)


def batch_lengths(shape: TalkerShape) -> np.ndarray:
    """Per-sequence prefill lengths, uniform integers in [512, 4096]."""
    return _rng(shape.emb_seed, _TAG_LENGTHS).integers(
        512, 4096, size=shape.n_seqs, endpoint=True).astype(np.int64)


def embedding_tables(shape: TalkerShape, n_groups: int = 16,
                     codec_rows: int = 3072, acoustic_rows: int = 2048):
    """The frame step's tables: the codec embedding ``[codec_rows][hidden]``
    then ``n_groups - 1`` acoustic tables ``[acoustic_rows][hidden]``, float32
    ``0.25 * N(0, 1)`` (a 16-row sum has unit scale, like the other inputs)."""
    out = [np.float32(0.25) * _normal((codec_rows, shape.hidden), shape.seed, _TAG_TABLE, 0)]
    for g in range(1, n_groups):
        out.append(np.float32(0.25) * _normal((acoustic_rows, shape.hidden),
                                              shape.seed, _TAG_TABLE, g))
    return out


def overlay_row(shape: TalkerShape, frame: int) -> np.ndarray:
    """``[hidden]`` float32 N(0, 1) trailing-text overlay of frame ``frame``."""
    return _normal((shape.hidden,), shape.emb_seed, _TAG_OVERLAY, frame)
