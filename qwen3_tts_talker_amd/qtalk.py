"""Python binding of the C ABI in ``include/qtalk.h`` (ctypes).

Argument marshalling only: every step of the forward runs in the HIP kernels
of ``libqtalk.so``.  Functions keep the C names; activations are passed as
float32 CUDA (HIP) torch tensors or raw device addresses.  The library is
loaded from this package's directory and the import fails loudly when it is
missing: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqtalk.so")

QTALK_OK = 0
QTALK_E_INVAL = -1
QTALK_E_OVERFLOW = -2
QTALK_E_NOMEM = -3
QTALK_E_DEVICE = -4
QTALK_F32, QTALK_BF16, QTALK_F16, QTALK_Q8 = 0, 1, 2, 3

EXPORTS = ("qtalk_create", "qtalk_destroy", "qtalk_prefill", "qtalk_extend",
           "qtalk_decode", "qtalk_decode_batch", "qtalk_kv_rewind",
           "qtalk_kv_len", "qtalk_kv_read", "qtalk_prefill_batch", "qtalk_embed_sum",
           "qtalk_argmax", "qtalk_argmax_embed",
           "qtalk_select_head", "qtalk_sync", "qtalk_last_error",
           "qtalk_set_wait_limit", "qtalk_decode_noalloc", "qtalk_decode_step")


class qtalk_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("max_seq_len", ctypes.c_int32),
                ("max_seqs", ctypes.c_int32), ("weight_dtype", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("n_output_heads", ctypes.c_int32)]


class qtalk_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj",
        "down_proj", "input_norm", "post_attn_norm", "q_norm", "k_norm")]


class qtalk_weights(ctypes.Structure):
    _fields_ = [("layers", ctypes.POINTER(qtalk_layer_weights)),
                ("final_norm", ctypes.c_void_p), ("codec_head", ctypes.c_void_p)]


QTALK_MAX_GATHER = 16


class qtalk_gather(ctypes.Structure):
    _fields_ = [("n_tables", ctypes.c_int32),
                ("tables", ctypes.c_void_p * QTALK_MAX_GATHER),
                ("table_rows", ctypes.c_int32 * QTALK_MAX_GATHER),
                ("ids", ctypes.c_void_p), ("overlay", ctypes.c_void_p)]


class QtalkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"qtalk status {status}: {msg}")
        self.status = status


_lib = None


def load_library() -> ctypes.CDLL:
    """Load ``libqtalk.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m qwen3_tts_talker_amd.build` (there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
    sig = {
        "qtalk_create": (st, [ctypes.POINTER(qtalk_config),
                              ctypes.POINTER(qtalk_weights), P,
                              ctypes.POINTER(P)]),
        "qtalk_destroy": (None, [P]),
        "qtalk_prefill": (st, [P, I32, P, I32, P, P]),
        "qtalk_extend": (st, [P, I32, P, I32, P, P]),
        "qtalk_decode": (st, [P, I32, P, P, P]),
        "qtalk_decode_batch": (st, [P, I32, ctypes.POINTER(I32), P, P, P]),
        "qtalk_kv_rewind": (st, [P, I32, I32]),
        "qtalk_kv_len": (I32, [P, I32]),
        "qtalk_kv_read": (st, [P, I32, I32, I32, P]),
        "qtalk_prefill_batch": (st, [P, I32, ctypes.POINTER(I32), P, I32, P, P]),
        "qtalk_embed_sum": (st, [P, I32, ctypes.POINTER(P), ctypes.POINTER(I32),
                                 P, I32, P, P]),
        "qtalk_argmax": (st, [P, P, I32, I32, I32, I32, P]),
        "qtalk_argmax_embed": (st, [P, P, I32, I32, I32, I32, P, I32, P, P]),
        "qtalk_select_head": (st, [P, I32]),
        "qtalk_sync": (st, [P]),
        "qtalk_last_error": (ctypes.c_char_p, [P]),
        "qtalk_set_wait_limit": (st, [P, ctypes.c_int64]),
        "qtalk_decode_noalloc": (st, [P, I32, P, P, P]),
        "qtalk_decode_step": (st, [P, I32, P, ctypes.POINTER(qtalk_gather), P, P, I32, I32, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(t) -> Optional[int]:
    """Device address of a float32 CUDA tensor (or an int address / None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    import torch
    if not t.is_cuda:
        raise ValueError("activations must be device tensors")
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError("activations must be contiguous float32")
    return t.data_ptr()


def _check(ctx, status: int) -> int:
    if status != QTALK_OK:
        msg = load_library().qtalk_last_error(ctx) if ctx else b""
        raise QtalkError(status, (msg or b"").decode())
    return status


# -- the C entry points, same names ------------------------------------------

def qtalk_create(config: qtalk_config, weights: qtalk_weights, stream=None):
    lib = load_library()
    out = ctypes.c_void_p()
    s = lib.qtalk_create(ctypes.byref(config), ctypes.byref(weights),
                         ctypes.c_void_p(stream) if stream else None,
                         ctypes.byref(out))
    if s != QTALK_OK:
        raise QtalkError(s, "qtalk_create failed")
    return out.value


def qtalk_destroy(ctx) -> None:
    load_library().qtalk_destroy(ctx)


def qtalk_prefill(ctx, seq, emb, T, logits, hidden_out=None) -> int:
    return _check(ctx, load_library().qtalk_prefill(
        ctx, seq, _ptr(emb), T, _ptr(logits), _ptr(hidden_out)))


def qtalk_extend(ctx, seq, emb, T, logits, hidden_out=None) -> int:
    return _check(ctx, load_library().qtalk_extend(
        ctx, seq, _ptr(emb), T, _ptr(logits), _ptr(hidden_out)))


def qtalk_decode(ctx, seq, emb, logits, hidden_out=None) -> int:
    return _check(ctx, load_library().qtalk_decode(
        ctx, seq, _ptr(emb), _ptr(logits), _ptr(hidden_out)))


def qtalk_decode_noalloc(ctx, seq, emb, logits, hidden_out=None) -> int:
    return _check(ctx, load_library().qtalk_decode_noalloc(
        ctx, seq, _ptr(emb), _ptr(logits), _ptr(hidden_out)))


def make_gather(tables, ids, overlay=None) -> qtalk_gather:
    """``tables``: float32 device tensors ``[rows][hidden]``; ``ids``: int32
    device tensor of ``len(tables)`` ids; ``overlay``: ``[hidden]`` or None."""
    g = qtalk_gather()
    g.n_tables = len(tables)
    for i, t in enumerate(tables):
        g.tables[i] = _ptr(t)
        g.table_rows[i] = int(t.shape[0])
    g.ids = _iptr(ids)
    g.overlay = _ptr(overlay)
    return g


def qtalk_decode_step(ctx, seq, emb, gather, logits, hidden_out=None,
                      suppress_begin=None, keep_id=-1, out_id=None) -> int:
    """``gather``: a ``qtalk_gather`` (see ``make_gather``) or None."""
    sb = suppress_begin if suppress_begin is not None else 1 << 30
    return _check(ctx, load_library().qtalk_decode_step(
        ctx, seq, _ptr(emb), ctypes.byref(gather) if gather is not None else None,
        _ptr(logits), _ptr(hidden_out), sb, keep_id,
        _iptr(out_id) if out_id is not None else None))


def qtalk_decode_batch(ctx, n, seqs: Sequence[int], emb, logits,
                       hidden_out=None) -> int:
    arr = (ctypes.c_int32 * len(seqs))(*seqs)
    return _check(ctx, load_library().qtalk_decode_batch(
        ctx, n, arr, _ptr(emb), _ptr(logits), _ptr(hidden_out)))


def qtalk_kv_rewind(ctx, seq, n_keep) -> int:
    return _check(ctx, load_library().qtalk_kv_rewind(ctx, seq, n_keep))


def qtalk_kv_len(ctx, seq) -> int:
    return load_library().qtalk_kv_len(ctx, seq)


def qtalk_kv_read(ctx, seq, layer, kv, dst) -> int:
    return _check(ctx, load_library().qtalk_kv_read(ctx, seq, layer, kv,
                                                    _ptr(dst)))


def qtalk_prefill_batch(ctx, seqs: Sequence[int], emb, T, logits,
                        hidden_out=None) -> int:
    arr = (ctypes.c_int32 * len(seqs))(*seqs)
    return _check(ctx, load_library().qtalk_prefill_batch(
        ctx, len(seqs), arr, _ptr(emb), T, _ptr(logits), _ptr(hidden_out)))


def _iptr(t) -> int:
    """Device address of an int32 CUDA tensor."""
    import torch
    if not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError("ids must be contiguous int32 device tensors")
    return t.data_ptr()


def qtalk_embed_sum(ctx, tables, ids, overlay, out) -> int:
    """``tables``: list of float32 device tensors ``[rows][hidden]``;
    ``ids``: int32 device tensor ``[n_groups][n]``."""
    G = len(tables)
    tp = (ctypes.c_void_p * G)(*[_ptr(t) for t in tables])
    rows = (ctypes.c_int32 * G)(*[int(t.shape[0]) for t in tables])
    n = int(ids.shape[1])
    return _check(ctx, load_library().qtalk_embed_sum(
        ctx, G, tp, rows, _iptr(ids), n, _ptr(overlay), _ptr(out)))


def qtalk_argmax(ctx, logits, n, vocab, suppress_begin, keep_id, out_ids) -> int:
    return _check(ctx, load_library().qtalk_argmax(
        ctx, _ptr(logits), n, vocab, suppress_begin, keep_id, _iptr(out_ids)))


def qtalk_argmax_embed(ctx, logits, n, vocab, suppress_begin, keep_id, table, table_rows,
                       out_ids, out_rows) -> int:
    return _check(ctx, load_library().qtalk_argmax_embed(
        ctx, _ptr(logits), n, vocab, suppress_begin, keep_id, _ptr(table), table_rows,
        _iptr(out_ids), _ptr(out_rows)))


def qtalk_select_head(ctx, head) -> int:
    return _check(ctx, load_library().qtalk_select_head(ctx, head))


def qtalk_sync(ctx) -> int:
    return _check(ctx, load_library().qtalk_sync(ctx))


def qtalk_last_error(ctx) -> str:
    return (load_library().qtalk_last_error(ctx) or b"").decode()


def qtalk_set_wait_limit(ctx, polls) -> int:
    return _check(ctx, load_library().qtalk_set_wait_limit(ctx, polls))


# -- convenience wrapper --------------------------------------------------------

def _host_weight(a: np.ndarray, bf16: bool) -> np.ndarray:
    """Host copy in the library's storage format (bf16 bit patterns or f32)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not bf16:
        return a
    u = a.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("weights are not bf16-representable")
    return (u >> 16).astype(np.uint16)


class Talker:
    """Owns one ``qtalk_ctx`` built from float32 weight arrays.

    ``weights`` = ``{"layers": [dict(wq, wk, wv, wo, wg, wu, wd, g_in, g_post,
    g_q, g_k)], "g_final", "w_head"}``; projections ``[out][in]``.  ``w_head``
    is ``[vocab][hidden]``, or ``[n][vocab][hidden]`` for n stacked output
    heads (the code predictor), chosen with ``select_head``.
    """

    def __init__(self, shape, weights: Dict, stream=None):
        import torch
        self.shape = shape
        bf16 = shape.weight_dtype == "bf16"
        cfg = qtalk_config(
            n_layers=len(weights["layers"]), hidden=shape.hidden,
            n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads,
            head_dim=shape.head_dim, intermediate=shape.intermediate,
            vocab=shape.vocab, rms_eps=shape.rms_eps,
            rope_theta=shape.rope_theta, max_seq_len=shape.cap,
            max_seqs=shape.n_seqs,
            weight_dtype=QTALK_BF16 if bf16 else QTALK_F32,
            kv_dtype={"f16": QTALK_F16, "q8": QTALK_Q8}.get(shape.kv_dtype, QTALK_F32),
            n_output_heads=(weights["w_head"].shape[0]
                            if np.ndim(weights["w_head"]) == 3 else 1))
        keep = []

        def hp(a, as_weight):
            h = _host_weight(a, bf16) if as_weight else np.ascontiguousarray(
                a, dtype=np.float32)
            keep.append(h)
            return h.ctypes.data

        L = len(weights["layers"])
        layers = (qtalk_layer_weights * L)()
        for i, lw in enumerate(weights["layers"]):
            layers[i] = qtalk_layer_weights(
                hp(lw["wq"], 1), hp(lw["wk"], 1), hp(lw["wv"], 1),
                hp(lw["wo"], 1), hp(lw["wg"], 1), hp(lw["wu"], 1),
                hp(lw["wd"], 1), hp(lw["g_in"], 0), hp(lw["g_post"], 0),
                hp(lw["g_q"], 0), hp(lw["g_k"], 0))
        w = qtalk_weights(layers, hp(weights["g_final"], 0),
                          hp(weights["w_head"], 1))
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        self.stream = stream
        self.ctx = qtalk_create(cfg, w, stream)
        del keep
        self.n_layers = L

    def close(self):
        if getattr(self, "ctx", None):
            qtalk_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _out(self, *shape):
        import torch
        return torch.empty(*shape, dtype=torch.float32, device="cuda")

    def prefill(self, seq, emb, hidden=False):
        lg = self._out(self.shape.vocab)
        hd = self._out(self.shape.hidden) if hidden else None
        qtalk_prefill(self.ctx, seq, emb, emb.shape[0], lg, hd)
        return (lg, hd) if hidden else lg

    def extend(self, seq, emb, hidden=False):
        lg = self._out(self.shape.vocab)
        hd = self._out(self.shape.hidden) if hidden else None
        qtalk_extend(self.ctx, seq, emb, emb.shape[0], lg, hd)
        return (lg, hd) if hidden else lg

    def decode(self, seq, emb, hidden=False):
        lg = self._out(self.shape.vocab)
        hd = self._out(self.shape.hidden) if hidden else None
        qtalk_decode(self.ctx, seq, emb, lg, hd)
        return (lg, hd) if hidden else lg

    def prefill_batch(self, seqs, emb, hidden=False):
        """``emb`` ``[n][T][hidden]``: prefill each listed sequence."""
        n, T = len(seqs), int(emb.shape[1])
        lg = self._out(n, self.shape.vocab)
        hd = self._out(n, self.shape.hidden) if hidden else None
        qtalk_prefill_batch(self.ctx, list(seqs), emb, T, lg, hd)
        return (lg, hd) if hidden else lg

    def decode_batch(self, seqs, emb, hidden=False):
        n = len(seqs)
        lg = self._out(n, self.shape.vocab)
        hd = self._out(n, self.shape.hidden) if hidden else None
        qtalk_decode_batch(self.ctx, n, list(seqs), emb, lg, hd)
        return (lg, hd) if hidden else lg

    def kv_len(self, seq):
        return qtalk_kv_len(self.ctx, seq)

    def kv_rewind(self, seq, n_keep):
        qtalk_kv_rewind(self.ctx, seq, n_keep)

    def kv_read(self, seq, layer, which):
        n = self.kv_len(seq)
        dst = self._out(self.shape.n_kv_heads, max(n, 1), self.shape.head_dim)
        qtalk_kv_read(self.ctx, seq, layer, which, dst)
        return dst[:, :n]

    def select_head(self, head):
        qtalk_select_head(self.ctx, head)

    def embed_sum(self, tables, ids, overlay=None, out=None):
        """Step embeddings ``[n][hidden]`` of the int32 ids ``[G][n]``."""
        if out is None:
            out = self._out(int(ids.shape[1]), self.shape.hidden)
        qtalk_embed_sum(self.ctx, tables, ids, overlay, out)
        return out

    def argmax(self, logits, suppress_begin=None, keep_id=-1, out=None):
        """Greedy ids (int32 device tensor ``[n]``) of logits ``[n][vocab]``."""
        import torch
        lg = logits if logits.dim() == 2 else logits.view(1, -1)
        n, vocab = int(lg.shape[0]), int(lg.shape[1])
        if out is None:
            out = torch.empty(n, dtype=torch.int32, device="cuda")
        qtalk_argmax(self.ctx, lg, n, vocab,
                     vocab if suppress_begin is None else suppress_begin, keep_id, out)
        return out

    def argmax_embed(self, logits, table, suppress_begin=None, keep_id=-1, out=None,
                     out_rows=None):
        """Greedy ids of logits ``[n][vocab]`` (as ``argmax``) and the
        ``table`` rows of those ids; returns ``(ids [n] int32, rows [n][hidden])``."""
        import torch
        lg = logits if logits.dim() == 2 else logits.view(1, -1)
        n, vocab = int(lg.shape[0]), int(lg.shape[1])
        if out is None:
            out = torch.empty(n, dtype=torch.int32, device="cuda")
        if out_rows is None:
            out_rows = torch.empty(n, self.shape.hidden, device="cuda")
        qtalk_argmax_embed(self.ctx, lg, n, vocab,
                           vocab if suppress_begin is None else suppress_begin, keep_id,
                           table, int(table.shape[0]), out, out_rows)
        return out, out_rows

    def sync(self):
        qtalk_sync(self.ctx)

    def set_wait_limit(self, polls):
        qtalk_set_wait_limit(self.ctx, polls)
