"""Benchmark of the KV-cached Talker forward on one MI355X.

Headline: batch-1 decode of the 28-layer Talker (bf16 weights, f16 KV cache)
at context 1921..2048, after a 1920-row prefill on the same weights.  A step
is one decode token through the whole stack (every layer plus the final norm
and codec head).  Prefill tok/s of the 1920-row prefill is reported beside it.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]

Inputs are synthetic (seeded N(0, 1) embeddings, N(0, 0.02) bf16 weights) and
resident in device memory before the timed region starts.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Talker decode tok/s (bs1, KV 2k) + prefill tok/s; % HBM BW / % MFMA peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def kv_row_bytes(s) -> int:
    """Bytes of one cached K or V row of one head: float16 / float32 values,
    or Q8_0 (head_dim codes, then a float16 scale per 32 values)."""
    if s.kv_dtype == "q8":
        return s.head_dim + s.head_dim // 16
    return s.head_dim * (2 if s.kv_dtype == "f16" else 4)


def kv_bytes_per_position(s) -> int:
    return s.n_layers * 2 * s.n_kv_heads * kv_row_bytes(s)


def weight_bytes(s) -> int:
    per = s.params_per_layer() * s.n_layers + s.vocab * s.hidden
    return per * (2 if s.weight_dtype == "bf16" else 4)


def decode_bytes(s, keys: int) -> int:
    """Algorithmic HBM bytes of one decode token attending `keys` positions:
    every weight once, K and V of every attended position once, plus the
    new position's K and V written."""
    kvp = kv_bytes_per_position(s)
    return weight_bytes(s) + kvp * keys + kvp


def prefill_flops(s, T: int, p0: int = 0) -> float:
    """Matrix flops of a T-row prefill at offset p0: projections on every row,
    causal attention (QK^T and PV) over each row's context, head on the last
    row."""
    proj = 2.0 * (s.params_per_layer()) * T * s.n_layers
    ctx = sum(p0 + t + 1 for t in range(T))
    attn = 4.0 * s.q_dim * ctx * s.n_layers
    return proj + attn + 2.0 * s.vocab * s.hidden


DECODE_SOURCES = ("qwen3_tts_talker_amd/csrc/k_decode_fused.hip",
                  "qwen3_tts_talker_amd/csrc/common.h")
DECODE_ARGS_HEADER = "qwen3_tts_talker_amd/csrc/kernels.h"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_decode_fused_talker28_kv2k_pmc.md")


def decode_source_digest() -> str:
    """sha256 over the persistent decode kernel's sources (the counters in
    profiles/ apply only to the kernel they were taken on)."""
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    with open(os.path.join(ROOT, DECODE_ARGS_HEADER)) as f:
        hdr = f.read()
    m = re.search(r"struct FusedDecodeArgs \{.*?\};", hdr, re.S)
    h.update((m.group(0) if m else hdr).encode())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a device copy of known size),
    or None when it is missing or was taken on other kernel sources."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.]+)", text)
    d = re.search(r"decode_source_sha256:\s*([0-9a-f]{64})", text)
    if not m or not d or d.group(1) != decode_source_digest():
        return None
    return float(m.group(1))


def cpu_baseline(shape, weights, emb, steps_emb, n_steps: int):
    """The oracle (float64 NumPy) on this host: a bounded sample of the same
    workload — the 1920-row prefill, then `n_steps` decode steps."""
    from oracle import TalkerOracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 0) for i in threadpool_info()] or [0])
    except Exception:  # pragma: no cover
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    orc = TalkerOracle(shape, weights)
    t0 = time.perf_counter()
    orc.prefill(0, emb)
    t1 = time.perf_counter()
    for k in range(n_steps):
        orc.decode(0, steps_emb[k])
    t2 = time.perf_counter()
    return {
        "value": n_steps / (t2 - t1), "unit": "tok/s",
        "cores": blas_threads or cores,
        "kind": "oracle",
        "sample": (f"float64 NumPy oracle on {cores} host cores (BLAS threads "
                   f"{blas_threads}): {n_steps} decode steps at context "
                   f"{emb.shape[0] + 1}..{emb.shape[0] + n_steps} after its own "
                   f"{emb.shape[0]}-row prefill; value = decode tok/s"),
        "prefill_tok_s": emb.shape[0] / (t1 - t0),
    }


def batched_decode(n_steps: int, warmup: int = 4, kv_dtype: str = "f16") -> dict:
    """Batched decode of 16 independent utterances on the 28-layer Talker
    (its own seeded weights): KV lengths drawn uniformly from 512..4096, each
    sequence filled by a prefill and 2048-row extends, then one token per
    sequence and step (qtalk_decode_batch).  Algorithmic bytes per step:
    every weight once plus K and V of every attended position (in the cache
    type: float16, or Q8_0 rows)."""
    import torch
    from qwen3_tts_talker_amd import Talker
    from synth import batch_lengths, make_weights, prefill_embeddings, step_embedding, workload
    shape = workload("talker_28l_batch16_ragged").with_(kv_dtype=kv_dtype)
    tk = Talker(shape, make_weights(shape))
    lens = [int(x) for x in batch_lengths(shape)]
    for s, L in enumerate(lens):
        e = torch.from_numpy(prefill_embeddings(shape, L, seq=s)).cuda()
        tk.prefill(s, e[:shape.chunk])
        for c0 in range(shape.chunk, L, shape.chunk):
            tk.extend(s, e[c0:c0 + shape.chunk])
    seqs = list(range(shape.n_seqs))
    embs = [torch.from_numpy(np.stack([step_embedding(shape, k, seq=s) for s in seqs])).cuda()
            for k in range(warmup + n_steps)]
    for k in range(warmup):
        tk.decode_batch(seqs, embs[k])
    tk.sync()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for k in range(n_steps):
        tk.decode_batch(seqs, embs[warmup + k])
    e1.record(st)
    torch.cuda.synchronize()
    tk.sync()
    us = e0.elapsed_time(e1) * 1e3 / n_steps
    ctx = [L + warmup for L in lens]  # context of the first timed step
    kv_pos = sum(c + 1 for c in ctx) + len(seqs) * (n_steps - 1) / 2
    nbytes = weight_bytes(shape) + kv_bytes_per_position(shape) * kv_pos
    tk.close()
    return {"workload": "talker_28l_batch16_ragged", "kv_cache": kv_dtype, "seqs": len(seqs),
            "kv_len_range": [min(lens), max(lens)],
            "steps": n_steps, "step_us": round(us, 1), "tok_s": round(len(seqs) * 1e6 / us, 1),
            "bytes_per_step": int(nbytes), "achieved_gbs": round(nbytes / us / 1e3, 1),
            "hbm_frac": round(nbytes / us / 1e3 / 8000.0, 4)}


def q8_decode(n_steps: int, warmup: int = 8) -> dict:
    """The headline workload (28 layers, 1920-row prefill, batch-1 decode)
    with the 8-bit cache: decode tok/s and the HBM fraction of its
    algorithmic bytes (every weight once, Q8_0 K/V rows of every attended
    position, the new position written)."""
    import torch
    from qwen3_tts_talker_amd import Talker
    from synth import make_weights, prefill_embeddings, step_embedding, workload
    shape = workload("talker_28l_kv2k").with_(kv_dtype="q8")
    T = shape.prefill_len
    tk = Talker(shape, make_weights(shape))
    emb = torch.from_numpy(prefill_embeddings(shape, T)).cuda()
    steps = [torch.from_numpy(step_embedding(shape, k)).cuda() for k in range(n_steps)]
    tk.prefill(0, emb)
    for k in range(warmup):
        tk.decode(0, steps[k % n_steps])
    tk.sync()
    tk.kv_rewind(0, T)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for k in range(n_steps):
        tk.decode(0, steps[k])
    e1.record(st)
    torch.cuda.synchronize()
    tk.sync()
    assert tk.kv_len(0) == T + n_steps
    us = e0.elapsed_time(e1) * 1e3 / n_steps
    nbytes = sum(decode_bytes(shape, T + k + 1) for k in range(n_steps)) / n_steps
    tk.close()
    return {"workload": "talker_28l_kv2k", "kv_cache": "q8", "steps": n_steps,
            "decode_ctx": [T + 1, T + n_steps], "step_us": round(us, 1),
            "tok_s": round(1e6 / us, 1), "bytes_per_step": int(nbytes),
            "achieved_gbs": round(nbytes / us / 1e3, 1), "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}


def long_context(n_steps: int, warmup: int = 4) -> dict:
    """The long-context workload: the 28-layer Talker (its own seeded
    weights), rows carrying +-3e4 on four fixed channels, prefilled in 16
    chunks of 2048 rows (one qtalk_prefill, then qtalk_extend) to 32,768
    positions, then batch-1 decode steps at context 32,769 onwards.  Events
    on the library's stream time every chunk and every step.  Matrix flops
    per chunk: projections on every row, causal attention over each row's
    context, the head on the last row; bytes per step as the headline's."""
    import torch
    from qwen3_tts_talker_amd import Talker
    from synth import make_weights, prefill_embeddings, step_embedding, workload
    shape = workload("talker_28l_ctx32k_outlier")
    tk = Talker(shape, make_weights(shape))
    n, ch = shape.prefill_len, shape.chunk
    emb = torch.from_numpy(prefill_embeddings(shape, n)).cuda()
    n_steps = min(n_steps, shape.cap - n)
    steps = torch.from_numpy(np.stack([step_embedding(shape, k) for k in range(max(n_steps, warmup))])).cuda()
    st = torch.cuda.current_stream()
    tk.prefill(0, emb[:ch])  # warm-up of the prefill kernels
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n // ch + 1)]
    ev[0].record(st)
    for ci, c0 in enumerate(range(0, n, ch)):
        (tk.prefill if ci == 0 else tk.extend)(0, emb[c0:c0 + ch])
        ev[ci + 1].record(st)
    torch.cuda.synchronize()
    tk.sync()
    chunk_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(n // ch)]
    flops = [prefill_flops(shape, ch, c0) for c0 in range(0, n, ch)]
    for k in range(warmup):
        tk.decode(0, steps[k])
    torch.cuda.synchronize()
    tk.sync()
    tk.kv_rewind(0, n)
    dev_ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps + 1)]
    dev_ev[0].record(st)
    for k in range(n_steps):
        tk.decode(0, steps[k])
        dev_ev[k + 1].record(st)
    torch.cuda.synchronize()
    tk.sync()
    step_ms = np.array([dev_ev[k].elapsed_time(dev_ev[k + 1]) for k in range(n_steps)])
    dec_ms = dev_ev[0].elapsed_time(dev_ev[n_steps])
    nbytes = sum(decode_bytes(shape, n + k + 1) for k in range(n_steps))
    tk.close()
    tot = sum(chunk_ms)
    return {"workload": shape.name, "chunks": n // ch, "chunk_rows": ch,
            "prefill_ms": round(tot, 3), "prefill_tok_s": round(n / (tot / 1e3), 1),
            "prefill_tflops": round(sum(flops) / (tot / 1e3) / 1e12, 2),
            "prefill_mfma_frac": round(sum(flops) / (tot / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "last_chunk": {"p0": n - ch, "ms": round(chunk_ms[-1], 3),
                           "tflops": round(flops[-1] / (chunk_ms[-1] / 1e3) / 1e12, 2),
                           "mfma_frac": round(flops[-1] / (chunk_ms[-1] / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
            "decode_steps": n_steps, "decode_ctx": [n + 1, n + n_steps],
            "decode_us": round(dec_ms * 1e3 / n_steps, 1),
            "decode_p99_us": round(float(np.percentile(step_ms, 99)) * 1e3, 1),
            "decode_tok_s": round(n_steps / (dec_ms / 1e3), 1),
            "decode_achieved_gbs": round(nbytes / (dec_ms / 1e3) / 1e9, 1),
            "decode_hbm_frac": round(nbytes / (dec_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}


def batched_prefill(shape, weights, n: int, T: int, reps: int = 5) -> dict:
    """Batched prefill of n utterances of T rows each (one call) against n
    consecutive single prefills, on a context with n sequences."""
    import torch
    from qwen3_tts_talker_amd import Talker, qtalk
    from synth import prefill_embeddings

    s = shape.with_(n_seqs=n, cap=T)
    tk = Talker(s, weights)
    ctx, lib = tk.ctx, qtalk.load_library()
    emb = torch.from_numpy(np.stack([prefill_embeddings(s, T, seq=b) for b in range(n)])).cuda()
    lg = torch.empty(n, s.vocab, device="cuda")
    seqs = (ctypes.c_int32 * n)(*range(n))
    st = torch.cuda.current_stream()

    def batched():
        return lib.qtalk_prefill_batch(ctx, n, seqs, emb.data_ptr(), T, lg.data_ptr(), None)

    def serial():
        r = 0
        for b in range(n):
            r |= lib.qtalk_prefill(ctx, b, emb[b].data_ptr(), T, lg[b].data_ptr(), None)
        return r

    res = {}
    for name, fn in (("batched", batched), ("serial", serial)):
        assert fn() == 0, qtalk.qtalk_last_error(ctx)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            assert fn() == 0, qtalk.qtalk_last_error(ctx)
            e1.record(st)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        res[name] = sorted(ts)[len(ts) // 2]
    assert lib.qtalk_sync(ctx) == 0, qtalk.qtalk_last_error(ctx)
    tk.close()
    fl = n * prefill_flops(s, T)
    return {"seqs": n, "T": T, "batched_ms": round(res["batched"], 3),
            "tok_s": round(n * T / (res["batched"] / 1e3), 1),
            "tflops": round(fl / (res["batched"] / 1e3) / 1e12, 2),
            "mfma_frac": round(fl / (res["batched"] / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "serial_ms": round(res["serial"], 3)}


def device_frames(talker, cp, n_frames: int, warmup: int, fused: bool = False) -> dict:
    """Whole codec frames on the device, with no host round trip: the
    Talker's step embedding gathered from the previous frame's 16 ids plus
    an overlay row, one Talker decode, the suppressed codebook-0 pick, the
    code predictor's two-row prefill (the Talker's hidden state, the codec
    row of that id) and 14 steps, each step's input gathered from the table
    of the previous code and each code picked on the device.  fused: every
    step is one qtalk_decode_step (gather and pick inside the persistent
    decode, no other kernel); else separate gather / pick kernels."""
    import torch
    from qwen3_tts_talker_amd import qtalk
    from synth import embedding_tables, overlay_row

    ts = talker.shape
    V, H, EOS = ts.vocab, ts.hidden, 2150
    tabs = [torch.from_numpy(t).cuda() for t in embedding_tables(ts)]
    ov = torch.from_numpy(overlay_row(ts, 0)).cuda().view(1, H)
    ids = torch.zeros((2, 16), dtype=torch.int32, device="cuda")
    emb = torch.empty(1, H, device="cuda")
    lg_t = torch.empty(V, device="cuda")
    cp_in = torch.empty(2, H, device="cuda")
    lg_c = torch.empty(15, cp.shape.vocab, device="cuda")
    steps = torch.empty(15, 1, H, device="cuda")
    st = torch.cuda.current_stream()

    gathers = []  # per parity: the Talker's 16-table gather, then each code predictor step's
    for i in range(2):
        a, b = ids[i % 2], ids[(i + 1) % 2]
        gathers.append([qtalk.make_gather(tabs, a, ov.view(-1)), qtalk.make_gather(tabs[0:1], b[0:1])] +
                       [qtalk.make_gather(tabs[j:j + 1], b[j:j + 1]) for j in range(1, 15)])

    def frame_fused(i):
        a, b = ids[i % 2], ids[(i + 1) % 2]
        g = gathers[i % 2]
        qtalk.qtalk_decode_step(talker.ctx, 0, None, g[0], lg_t, cp_in[0], V - 1024, EOS, b[0:1])
        cp.kv_rewind(0, 0)
        cp.select_head(0)
        qtalk.qtalk_decode_step(cp.ctx, 0, cp_in[0], None, lg_c[0])
        qtalk.qtalk_decode_step(cp.ctx, 0, None, g[1], lg_c[0], None, out_id=b[1:2])
        for j in range(1, 15):
            cp.select_head(j)
            qtalk.qtalk_decode_step(cp.ctx, 0, None, g[j + 1], lg_c[j], None, out_id=b[j + 1:j + 2])

    def frame(i):
        if fused:
            return frame_fused(i)
        # each pick also fetches the table row the next call feeds on
        # (qtalk_argmax_embed), so no separate lookup kernel runs
        a, b = ids[i % 2], ids[(i + 1) % 2]
        talker.embed_sum(tabs, a.view(16, 1), ov, out=emb)
        qtalk.qtalk_decode(talker.ctx, 0, emb, lg_t, cp_in[0])
        talker.argmax_embed(lg_t, tabs[0], suppress_begin=V - 1024, keep_id=EOS, out=b[0:1],
                            out_rows=cp_in[1:2])
        cp.select_head(0)
        qtalk.qtalk_prefill(cp.ctx, 0, cp_in, 2, lg_c[0])
        cp.argmax_embed(lg_c[0], tabs[1], out=b[1:2], out_rows=steps[1])
        for j in range(1, 15):
            cp.select_head(j)
            qtalk.qtalk_decode(cp.ctx, 0, steps[j], lg_c[j])
            if j < 14:
                cp.argmax_embed(lg_c[j], tabs[j + 1], out=b[j + 1:j + 2], out_rows=steps[j + 1])
            else:
                cp.argmax(lg_c[j], out=b[j + 1:j + 2])

    for i in range(warmup):
        frame(i)
    torch.cuda.synchronize()
    talker.sync()
    cp.sync()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(n_frames):
        frame(warmup + i)
    e1.record(st)
    torch.cuda.synchronize()
    talker.sync()
    cp.sync()
    ms = e0.elapsed_time(e1) / n_frames
    return {"frames": n_frames, "talker_ctx": [talker.kv_len(0) - n_frames + 1, talker.kv_len(0)],
            "frame_us": round(ms * 1e3, 1), "frames_per_s": round(1e3 / ms, 1),
            "glue_launches": 0 if fused else 18}


def code_predictor(n_frames: int, warmup: int, talker=None) -> dict:
    """Frames of the 5-layer code predictor (15 heads of 2048 codes): per
    frame a two-row prefill through head 0, then 14 one-token decode steps,
    step j through head j.  Inputs are synthetic rows standing in for the
    Talker's hidden state, the codebook-0 embedding and the per-step table
    rows.  Events on the library's stream time the frame and its 14 steps."""
    import torch
    from qwen3_tts_talker_amd import Talker, qtalk
    from synth import make_weights, prefill_embeddings, step_embedding, workload

    shape = workload("code_predictor_5l")
    tk = Talker(shape, make_weights(shape))
    lib = qtalk.load_library()
    ctx = tk.ctx
    first = torch.from_numpy(prefill_embeddings(shape, 2)).cuda()
    steps = torch.from_numpy(np.stack([step_embedding(shape, j) for j in range(14)])).cuda()
    lg = torch.empty(15, shape.vocab, device="cuda")
    st = torch.cuda.current_stream()

    def frame():
        s = lib.qtalk_select_head(ctx, 0) | lib.qtalk_prefill(ctx, 0, first.data_ptr(), 2,
                                                               lg[0].data_ptr(), None)
        for j in range(1, 15):
            s |= lib.qtalk_select_head(ctx, j)
            s |= lib.qtalk_decode(ctx, 0, steps[j - 1].data_ptr(), lg[j].data_ptr(), None)
        return s

    for _ in range(warmup):
        assert frame() == 0, qtalk.qtalk_last_error(ctx)
    torch.cuda.synchronize()
    assert lib.qtalk_sync(ctx) == 0, qtalk.qtalk_last_error(ctx)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_frames)]
    status = 0
    for f in range(n_frames):
        ev[f][0].record(st)
        status |= lib.qtalk_select_head(ctx, 0) | lib.qtalk_prefill(
            ctx, 0, first.data_ptr(), 2, lg[0].data_ptr(), None)
        ev[f][1].record(st)
        for j in range(1, 15):
            status |= lib.qtalk_select_head(ctx, j)
            status |= lib.qtalk_decode(ctx, 0, steps[j - 1].data_ptr(), lg[j].data_ptr(), None)
        ev[f][2].record(st)
    torch.cuda.synchronize()
    assert status == 0 and lib.qtalk_sync(ctx) == 0, qtalk.qtalk_last_error(ctx)
    dev_frames = device_frames(talker, tk, n_frames, warmup) if talker is not None else None
    dev_fused = device_frames(talker, tk, n_frames, warmup, fused=True) if talker is not None else None
    frame_ms = float(np.mean([e[0].elapsed_time(e[2]) for e in ev]))
    pre_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    step_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) / 14
    step_bytes = float(np.mean([decode_bytes(shape, 2 + j) for j in range(1, 15)]))
    achieved = step_bytes / (step_ms / 1e3) / 1e9
    tk.close()
    res = {"workload": shape.name, "layers": shape.n_layers, "vocab": shape.vocab,
            "heads": 15, "frames": n_frames, "frame_us": round(frame_ms * 1e3, 1),
            "frames_per_s": round(1e3 / frame_ms, 1),
            "prefill_2rows_us": round(pre_ms * 1e3, 1), "step_us": round(step_ms * 1e3, 2),
            "step_bytes": int(step_bytes), "step_achieved_gbs": round(achieved, 1),
            "step_hbm_frac": round(achieved / HBM_PEAK_GBS, 4)}
    if dev_frames is not None:
        res["device_frame"] = dev_frames
        res["device_frame_fused"] = dev_fused
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--prefill-reps", type=int, default=5)
    ap.add_argument("--workload", default="talker_28l_kv2k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-steps", type=int, default=8)
    ap.add_argument("--batch-prefill", type=int, default=16,
                    help="utterances of 128 rows in the batched-prefill leg (0: skip)")
    ap.add_argument("--batch-decode", type=int, default=32,
                    help="timed steps of the 16-utterance batched decode leg (0: skip)")
    ap.add_argument("--long-context", type=int, default=256,
                    help="decode steps of the 32k long-context leg after its 16 x 2048-row "
                         "prefill (0: skip the leg)")
    ap.add_argument("--q8", type=int, default=64,
                    help="decode steps of the 8-bit-cache legs (batch-1 headline workload and the "
                         "16-utterance batch; 0: skip)")
    ap.add_argument("--cp-frames", type=int, default=20,
                    help="code predictor frames timed after the Talker (0: skip)")
    ap.add_argument("--pmc-calibration-mib", type=int, default=0,
                    help="before the timed region, copy this many MiB device to "
                         "device (a known-size reference for HBM byte counters)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(it would shard independent utterances, one process per GPU)",
              file=sys.stderr)
        return 2

    import torch
    from qwen3_tts_talker_amd import Talker, qtalk
    from synth import make_weights, prefill_embeddings, step_embedding, workload

    shape = workload(args.workload)
    T = shape.prefill_len
    K = args.steps
    if T + K > shape.cap:
        K = shape.cap - T
    torch.cuda.set_device(0)
    weights = make_weights(shape)
    emb_h = prefill_embeddings(shape, T)
    steps_h = np.stack([step_embedding(shape, k) for k in range(max(K, args.cpu_steps))])
    tk = Talker(shape, weights)
    lib = qtalk.load_library()
    ctx = tk.ctx
    emb = torch.from_numpy(emb_h).cuda()
    steps = torch.from_numpy(steps_h).cuda()
    logits = torch.empty(shape.vocab, device="cuda")
    st = torch.cuda.current_stream()

    # prefill: warm once, then time reps (events on the library's stream)
    def prefill_once():
        s = lib.qtalk_prefill(ctx, 0, emb.data_ptr(), T, logits.data_ptr(), None)
        assert s == 0, qtalk.qtalk_last_error(ctx)

    prefill_once()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.prefill_reps)]
    for r in range(args.prefill_reps):
        ev[2 * r].record(st)
        prefill_once()
        ev[2 * r + 1].record(st)
    torch.cuda.synchronize()
    pre_ms = sorted(ev[2 * r].elapsed_time(ev[2 * r + 1]) for r in range(args.prefill_reps))
    pre_med = pre_ms[len(pre_ms) // 2]

    if args.pmc_calibration_mib > 0:
        n = args.pmc_calibration_mib << 18  # float32 elements
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # decode warmup from context T, then rewind and time K steps
    for k in range(args.warmup):
        s = lib.qtalk_decode(ctx, 0, steps[k % K].data_ptr(), logits.data_ptr(), None)
        assert s == 0, qtalk.qtalk_last_error(ctx)
    torch.cuda.synchronize()
    # the persistent decode reports a failed step (a wait that gave up, an
    # unexpected block placement) through the library's status word
    assert lib.qtalk_sync(ctx) == 0, qtalk.qtalk_last_error(ctx)
    lib.qtalk_kv_rewind(ctx, 0, T)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(st)
    status = 0
    for k in range(K):
        status |= lib.qtalk_decode(ctx, 0, steps[k].data_ptr(), logits.data_ptr(), None)
        evs[k + 1].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert status == 0 and lib.qtalk_sync(ctx) == 0, qtalk.qtalk_last_error(ctx)
    assert tk.kv_len(0) == T + K
    step_ms = np.array([evs[k].elapsed_time(evs[k + 1]) for k in range(K)])
    total_ms = evs[0].elapsed_time(evs[K])
    tok_s = K / (total_ms / 1e3)

    alg_bytes = sum(decode_bytes(shape, T + k + 1) for k in range(K))
    achieved = alg_bytes / (total_ms / 1e3) / 1e9
    traffic = measured_traffic()
    roof = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": None if traffic is None else int(traffic),
        "kernel": ("k_decode_fused (one persistent launch per token)"
                   if os.environ.get("QTALK_FUSED_DECODE", "1") != "0"
                   else "decode step (all launches of one token)"),
        "bytes_per_step": int(alg_bytes / K),
    }
    pf = prefill_flops(shape, T)
    out = {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tok/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(total_ms / K, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": shape.name, "layers": shape.n_layers,
                   "hidden": shape.hidden, "heads": f"{shape.n_heads}q/{shape.n_kv_heads}kv",
                   "head_dim": shape.head_dim, "intermediate": shape.intermediate,
                   "vocab": shape.vocab, "batch": 1, "prefill_len": T,
                   "decode_ctx": [T + 1, T + K], "weights": shape.weight_dtype,
                   "kv_cache": shape.kv_dtype},
        "p50_step_us": round(float(np.percentile(step_ms, 50)) * 1e3, 1),
        "p99_step_us": round(float(np.percentile(step_ms, 99)) * 1e3, 1),
        "wall_s": round(wall, 3),
        "prefill_tok_s": round(T / (pre_med / 1e3), 1),
        "prefill_ms": round(pre_med, 3),
        "prefill_tflops": round(pf / (pre_med / 1e3) / 1e12, 2),
        "prefill_mfma_frac": round(pf / (pre_med / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": roof,
    }
    if args.cp_frames > 0:
        # whole frames continue the Talker from context T
        lib.qtalk_kv_rewind(ctx, 0, T)
        out["code_predictor"] = code_predictor(args.cp_frames, warmup=3, talker=tk)
    tk.close()
    if args.batch_prefill > 0:
        out["prefill_batch"] = batched_prefill(shape, weights, args.batch_prefill, 128)
    if args.batch_decode > 0:
        out["decode_batch"] = batched_decode(args.batch_decode)
    if args.long_context > 0:
        out["long_context"] = long_context(args.long_context)
    if args.q8 > 0:
        out["kv_q8"] = {"decode": q8_decode(args.q8),
                        "decode_batch": batched_decode(max(8, args.q8 // 4), kv_dtype="q8")}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shape, weights, emb_h, steps_h, args.cpu_steps)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
