"""Pins of the oracle's whole forward: an independent library model, closed
forms, path invariants, error behaviour and planted mistakes (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle.talker as ot
from oracle import TalkerOracle
from synth import TalkerShape, make_weights, prefill_embeddings, step_embedding, workload


def small_shape(**kw):
    """A Talker-like geometry with q_dim != hidden (as in the Talker)."""
    base = dict(name="pin", n_layers=2, hidden=64, n_heads=4, n_kv_heads=2,
                head_dim=32, intermediate=96, vocab=40, rms_eps=1e-6,
                rope_theta=1e6, weight_dtype="f32", kv_dtype="f32", cap=48,
                n_seqs=3, seed=77, emb_seed=78)
    base.update(kw)
    return TalkerShape(**base)


def scaled_weights(shape, wscale=0.15):
    """Weights with larger spread than 0.02 so every term matters in the pins."""
    w = make_weights(shape)
    f = np.float32(wscale / 0.02)
    for lw in w["layers"]:
        for k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
            lw[k] = lw[k] * f
    w["w_head"] = w["w_head"] * f
    return w


# -- independent library model ---------------------------------------------------

def _transformers_model(shape, w):
    from transformers import Qwen3Config
    from transformers.models.qwen3.modeling_qwen3 import Qwen3Model
    cfg = Qwen3Config(
        vocab_size=8, hidden_size=shape.hidden,
        intermediate_size=shape.intermediate,
        num_hidden_layers=shape.n_layers, num_attention_heads=shape.n_heads,
        num_key_value_heads=shape.n_kv_heads, head_dim=shape.head_dim,
        rms_norm_eps=shape.rms_eps, attention_bias=False,
        rope_parameters={"rope_type": "default",
                         "rope_theta": shape.rope_theta})
    cfg._attn_implementation = "eager"
    m = Qwen3Model(cfg).double().eval()
    names = {"wq": "self_attn.q_proj.weight", "wk": "self_attn.k_proj.weight",
             "wv": "self_attn.v_proj.weight", "wo": "self_attn.o_proj.weight",
             "wg": "mlp.gate_proj.weight", "wu": "mlp.up_proj.weight",
             "wd": "mlp.down_proj.weight",
             "g_in": "input_layernorm.weight",
             "g_post": "post_attention_layernorm.weight",
             "g_q": "self_attn.q_norm.weight", "g_k": "self_attn.k_norm.weight"}
    sd = {}
    for l, lw in enumerate(w["layers"]):
        for k, n in names.items():
            sd[f"layers.{l}.{n}"] = torch.from_numpy(lw[k].astype(np.float64))
    sd["norm.weight"] = torch.from_numpy(w["g_final"].astype(np.float64))
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert set(missing) == {"embed_tokens.weight"} and not unexpected
    return m


def _transformers_logits(shape, w, emb):
    m = _transformers_model(shape, w)
    with torch.no_grad():
        hs = m(inputs_embeds=torch.from_numpy(emb.astype(np.float64))[None],
               use_cache=False).last_hidden_state[0].numpy()
    return hs @ w["w_head"].astype(np.float64).T


def test_oracle_matches_transformers_qwen3_all_rows():
    # transformers' Qwen3 decoder (pre-norm, QK-norm, rotate-half RoPE, GQA,
    # SwiGLU) is an independent implementation of the same block; it keeps
    # RMSNorm and RoPE tables in float32 internally, hence the tolerance.
    shape = small_shape()
    w = scaled_weights(shape)
    emb = prefill_embeddings(shape, 20)
    ref = _transformers_logits(shape, w, emb)
    orc = TalkerOracle(shape, w)
    logits, _ = orc.prefill(0, emb, all_rows=True)
    err = np.abs(logits - ref).max() / np.abs(ref).max()
    assert err < 2e-5, err


def test_oracle_decode_path_matches_transformers():
    # prefill 12 rows, then 8 one-row decodes at positions 12..19: every
    # decode's logits equal the library model's row at that position
    shape = small_shape()
    w = scaled_weights(shape)
    emb = prefill_embeddings(shape, 20)
    ref = _transformers_logits(shape, w, emb)
    orc = TalkerOracle(shape, w)
    orc.prefill(1, emb[:12])
    for t in range(12, 20):
        lg, _ = orc.decode(1, emb[t])
        err = np.abs(lg - ref[t]).max() / np.abs(ref[t]).max()
        assert err < 2e-5, (t, err)
    assert orc.kv_len(1) == 20


# -- closed forms ------------------------------------------------------------------

def test_residual_path_closed_form():
    # with o_proj = down = 0 every layer returns its input, so the logits are
    # codec_head applied to the final RMSNorm of the embedding row
    shape = small_shape(n_layers=3)
    w = scaled_weights(shape)
    for lw in w["layers"]:
        lw["wo"][:] = 0
        lw["wd"][:] = 0
    emb = prefill_embeddings(shape, 5)
    lg, hid = TalkerOracle(shape, w).prefill(0, emb)
    x = emb[-1].astype(np.float64)
    hn = x / math.sqrt(np.mean(x * x) + shape.rms_eps) * w["g_final"]
    np.testing.assert_allclose(hid, hn, rtol=1e-12)
    np.testing.assert_allclose(lg, w["w_head"].astype(np.float64) @ hn,
                               rtol=1e-11, atol=1e-13)


def test_first_position_attention_is_v_projection():
    # at position 0 the attention output is the (cache-rounded) V of that row;
    # one layer with zero MLP: x1 = x + Wo @ repeat(V) exactly
    shape = small_shape(n_layers=1, kv_dtype="f16")
    w = scaled_weights(shape)
    lw = w["layers"][0]
    lw["wd"][:] = 0
    emb = prefill_embeddings(shape, 1)
    taps = []
    orc = TalkerOracle(shape, w)
    orc.extend(0, emb, taps=taps)
    x = emb[0].astype(np.float64)
    h = x / math.sqrt(np.mean(x * x) + shape.rms_eps) * lw["g_in"]
    v = (lw["wv"].astype(np.float64) @ h).astype(np.float32).astype(np.float16)
    v = v.astype(np.float64).reshape(shape.n_kv_heads, shape.head_dim)
    o = np.repeat(v, shape.n_heads // shape.n_kv_heads, axis=0).reshape(-1)
    np.testing.assert_allclose(taps[0][0], x + lw["wo"].astype(np.float64) @ o,
                               rtol=1e-12)


# -- path invariants -------------------------------------------------------------

@pytest.mark.parametrize("kv", ["f32", "f16"])
def test_prefill_equals_prefill_then_decode(kv):
    shape = small_shape(kv_dtype=kv)
    w = scaled_weights(shape)
    emb = prefill_embeddings(shape, 17)
    a = TalkerOracle(shape, w)
    la, ha = a.prefill(0, emb)
    b = TalkerOracle(shape, w)
    b.prefill(0, emb[:16])
    lb, hb = b.decode(0, emb[16])
    np.testing.assert_allclose(lb, la, rtol=1e-11, atol=1e-12)
    for l in range(shape.n_layers):
        for which in (0, 1):
            np.testing.assert_allclose(b.kv(0, l, which), a.kv(0, l, which),
                                       rtol=1e-11, atol=1e-12)


def test_layer_walk_over_a_stored_cache_reproduces_the_decode():
    # the harness of the 28-layer 32k GPU check: one decode step formed
    # layer by layer by one-layer oracles, each handed the stored K/V of the
    # earlier positions, equals the full oracle's decode step (logits and
    # the new K/V rows); a cache entry perturbed in the hand-over changes it
    shape = small_shape(kv_dtype="f16", n_layers=3)
    w = scaled_weights(shape)
    emb = prefill_embeddings(shape, 21)
    full = TalkerOracle(shape, w)
    full.prefill(0, emb[:20])
    ref, _ = full.decode(0, emb[20])
    pos = 20

    def walk(perturb=None):
        x = emb[20][None].astype(np.float64)
        for l in range(shape.n_layers):
            one = TalkerOracle(shape, {"layers": [w["layers"][l]], "g_final": w["g_final"],
                                       "w_head": w["w_head"]})
            one._reserve(0, pos + 1)
            one.kc[0][0, :, :pos] = full.kv(0, l, 0)[:, :pos]
            one.vc[0][0, :, :pos] = full.kv(0, l, 1)[:, :pos]
            if perturb == l:
                one.vc[0][0, 1, 3] += 0.25
            one.cur_len[0] = pos
            x = one.layer(0, x, 0, pos)
            if perturb is None:
                np.testing.assert_array_equal(one.kc[0][0, :, pos], full.kv(0, l, 0)[:, pos])
                np.testing.assert_array_equal(one.vc[0][0, :, pos], full.kv(0, l, 1)[:, pos])
        return one.head(x)[0][0]

    np.testing.assert_allclose(walk(), ref, rtol=1e-13, atol=1e-13)
    assert np.max(np.abs(walk(perturb=1) - ref)) > 1e-4 * np.max(np.abs(ref))


# -- the q8 cache: earlier positions quantised, the call's own rows fresh -------

def _q8_round_trip(t):
    """A cached K or V tensor [..., hd] replaced by its Q8_0 block round trip
    (the cache content the next call reads)."""
    a = t.numpy()
    return torch.from_numpy(ot.q8_block_dequantize(
        *ot.q8_block_quantize(a.astype(np.float32))).astype(np.float64).reshape(a.shape))


def test_q8_prefill_matches_transformers_unquantised():
    # a q8 prefill attends to its own rows unquantised, so every row equals
    # the library model, which never rounds K or V (the quantisation error
    # of Q8_0 is ~1/254 of a block's range, far above this tolerance)
    shape = small_shape(kv_dtype="q8")
    w = scaled_weights(shape)
    emb = prefill_embeddings(shape, 20)
    ref = _transformers_logits(shape, w, emb)
    logits, _ = TalkerOracle(shape, w).prefill(0, emb, all_rows=True)
    err = np.abs(logits - ref).max() / np.abs(ref).max()
    assert err < 2e-5, err


def test_q8_decode_and_extend_match_transformers_over_a_quantised_prefix():
    # transformers' own KV cache after a prefill of 12 rows, each layer's K
    # and V replaced by their Q8_0 round trip, then (a) one decode row and
    # (b) a 5-row extend through that cache: the library model joins the
    # quantised prefix with the fresh rows of the call, as the q8 oracle does
    from transformers import DynamicCache
    shape = small_shape(kv_dtype="q8")
    w = scaled_weights(shape)
    emb = prefill_embeddings(shape, 18)
    m = _transformers_model(shape, w)
    head = w["w_head"].astype(np.float64)
    for rows in (emb[12:13], emb[12:17]):
        cache = DynamicCache()
        with torch.no_grad():
            m(inputs_embeds=torch.from_numpy(emb[:12].astype(np.float64))[None],
              past_key_values=cache, use_cache=True)
            for lay in cache.layers:
                lay.keys = _q8_round_trip(lay.keys)
                lay.values = _q8_round_trip(lay.values)
            hs = m(inputs_embeds=torch.from_numpy(rows.astype(np.float64))[None],
                   past_key_values=cache, use_cache=True).last_hidden_state[0].numpy()
        ref = hs @ head.T
        orc = TalkerOracle(shape, w)
        orc.prefill(0, emb[:12])
        got, _ = orc.extend(0, rows, all_rows=True)
        err = np.abs(got - ref).max() / np.abs(ref).max()
        assert err < 2e-5, (len(rows), err)


def test_q8_prefill_and_prefill_plus_decode_differ_only_through_the_prefix():
    # prefill(T) attends to fresh rows; prefill(T-1) + decode reads rows
    # 0..T-2 back quantised.  Rows 0..T-2 of every layer's cache, and row
    # T-1 of layer 0 (a function of its own embedding only), are the same
    # either way; the logits differ, by about the quantisation error.
    shape = small_shape(kv_dtype="q8")
    w = scaled_weights(shape)
    emb = prefill_embeddings(shape, 17)
    a = TalkerOracle(shape, w)
    la, _ = a.prefill(0, emb)
    b = TalkerOracle(shape, w)
    b.prefill(0, emb[:16])
    lb, _ = b.decode(0, emb[16])
    for l in range(shape.n_layers):
        for which in (0, 1):
            np.testing.assert_array_equal(a.kv(0, l, which)[:, :16], b.kv(0, l, which)[:, :16])
    for which in (0, 1):
        np.testing.assert_array_equal(a.kv(0, 0, which), b.kv(0, 0, which))
    d = np.abs(la - lb).max() / np.abs(la).max()
    assert 1e-5 < d < 5e-2, d


def test_chunked_extend_equals_one_shot_and_batched_equals_serial():
    shape = small_shape(kv_dtype="f16")
    w = scaled_weights(shape)
    emb = prefill_embeddings(shape, 30)
    a = TalkerOracle(shape, w)
    la, _ = a.prefill(0, emb)
    b = TalkerOracle(shape, w)
    b.prefill(0, emb[:7])
    b.extend(0, emb[7:19])
    lb, _ = b.extend(0, emb[19:])
    np.testing.assert_allclose(lb, la, rtol=1e-11, atol=1e-12)
    # batched decode over three sequences equals three serial decodes
    c = TalkerOracle(shape, w)
    d = TalkerOracle(shape, w)
    for sq, n in ((0, 5), (1, 9), (2, 2)):
        e = prefill_embeddings(shape, n, seq=sq)
        c.prefill(sq, e)
        d.prefill(sq, e)
    steps = np.stack([step_embedding(shape, 0, seq=s) for s in (2, 0, 1)])
    lc, hc = c.decode_batch([2, 0, 1], steps)
    for i, sq in enumerate((2, 0, 1)):
        ld, hd_ = d.decode(sq, steps[i])
        np.testing.assert_array_equal(lc[i], ld)
    assert [c.kv_len(s) for s in range(3)] == [6, 10, 3]


def test_causality_later_rows_do_not_change_earlier_logits():
    shape = small_shape()
    w = scaled_weights(shape)
    emb = prefill_embeddings(shape, 12)
    la, _ = TalkerOracle(shape, w).prefill(0, emb, all_rows=True)
    emb2 = emb.copy()
    emb2[8:] += 5.0
    lb, _ = TalkerOracle(shape, w).prefill(0, emb2, all_rows=True)
    np.testing.assert_array_equal(la[:8], lb[:8])
    assert np.abs(la[8:] - lb[8:]).max() > 1e-3


def test_stale_cache_tail_is_never_read():
    shape = small_shape(kv_dtype="f16")
    w = scaled_weights(shape)
    emb = prefill_embeddings(shape, 20)
    a = TalkerOracle(shape, w)
    a.prefill(0, emb)
    a.kv_rewind(0, 11)
    for c in (a.kc[0], a.vc[0]):
        c[:, :, 11:, :] = np.nan
    la, _ = a.decode(0, emb[11])
    assert np.isfinite(la).all()
    b = TalkerOracle(shape, w)
    b.prefill(0, emb[:11])
    lb, _ = b.decode(0, emb[11])
    np.testing.assert_array_equal(la, lb)


def test_errors_leave_state_unchanged():
    shape = small_shape(cap=10)
    w = scaled_weights(shape)
    o = TalkerOracle(shape, w)
    o.prefill(0, prefill_embeddings(shape, 9))
    k_before = o.kv(0, 0, 0)
    o.decode(0, step_embedding(shape, 0))
    assert o.kv_len(0) == 10
    with pytest.raises(OverflowError):
        o.decode(0, step_embedding(shape, 1))
    with pytest.raises(OverflowError):
        o.prefill(1, prefill_embeddings(shape, 11))
    with pytest.raises(ValueError):
        o.kv_rewind(0, 11)
    with pytest.raises(ValueError):
        o.extend(0, np.zeros((0, shape.hidden)))
    assert o.kv_len(0) == 10 and o.kv_len(1) == 0
    np.testing.assert_array_equal(o.kv(0, 0, 0)[:, :9], k_before)


def test_precision_floor_f32_vs_f64():
    # the same forward in float32 stays within 1e-5 of float64 relative to the
    # logit scale: the floor under the kernel tolerances
    shape = small_shape(kv_dtype="f16", hidden=128, intermediate=384,
                        n_heads=8, n_kv_heads=4)
    w = make_weights(shape)
    emb = prefill_embeddings(shape, 24)
    l64, _ = TalkerOracle(shape, w).prefill(0, emb, all_rows=True)
    l32, _ = TalkerOracle(shape, w, dtype=np.float32).prefill(0, emb,
                                                               all_rows=True)
    err = np.abs(l32 - l64).max() / np.abs(l64).max()
    assert err < 1e-5, err


# -- planted mistakes: each must be caught by a pin above ------------------------

def _interleaved_rope(x, pos, theta):
    hd = x.shape[-1]
    inv = ot.rope_inv_freq(hd, theta)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = b * c + a * s
    return out


def _sign_flipped_rope(x, pos, theta):
    return ot.rope_neox(x, -np.asarray(pos), theta)


_plain_attention = ot.causal_gqa_attention


def _modulo_gqa(q, kc, vc, positions, scale):
    # wrong group map: h % n_kv instead of h // G
    nkv = kc.shape[0]
    perm = [h % nkv for h in range(q.shape[1])]
    return _plain_attention(q, kc[perm], vc[perm], positions, scale)


def _fresh_kv_in_prefill(self, l, x, seq, p0):
    # reads fresh float64 K/V for the rows just computed (not the f16 cache)
    s, w = self.s, self.layers[l]
    T = x.shape[0]
    pos = p0 + np.arange(T)
    h = ot.rms_norm(x, w["g_in"], s.rms_eps)
    q = (h @ w["wq"].T).reshape(T, s.n_heads, s.head_dim)
    k = (h @ w["wk"].T).reshape(T, s.n_kv_heads, s.head_dim)
    v = (h @ w["wv"].T).reshape(T, s.n_kv_heads, s.head_dim)
    q = ot.rope_neox(ot.rms_norm(q, w["g_q"], s.rms_eps), pos[:, None],
                     s.rope_theta)
    k = ot.rope_neox(ot.rms_norm(k, w["g_k"], s.rms_eps), pos[:, None],
                     s.rope_theta)
    kc = self.kc[seq][l].copy()
    vc = self.vc[seq][l].copy()
    kc[:, p0:p0 + T] = k.transpose(1, 0, 2)
    vc[:, p0:p0 + T] = v.transpose(1, 0, 2)
    self.kc[seq][l, :, p0:p0 + T] = ot.round_kv(k.transpose(1, 0, 2),
                                                s.kv_dtype, self.dtype)
    self.vc[seq][l, :, p0:p0 + T] = ot.round_kv(v.transpose(1, 0, 2),
                                                s.kv_dtype, self.dtype)
    o = ot.causal_gqa_attention(q, kc, vc, pos, self.scale)
    x = x + o.reshape(T, s.q_dim) @ w["wo"].T
    h2 = ot.rms_norm(x, w["g_post"], s.rms_eps)
    return x + ot.swiglu(h2 @ w["wg"].T, h2 @ w["wu"].T) @ w["wd"].T


def test_planted_rope_mistakes_are_caught(monkeypatch):
    import tests.test_oracle_steps as steps
    for bad in (_interleaved_rope, _sign_flipped_rope):
        monkeypatch.setattr(steps, "rope_neox", bad)
        with pytest.raises(AssertionError):
            steps.test_rope_hand_worked_examples("rope_neox_hd4_pos2_mixed.txt")
    monkeypatch.setattr(ot, "rope_neox", _interleaved_rope)
    with pytest.raises(AssertionError):
        test_oracle_matches_transformers_qwen3_all_rows()


def test_planted_gqa_mistake_is_caught(monkeypatch):
    import tests.test_oracle_steps as steps
    monkeypatch.setattr(steps, "causal_gqa_attention", _modulo_gqa)
    with pytest.raises(AssertionError):
        steps.test_attention_matches_torch_sdpa_gqa()


def test_planted_fresh_kv_reading_is_caught(monkeypatch):
    # the read-after-write reading makes prefill(T) equal prefill(T-1) + decode
    # to rounding; reading fresh values in prefill breaks it for an f16 cache
    monkeypatch.setattr(TalkerOracle, "layer", _fresh_kv_in_prefill)
    with pytest.raises(AssertionError):
        test_prefill_equals_prefill_then_decode("f16")


def test_planted_quantised_current_rows_are_caught(monkeypatch):
    # attending to the quantised current rows (the cache itself) instead of
    # the fresh ones must fail both q8 pins against the library model
    monkeypatch.setattr(TalkerOracle, "attended_kv",
                        lambda self, l, seq, p0, k, v: (self.kc[seq][l], self.vc[seq][l]))
    with pytest.raises(AssertionError):
        test_q8_prefill_matches_transformers_unquantised()
    with pytest.raises(AssertionError):
        test_q8_decode_and_extend_match_transformers_over_a_quantised_prefix()


def test_planted_missing_eps_and_gain_are_caught(monkeypatch):
    import tests.test_oracle_steps as steps
    monkeypatch.setattr(steps, "rms_norm",
                        lambda x, g, eps: x / np.sqrt(np.mean(x * x, -1,
                                                              keepdims=True)) * g)
    with pytest.raises(AssertionError):
        steps.test_rms_norm_constant_vector_closed_form()
    monkeypatch.setattr(steps, "rms_norm",
                        lambda x, g, eps: ot.rms_norm(x, 1.0 + g, eps))
    with pytest.raises(AssertionError):
        steps.test_rms_norm_matches_torch_rms_norm()


def test_planted_swapped_gate_up_is_caught(monkeypatch):
    monkeypatch.setattr(ot, "swiglu", lambda g, u: ot.silu(u) * g)
    with pytest.raises(AssertionError):
        test_oracle_matches_transformers_qwen3_all_rows()


def test_sampled_rows_equal_full_extend_on_one_layer():
    # the sampled-row path of the long-context checks is the full extend
    # restricted to the listed rows (same cache, same outputs)
    shape = workload("tiny_f32_2l").with_(cap=64)
    w = make_weights(shape, n_layers=1)
    emb = prefill_embeddings(shape, 40)
    full = TalkerOracle(shape, w)
    lf, hf = full.prefill(0, emb[:25], all_rows=True)
    lf2, hf2 = full.extend(0, emb[25:], all_rows=True)
    samp = TalkerOracle(shape, w)
    rows1 = [0, 7, 24]
    ls, hs = samp.extend_rows(0, emb[:25], rows1)
    rows2 = [0, 3, 14]
    ls2, hs2 = samp.extend_rows(0, emb[25:], rows2)
    np.testing.assert_allclose(ls, lf[rows1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hs2, hf2[rows2], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ls2, lf2[rows2], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(samp.kv(0, 0, 0), full.kv(0, 0, 0))
    np.testing.assert_array_equal(samp.kv(0, 0, 1), full.kv(0, 0, 1))
    with pytest.raises(ValueError):
        TalkerOracle(shape, make_weights(shape)).extend_rows(0, emb[:4], [0])


# -- stacked output heads and the code predictor frame ---------------------------

def test_selected_head_forms_the_logits():
    # heads i = 2^i * head 0 (exact in float32), so the logits read through
    # head i are exactly 2^i times head 0's; a wrong index changes the factor
    shape = small_shape(n_out_heads=4)
    w = scaled_weights(shape)
    w["w_head"] = np.stack([np.float32(2 ** i) * w["w_head"][0] for i in range(4)])
    emb = prefill_embeddings(shape, 6)
    base = None
    for i in range(4):
        orc = TalkerOracle(shape, w)
        orc.select_head(i)
        lg, hid = orc.prefill(0, emb)
        if base is None:
            base, hid0 = lg, hid
        np.testing.assert_array_equal(lg, 2 ** i * base)
        np.testing.assert_array_equal(hid, hid0)  # the hidden state does not depend on the head
    with pytest.raises(ValueError):
        orc.select_head(4)


def test_code_predictor_frame_equals_prefills_through_each_head():
    # step j of a frame (cache of j + 1 positions plus the new one, head j)
    # gives what a fresh prefill of the same j + 2 rows gives through head j
    shape = small_shape(n_out_heads=5, vocab=24)
    w = scaled_weights(shape)
    rows = prefill_embeddings(shape, 6)
    frame = ot.code_predictor_frame(TalkerOracle(shape, w), rows[0], rows[1], rows[2:])
    assert len(frame) == 5
    for j in range(5):
        orc = TalkerOracle(shape, w)
        orc.select_head(j)
        lg, _ = orc.prefill(0, rows[:j + 2])
        np.testing.assert_allclose(frame[j], lg, rtol=1e-10, atol=1e-12)
    # the heads differ, so a frame that kept head 0 would not match
    orc = TalkerOracle(shape, w)
    lg, _ = orc.prefill(0, rows[:4])
    assert not np.allclose(frame[2], lg, rtol=1e-3)


def test_prefill_batch_is_independent_prefills():
    # each listed sequence ends as a lone prefill leaves it; sequences not
    # listed keep their caches; duplicates and overlong rows are rejected
    shape = small_shape(n_seqs=4)
    w = scaled_weights(shape)
    embs = np.stack([prefill_embeddings(shape, 9, seq=s) for s in range(3)])
    orc = TalkerOracle(shape, w)
    keep_emb = prefill_embeddings(shape, 5, seq=3)
    orc.prefill(1, keep_emb)                 # will be overwritten
    orc.prefill(3, keep_emb)                 # not listed: untouched
    before = orc.kv(3, 1, 0)
    lg, hid = orc.prefill_batch([2, 0, 1], embs)
    for b, sq in enumerate([2, 0, 1]):
        ref = TalkerOracle(shape, w)
        rl, rh = ref.prefill(sq, embs[b])
        np.testing.assert_array_equal(lg[b], rl)
        np.testing.assert_array_equal(hid[b], rh)
        np.testing.assert_array_equal(orc.kv(sq, 1, 1), ref.kv(sq, 1, 1))
        assert orc.kv_len(sq) == 9
    np.testing.assert_array_equal(orc.kv(3, 1, 0), before)
    with pytest.raises(ValueError):
        orc.prefill_batch([0, 0], embs[:2])
    with pytest.raises(OverflowError):
        orc.prefill_batch([0], np.zeros((1, shape.cap + 1, shape.hidden)))


# -- power of the long-context attention check -----------------------------------

def _window_attention(q, kc, vc, positions, scale):
    # planted: keys older than 2048 positions dropped
    out = np.empty_like(q)
    for t in range(q.shape[0]):
        lo = max(0, int(positions[t]) - 2047)
        out[t:t + 1] = _plain_attention(q[t:t + 1], kc[:, lo:], vc[:, lo:],
                                        positions[t:t + 1] - lo, scale)
    return out


def _long_context_rows(shape, w, n_ctx, steps):
    """Logits of the rows the long-context GPU check reads: the last row of
    each 2048-row chunk, then ``steps`` decode steps."""
    from synth import step_embedding as se
    orc = TalkerOracle(shape, w)
    emb = prefill_embeddings(shape, n_ctx)
    out = []
    for c0 in range(0, n_ctx, 2048):
        ch = emb[c0:c0 + 2048]
        out.append(orc.extend_rows(0, ch, [len(ch) - 1])[0][0])
    for k in range(steps):
        out.append(orc.decode(0, se(shape, k))[0])
    return np.stack(out)


def test_long_context_check_sees_the_attention(monkeypatch):
    # the sharp-attention workload (q/k norm gains x4) at 4096 positions: the
    # GPU check's statistics (logit error over the checked rows; error over
    # the attention term) must reject an attention that is zeroed, that drops
    # keys older than 2048 positions, or that maps query heads to the wrong
    # KV head.  With the plain gains the attention term at long context is
    # about the size of the tolerance, which is why the check uses this one.
    shape = workload("talker_1l_ctx32k_sharp").with_(cap=4200)
    w = make_weights(shape)
    ref = _long_context_rows(shape, w, 4096, 4)
    import copy
    w0 = copy.deepcopy(w)
    w0["layers"][0]["wo"][:] = 0
    noatt = _long_context_rows(shape, w0, 4096, 4)
    att = np.abs(ref - noatt).max(axis=1)
    assert (att / np.abs(ref).max(axis=1) > 0.2).all()
    bad = {"zeroed": noatt}
    monkeypatch.setattr(ot, "causal_gqa_attention", _window_attention)
    bad["window"] = _long_context_rows(shape, w, 4096, 4)
    monkeypatch.setattr(ot, "causal_gqa_attention", _modulo_gqa)
    bad["gqa map"] = _long_context_rows(shape, w, 4096, 4)
    for name, got in bad.items():
        err = (np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)).max()
        ratio = (np.abs(got - ref).max(axis=1) / att).max()
        assert err > 2e-2 and ratio > 0.1, (name, err, ratio)
