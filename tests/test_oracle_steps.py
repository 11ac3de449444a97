"""Pins of the oracle's elementary steps against closed forms, hand-worked
values, brute force and independent library routines (CPU only)."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import (causal_gqa_attention, rms_norm, rope_inv_freq, rope_neox,
                    round_kv, silu, swiglu)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = [l for l in open(os.path.join(GOLDEN, name)) if l.strip()
            and not l.startswith("#")]
    hd, theta, pos = rows[0].split()
    x = np.array(rows[1].split(), dtype=np.float64)
    exp = np.array(rows[2].split(), dtype=np.float64)
    return int(hd), float(theta), int(pos), x, exp


# -- RMSNorm -------------------------------------------------------------------

def test_rms_norm_constant_vector_closed_form():
    # c * 1 has mean square c^2, so the result is c / sqrt(c^2 + eps) * w
    rng = np.random.default_rng(0)
    for c in (2.0, -0.5, 3.0e4):
        for eps in (1e-6, 0.25):
            w = rng.standard_normal(64)
            got = rms_norm(np.full(64, c), w, eps)
            np.testing.assert_allclose(got, c / math.sqrt(c * c + eps) * w,
                                       rtol=1e-14)


def test_rms_norm_scale_invariant_without_eps():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 32))
    w = rng.standard_normal(32)
    np.testing.assert_allclose(rms_norm(7.5 * x, w, 0.0), rms_norm(x, w, 0.0),
                               rtol=1e-13)
    # unit gain and eps 0: each row has mean square exactly 1
    y = rms_norm(x, np.ones(32), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)


def test_rms_norm_matches_torch_rms_norm():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 96)) * 3
    w = 1 + 0.05 * rng.standard_normal(96)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,),
                                       torch.from_numpy(w), eps=1e-6).numpy()
    np.testing.assert_allclose(rms_norm(x, w, 1e-6), ref, rtol=1e-12)


def test_qk_norm_per_head_rms_with_unit_gain():
    # per-head RMS over head_dim of the output equals sqrt(m / (m + eps)),
    # m the input's mean square over that head
    rng = np.random.default_rng(3)
    q = rng.standard_normal((3, 4, 16)) * 1e-3     # small m makes eps matter
    eps = 1e-6
    y = rms_norm(q, np.ones(16), eps)
    m = np.mean(q * q, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)),
                               np.sqrt(m / (m + eps)), rtol=1e-12)


# -- RoPE ------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["rope_neox_hd4_pos1.txt",
                                  "rope_neox_hd4_pos2_mixed.txt"])
def test_rope_hand_worked_examples(name):
    hd, theta, pos, x, exp = _read_golden(name)
    np.testing.assert_allclose(rope_neox(x, pos, theta), exp, rtol=0,
                               atol=1e-14)


def test_rope_identity_at_position_zero():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 3, 128))
    assert np.array_equal(rope_neox(x, 0, 1e6), x)


def test_rope_preserves_pair_norms():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((9, 128))
    pos = np.arange(9) * 1000 + 17
    y = rope_neox(x, pos, 1e6)
    n_in = x[:, :64] ** 2 + x[:, 64:] ** 2
    n_out = y[:, :64] ** 2 + y[:, 64:] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-12)


def test_rope_relative_position_invariance():
    rng = np.random.default_rng(6)
    q = rng.standard_normal(128)
    k = rng.standard_normal(128)
    for m, n, sh in ((5, 2, 11), (100, 40, 3000), (0, 0, 31999)):
        a = rope_neox(q, m, 1e6) @ rope_neox(k, n, 1e6)
        b = rope_neox(q, m + sh, 1e6) @ rope_neox(k, n + sh, 1e6)
        assert abs(a - b) < 1e-9 * max(1.0, abs(a))


def test_rope_inv_freq_endpoints():
    f = rope_inv_freq(128, 1e6)
    assert f[0] == 1.0
    np.testing.assert_allclose(f[-1], 1e6 ** (-126 / 128), rtol=1e-15)
    np.testing.assert_allclose(f[1:] / f[:-1], 1e6 ** (-2 / 128), rtol=1e-13)


# -- SwiGLU ------------------------------------------------------------------------

def test_silu_special_values_and_library():
    from scipy.special import expit
    assert silu(np.array(0.0)) == 0.0
    z = np.array([40.0, 80.0])
    np.testing.assert_allclose(silu(z), z, rtol=1e-15)
    assert abs(silu(np.array(-50.0))) < 1e-19
    z = np.linspace(-20, 20, 401)
    np.testing.assert_allclose(silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    g = np.random.default_rng(7).standard_normal(50)
    u = np.random.default_rng(8).standard_normal(50)
    ref = torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u
    np.testing.assert_allclose(swiglu(g, u), ref, rtol=1e-14)


def test_round_kv_is_ieee_half_and_single():
    z = np.array([1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 65504.0, 1e-8, 0.1])
    h = round_kv(z, "f16", np.float64)
    # ties to even: 1 + 2^-11 is halfway between 1 and 1 + 2^-10 -> 1
    assert h[0] == 1.0 and h[1] == 1.0 + 2 ** -9
    assert h[2] == 65504.0
    assert h[3] == np.float64(np.float16(1e-8))
    np.testing.assert_array_equal(round_kv(z, "f32", np.float64),
                                  z.astype(np.float32).astype(np.float64))


# -- attention --------------------------------------------------------------------

def _brute_attention(q, kc, vc, positions, scale):
    """Scalar loops: one query row, one head, one key at a time."""
    T, nq, hd = q.shape
    nkv = kc.shape[0]
    G = nq // nkv
    out = np.zeros_like(q)
    for t in range(T):
        for h in range(nq):
            g = h // G
            sc = []
            for j in range(positions[t] + 1):
                acc = 0.0
                for d in range(hd):
                    acc += q[t, h, d] * kc[g, j, d]
                sc.append(acc * scale)
            mx = max(sc)
            e = [math.exp(v - mx) for v in sc]
            z = sum(e)
            for d in range(hd):
                acc = 0.0
                for j in range(len(e)):
                    acc += e[j] / z * vc[g, j, d]
                out[t, h, d] = acc
    return out


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(9)
    T, nq, nkv, hd, n = 3, 4, 2, 5, 7
    q = rng.standard_normal((T, nq, hd))
    kc = rng.standard_normal((nkv, n, hd))
    vc = rng.standard_normal((nkv, n, hd))
    pos = np.array([2, 4, 6])
    got = causal_gqa_attention(q, kc, vc, pos, 0.37)
    np.testing.assert_allclose(got, _brute_attention(q, kc, vc, pos, 0.37),
                               rtol=1e-12, atol=1e-14)


def test_attention_first_position_returns_v():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 4, 8))
    kc = rng.standard_normal((2, 3, 8))
    vc = rng.standard_normal((2, 3, 8))
    out = causal_gqa_attention(q, kc, vc, np.array([0]), 0.1)
    for h in range(4):
        assert np.array_equal(out[0, h], vc[h // 2, 0])


def test_attention_weights_sum_to_one():
    # with every value row equal to 1 the output is the sum of the softmax weights
    rng = np.random.default_rng(11)
    q = rng.standard_normal((5, 4, 8)) * 10
    kc = rng.standard_normal((2, 9, 8)) * 10
    out = causal_gqa_attention(q, kc, np.ones((2, 9, 8)),
                               np.array([0, 3, 5, 7, 8]), 1.0)
    np.testing.assert_allclose(out, 1.0, rtol=1e-13)


def test_attention_mha_special_case_and_gqa_repeat():
    rng = np.random.default_rng(12)
    T, nq, hd, n = 4, 6, 16, 10
    q = rng.standard_normal((T, nq, hd))
    pos = np.array([3, 6, 8, 9])
    # GQA with 2 KV heads equals MHA over K/V repeated per query group
    kc = rng.standard_normal((2, n, hd))
    vc = rng.standard_normal((2, n, hd))
    gqa = causal_gqa_attention(q, kc, vc, pos, 0.25)
    mha = causal_gqa_attention(q, np.repeat(kc, 3, axis=0),
                               np.repeat(vc, 3, axis=0), pos, 0.25)
    np.testing.assert_allclose(gqa, mha, rtol=1e-13)


def test_attention_matches_torch_sdpa_gqa():
    rng = np.random.default_rng(13)
    T, nq, nkv, hd, n = 6, 16, 8, 32, 20
    q = rng.standard_normal((T, nq, hd))
    kc = rng.standard_normal((nkv, n, hd))
    vc = rng.standard_normal((nkv, n, hd))
    pos = np.arange(n - T, n)
    got = causal_gqa_attention(q, kc, vc, pos, 1 / math.sqrt(hd))
    mask = torch.from_numpy(np.arange(n)[None, :] <= pos[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(1, 0, 2))[None],
        torch.from_numpy(kc)[None], torch.from_numpy(vc)[None],
        attn_mask=mask, enable_gqa=True)[0].numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)


# -- Q8_0 KV blocks -------------------------------------------------------------

def test_q8_block_closed_forms():
    from oracle.talker import q8_block_dequantize, q8_block_quantize
    # a block on the grid of its own scale comes back exactly
    d = np.float32(0.5)
    codes = np.arange(-127, 128, 8, dtype=np.int8)[:32]
    codes = np.concatenate([codes, np.zeros(32 - codes.size, np.int8)])
    codes[0] = 127
    x = codes.astype(np.float32) * d
    q, s = q8_block_quantize(x)
    assert s[0] == np.float16(0.5)
    np.testing.assert_array_equal(q[0], codes)
    np.testing.assert_array_equal(q8_block_dequantize(q, s), x)
    # zero block: zero scale and codes
    q, s = q8_block_quantize(np.zeros(64, np.float32))
    assert not q.any() and not s.any()
    # sign symmetry, the largest magnitude maps to +-127
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 128)).astype(np.float32)
    q, s = q8_block_quantize(x)
    qn, sn = q8_block_quantize(-x)
    np.testing.assert_array_equal(qn, -q)
    np.testing.assert_array_equal(sn, s)
    assert (np.abs(q).max(axis=-1) == 127).all()
    # ties go away from zero: 0.5 and 1.5 steps of d = 127 / 127
    x = np.zeros(32, np.float32)
    x[0], x[1], x[2], x[3] = 127.0, 0.5, -0.5, 1.5
    q, _ = q8_block_quantize(x)
    assert list(q[0, :4]) == [127, 1, -1, 2]


def test_q8_round_trip_error_bound():
    from oracle.talker import round_kv
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((7, 128)) * rng.uniform(0.01, 10, (7, 1))).astype(np.float32)
    y = round_kv(x, "q8", np.float64)
    b = np.abs(x.reshape(7, 4, 32)).max(axis=-1) / 127.0     # float32 scale per block
    err = np.abs(y - x).reshape(7, 4, 32).max(axis=-1)
    # half a step of the float32 scale, plus the float16 rounding of the
    # scale applied to codes up to 127
    assert (err <= b * (0.5 + 127 * 2.0 ** -11) + 1e-12).all()
    assert (err > 0).any()
