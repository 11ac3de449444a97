"""Pins of the frame-step oracle (CPU only): the step-embedding gather-sum
against a one-hot matrix product in float64 and exact special cases; the
suppressed greedy pick against hand examples and numpy's argmax on a masked
copy."""
import numpy as np
import pytest

from oracle.frame import embed_sum, suppressed_argmax


def _tables(rng, G=4, rows=(7, 5, 5, 5), hidden=6):
    return [rng.standard_normal((rows[g], hidden)).astype(np.float32) for g in range(G)]


def test_embed_sum_equals_one_hot_products():
    rng = np.random.default_rng(5)
    tabs = _tables(rng)
    ids = np.array([[0, 6, 3], [4, 0, 2], [1, 1, 1], [3, 2, 0]])
    ov = rng.standard_normal((3, 6)).astype(np.float32)
    got = embed_sum(tabs, ids, ov)
    want = sum(np.eye(t.shape[0])[ids[g]] @ t.astype(np.float64) for g, t in enumerate(tabs))
    want = want + ov
    np.testing.assert_allclose(got, want, rtol=2e-6, atol=2e-6)
    assert got.dtype == np.float32


def test_embed_sum_special_cases():
    rng = np.random.default_rng(6)
    tabs = _tables(rng, G=1, rows=(9,))
    ids = np.array([[8, 0, 8]])
    np.testing.assert_array_equal(embed_sum(tabs, ids), tabs[0][[8, 0, 8]])
    # a zero table adds nothing, exactly
    z = [tabs[0], np.zeros((4, 6), np.float32)]
    np.testing.assert_array_equal(embed_sum(z, np.array([[2], [3]])), tabs[0][[2]])
    with pytest.raises(IndexError):
        embed_sum(tabs, np.array([[9]]))
    with pytest.raises(IndexError):
        embed_sum(tabs, np.array([[-1]]))


def test_suppressed_argmax_hand_examples():
    assert suppressed_argmax([1.0, 3.0, 3.0, 2.0], 4, -1) == 1          # tie: lowest index
    assert suppressed_argmax([1.0, 0.0, 2.0, 9.0, 8.0], 3, -1) == 2      # 3, 4 suppressed
    assert suppressed_argmax([1.0, 0.0, 2.0, 9.0, 8.0], 3, 4) == 4       # 4 kept
    assert suppressed_argmax([1.0, 0.0, 2.0, 9.0, 8.0], 3, 3) == 3
    assert suppressed_argmax([np.nan, 0.5, np.nan], 3, -1) == 1          # NaN never wins
    assert suppressed_argmax([-np.inf, -np.inf, 5.0], 2, -1) == 0        # nothing finite
    assert suppressed_argmax([np.nan], 1, -1) == 0


def test_suppressed_argmax_equals_masked_numpy_argmax():
    rng = np.random.default_rng(7)
    V = 3072
    for trial in range(20):
        lg = rng.standard_normal(V).astype(np.float32)
        if trial % 3 == 0:
            lg[rng.integers(V - 1024, V)] = 50.0   # a suppressed spike
        keep = 2150 if trial % 2 else -1
        if trial % 4 == 1:
            lg[2150] = 60.0                          # the kept id wins
        m = lg.astype(np.float64).copy()
        mask = np.arange(V) >= V - 1024
        if keep >= 0:
            mask[keep] = False
        m[mask] = -np.inf
        assert suppressed_argmax(lg, V - 1024, keep) == int(np.argmax(m)), trial
