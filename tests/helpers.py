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


def argmax_ok(g, o, tol) -> bool:
    """Codebook-0 argmax: equal to the oracle's, except where other logits lie
    within 2 * tol * max|logit| of the oracle's maximum; then the GPU's pick
    must be one of those (several answers are correct inside the band)."""
    g = np.asarray(g)
    o = np.asarray(o)
    ig, io = int(np.argmax(g)), int(np.argmax(o))
    if ig == io:
        return True
    return bool(o[io] - o[ig] <= 2 * tol * np.abs(o).max())


def argmax_in_band(o, tol) -> bool:
    """True when the oracle's top-2 gap is inside the tolerance band."""
    o = np.asarray(o)
    top2 = np.sort(o)[-2:]
    return bool(top2[1] - top2[0] <= 2 * tol * np.abs(o).max())
