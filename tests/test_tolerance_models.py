"""CPU checks of the error models that set the GPU parity tolerances
(tests/_tolerances.py): the model must bound what the arithmetic it
describes actually does, and must not be vacuous."""
import numpy as np

import workloads as W
from _tolerances import N_SIGMA, projection_bound, sum_sigma


def _chain_f32(x, w):
    """Each product added to an f32 running sum with one rounding (a chain of
    fused multiply-adds): the most roundings any order of the kernel's steps
    makes."""
    xd, wd = x.astype(np.float64), w.astype(np.float64)
    s = np.zeros((x.shape[0], w.shape[0]), np.float32)
    for j in range(x.shape[1]):
        s = (s.astype(np.float64) + np.outer(xd[:, j], wd[:, j])).astype(np.float32)
    return s


def test_projection_sum_model_bounds_an_f32_chain():
    d = W.PROJ_D_MODEL
    x = W.hidden_states(256, d, 3)
    w = W.projection_weights(d, 3)["w_q"]
    got = _chain_f32(x, w)
    xd, wd = x.astype(np.float64), w.astype(np.float64)
    y = xd @ wd.T
    v = (xd * xd) @ (wd * wd).T
    r = (got - y) / sum_sigma(y, v, d)
    rms, mx = float(np.sqrt(np.mean(r * r))), float(np.abs(r).max())
    print(f"error / sigma over {r.size} sums: rms {rms:.3f}, max {mx:.2f}")
    assert 0.5 <= rms <= 1.0          # sigma bounds the per-rounding spread without being vacuous
    assert mx < 0.8 * N_SIGMA         # the tail stays well inside the bound
    # magnitude-aware: the same model holds for small and large outputs
    for lo, hi in ((0.0, 1.0), (1.0, 2.0), (2.0, 9.0)):
        m = (np.abs(y) >= lo) & (np.abs(y) < hi)
        assert 0.5 <= np.sqrt(np.mean(r[m] ** 2)) <= 1.0, (lo, hi)


def test_projection_bound_catches_a_lost_term():
    """Dropping one product from a sum (the kind of slip a kernel makes) is
    far outside the bound, at every output."""
    d = 768
    x = W.hidden_states(64, d, 4)
    p = W.projection_weights(d, 4)
    b = projection_bound(x, p["w_q"], p["g_q"], W.PROJ_ROT_DIM, W.PROJ_EPS)
    assert b.shape == (64, 4, 128)
    assert float(b.max()) < 1e-4
    # the size of one term's contribution after the norm is about 1/sqrt(d)
    term = np.abs(x[:, :1].astype(np.float64) * p["w_q"][:, 0].astype(np.float64)[None]).reshape(64, 4, 128)
    assert np.median(term / b) > 10
