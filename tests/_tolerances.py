"""Error bounds that the parity tests derive from the arithmetic (no GPU).

Index projection (msa_index_project).  Per token t and group g the kernel
sums the d_model products w[o][j] * x[t][j] of each output o in f32 on the
matrix cores, then normalises the head (f32) and rotates half of it (angles
in f64, products in f32).  Model of the f32 sum:

  * every product is added to a running partial sum S_k and rounded once
    (a chain of d_model f32 fused multiply-adds: the most roundings any
    order of the matrix-core steps can make; a step that rounds once per
    four products makes a quarter of them);
  * a rounding of a value of magnitude |S| errs by at most half an ulp,
    uniformly, so its standard deviation is at most u|S| / sqrt(3) with
    u = 2^-24 (an ulp is at most 2u|S|);
  * the terms come in an order unrelated to their values, so the increments
    are exchangeable: given the exact sum y and V = sum_j (w_j x_j)^2,
    E[S_k^2] = (k/n)^2 y^2 + k(n-k)/(n-1) (V/n - y^2/n^2), and summed over
    the n = d_model steps  sum_k E[S_k^2] ~= n (y^2 / 3 + V / 6).

So the error of y has standard deviation sigma_y = u / sqrt(3) * sqrt(n (y^2/3
+ V/6)): it grows with the output's own magnitude, which a fixed bound
ignores (an output near 5 sigma of the head's distribution errs ~3x more
than a typical one).  sigma_y is the expectation over summation orders; a
particular order's partial sums can wander further than that expectation,
so the error / sigma_y ratio has a heavier tail than a Gaussian: over an
emulated f32 chain at d_model 3072 its rms is 0.73 and its quantiles are
3.3 (1e-3), 4.4 (1e-4), 5.4 (1e-5), with a maximum of 7.7 over 4.2 million
outputs (about one more unit per decade).  The norm multiplies by r (1 + gamma), r = 1/rms(y);
the rotation mixes a pair with weights cos, sin (so the pair's larger sigma
bounds the result).  The norm's own sum of 128 squares, the reciprocal
square root, the gain and the rotation's products and f32 sin/cos round
a bounded number of times at the magnitude of the result: 16 u |z| per
element covers them.  The bound per element is 10 sigma + 16 u |z|: by the
tail above, a ratio of 10 is reached about once in 1e9 outputs, against
4.2 million outputs in a 4096-token prefill chunk.  For a typical output
(|y| ~ 1) at d_model 3072 that is 1.4e-5, for |y| ~ 5 5.6e-5.
tests/test_tolerance_models.py checks the model against an f32 chain
emulated on the CPU.
"""
from __future__ import annotations

import numpy as np

U32 = 2.0 ** -24
N_SIGMA = 10.0


def sum_sigma(y: np.ndarray, v: np.ndarray, n: int) -> np.ndarray:
    """Standard deviation of an f32 chain sum of n terms with exact sum y and
    sum of squared terms v (the model above)."""
    return U32 / np.sqrt(3.0) * np.sqrt(n * (y * y / 3.0 + v / 6.0))


def projection_bound(x, w, gain, rot_dim: int, eps: float, n_group: int = 4) -> np.ndarray:
    """Per-element bound |gpu - exact| for one projection (queries or keys).

    x [n_tok][d] f32, w [n_group * hd][d] f32, gain [n_group][hd] f32.
    Returns [n_tok][n_group][hd] f64."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    n_tok, d = x.shape
    hd = w.shape[0] // n_group
    y = (x @ w.T).reshape(n_tok, n_group, hd)
    v = ((x * x) @ (w * w).T).reshape(n_tok, n_group, hd)
    r = 1.0 / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)
    fac = np.abs(r * (1.0 + np.asarray(gain, np.float64))[None])
    sig = fac * sum_sigma(y, v, d)
    z = np.abs(y * r * (1.0 + np.asarray(gain, np.float64))[None])
    mag = z.copy()
    if rot_dim:
        half = rot_dim // 2
        a, b = slice(0, half), slice(half, rot_dim)
        s_pair = np.maximum(sig[..., a], sig[..., b])
        m_pair = z[..., a] + z[..., b]
        sig[..., a] = s_pair
        sig[..., b] = s_pair
        mag[..., a] = m_pair
        mag[..., b] = m_pair
    return N_SIGMA * sig + 16.0 * U32 * mag + 1e-9
