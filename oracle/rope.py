"""Rotary position embedding in fp64 (RoFormer, named by Tree Training's reference list).

The pages give no convention.  Reading used here: frequencies
theta_k = base^(-2k/d) for k < d/2, "rotate-half" pairing of coordinate k
with k + d/2:

    x'_k       = x_k cos(p theta_k) - x_{k+d/2} sin(p theta_k)
    x'_{k+d/2} = x_{k+d/2} cos(p theta_k) + x_k sin(p theta_k)

with p the position of the token in its branch (its depth in the tree).
"""
import numpy as np


def angles(pos, d, base):
    half = d // 2
    k = np.arange(half, dtype=np.float64)
    theta = np.power(float(base), -2.0 * k / d)
    return np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]


def rotate(x, pos, base, inverse=False):
    """x: [L, H, d] fp64, pos: [L]; returns R(pos) x (or R(pos)^T x)."""
    if base is None or base == 0:
        return np.array(x, dtype=np.float64, copy=True)
    d = x.shape[-1]
    half = d // 2
    a = angles(pos, d, base)
    c = np.cos(a)[:, None, :]
    s = np.sin(a)[:, None, :]
    if inverse:
        s = -s
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
