"""Equivariant merged RMS layer norm, fp64 (test infrastructure only).

"EquiformerV3: Scaling Efficient, Expressive, and General SE(3)-Equivariant
Graph Attention Transformers", technical summary, section 2.B.1: one
root-mean-square statistic is shared by all degrees l >= 0 of a node's
irreps features (earlier models normalised each degree, or groups of
degrees, on their own), which keeps the relative weight of the degrees.

Reading (the page gives no formula): for node i with features
x[(l, m), c], l = 0..L, m = -l..l, c = 0..C-1,

    s_i = mean over all (l, m, c) of x_i[(l, m), c]^2
    y_i[(l, m), c] = gamma[l][c] * x_i[(l, m), c] / sqrt(s_i + eps)

with a gain per degree and channel (shared by the 2l + 1 components of a
degree, so the map commutes with rotations), no centring and no bias.

Parity pinned by tests/test_oracle_norm.py: unit mean square of the output,
scale invariance, equivariance under Wigner-D rotations, the gain acting
per degree, one statistic shared across degrees, and the zero input.
"""

import numpy as np


def merged_rms_norm_ref(x, gamma, eps=1e-5):
    """x: [n][(L+1)^2][C]; gamma: [L+1][C]; returns y, same shape, fp64."""
    x = np.asarray(x, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    n, nc, C = x.shape
    L = int(round(np.sqrt(nc))) - 1
    if (L + 1) ** 2 != nc or gamma.shape != (L + 1, C):
        raise ValueError("x must be [n][(L+1)^2][C] and gamma [L+1][C]")
    s = np.mean(x * x, axis=(1, 2))  # one statistic per node, over every degree
    inv = 1.0 / np.sqrt(s + eps)
    g = np.concatenate([np.repeat(gamma[l][None, :], 2 * l + 1, axis=0) for l in range(L + 1)], axis=0)
    return x * inv[:, None, None] * g[None, :, :]
