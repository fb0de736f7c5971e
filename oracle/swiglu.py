"""SwiGLU-S2 activation of node features, fp64 (test infrastructure only).

"EquiformerV3: Scaling Efficient, Expressive, and General SE(3)-Equivariant
Graph Attention Transformers", technical summary, section 2.C (SwiGLU-S2
activation) and key contribution 2: the irreps features are projected to a
grid on the sphere S2; instead of a pointwise nonlinearity on the grid (which
needs dense sampling and breaks strict equivariance), the nonlinear gate acts
on the scalar features only and the grid features are multiplied
bilinearly, which amounts to a tensor product of the features with
themselves (many-body terms).  "DPA4 ...", technical summary, section 2.1
(the FFN uses a spherical-grid SwiGLU; the projection keeps SO(3)
equivariance to machine precision when the quadrature is exact).

Reading (the pages print no formula).  For node features x[(l, m), c],
l = 0..L, with per-degree channel maps A_l, B_l, O_l (C x C, [in][out], the
same matrix for the 2l + 1 components of a degree) and a scalar map G:

    u[(l, m)] = x[(l, m)] A_l,    v[(l, m)] = x[(l, m)] B_l      (row vectors)
    g         = x[(0, 0)] G
    u(r), v(r) = sum_(l, m) u[(l, m)] Y_lm(r)   at the grid points r_p
    h[(l, m)] = sum_p w_p Y_lm(r_p) u(r_p) v(r_p)      for l = 0..L
    s[(l, m)] = SiLU(g) * h[(l, m)]                    (per channel)
    y[(l, m)] = s[(l, m)] O_l

SiLU(z) = z / (1 + exp(-z)).  The grid is a product grid: Gauss-Legendre
nodes in cos(theta) (n_theta = ceil((3L + 1) / 2)) times n_phi = 3L + 1
equally spaced phi, weights w = w_GL * 2 pi / n_phi.  u v has degree <= 2L,
so its projection onto degree <= L integrates polynomials of degree <= 3L,
which this grid does exactly: the map is then exactly equivariant.

Parity pinned by tests/test_oracle_swiglu.py: the grid integrates products of
harmonics exactly up to degree 3L; the hand-worked product Y_10 * Y_10 =
Y_00 / sqrt(4 pi) + Y_20 / sqrt(5 pi); the L = 0 closed form; equivariance
under Wigner-D rotations (and its failure on a grid one node short).
"""

import numpy as np

from .sh import n_comp, real_sh


def s2_grid(l_max: int, n_theta=None, n_phi=None):
    """Directions [P, 3] and weights [P] of the product grid (see module)."""
    nt = (3 * l_max + 2) // 2 if n_theta is None else n_theta
    npf = 3 * l_max + 1 if n_phi is None else n_phi
    ct, wt = np.polynomial.legendre.leggauss(max(nt, 1))
    st = np.sqrt(1.0 - ct * ct)
    ph = 2.0 * np.pi * np.arange(npf) / npf
    dirs = np.stack(
        [np.outer(st, np.cos(ph)).ravel(), np.outer(st, np.sin(ph)).ravel(), np.repeat(ct, npf)], axis=1
    )
    w = np.repeat(wt, npf) * (2.0 * np.pi / npf)
    return dirs, w


def _per_degree(x, W, L):
    """y[:, (l, m), :] = x[:, (l, m), :] @ W[l] for every degree l."""
    out = np.empty(x.shape[:2] + (W.shape[2],), dtype=np.float64)
    for l in range(L + 1):
        sl = slice(l * l, (l + 1) * (l + 1))
        out[:, sl, :] = x[:, sl, :] @ W[l]
    return out


def silu(z):
    return z / (1.0 + np.exp(-z))


def swiglu_s2_ref(x, w_a, w_b, w_g, w_o, grid=None):
    """x: [n][(L+1)^2][C]; w_a, w_b, w_o: [L+1][C][C]; w_g: [C][C].
    Returns y [n][(L+1)^2][C] in fp64.  `grid` = (dirs, weights) replaces the
    product grid (the tests use it to show that a coarser grid breaks
    equivariance)."""
    x = np.asarray(x, dtype=np.float64)
    n, nc, C = x.shape
    L = int(round(np.sqrt(nc))) - 1
    if n_comp(L) != nc:
        raise ValueError("x must be [n][(L+1)^2][C]")
    w_a, w_b, w_o = (np.asarray(w, dtype=np.float64) for w in (w_a, w_b, w_o))
    w_g = np.asarray(w_g, dtype=np.float64)
    for w in (w_a, w_b, w_o):
        if w.shape != (L + 1, C, C):
            raise ValueError("per-degree weights must be [L+1][C][C]")
    if w_g.shape != (C, C):
        raise ValueError("w_g must be [C][C]")
    dirs, wq = s2_grid(L) if grid is None else grid
    Y = real_sh(L, dirs)  # [P][nc]
    u = _per_degree(x, w_a, L)
    v = _per_degree(x, w_b, L)
    g = x[:, 0, :] @ w_g
    ug = np.einsum("pk,nkc->npc", Y, u)
    vg = np.einsum("pk,nkc->npc", Y, v)
    h = np.einsum("p,pk,npc->nkc", wq, Y, ug * vg)
    s = silu(g)[:, None, :] * h
    return _per_degree(s, w_o, L)
