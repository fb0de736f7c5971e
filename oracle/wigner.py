"""Wigner-D blocks for real spherical harmonics and the edge frame, fp64.
Test infrastructure (see oracle/__init__).

E2Former-V2 summary, technical section 2.1 (EAAS): each edge is handled in
the frame whose axis is the edge vector.  Here that is a proper rotation R
with R r_hat = z_hat, and D^l(R) is the matrix with

    Y_l(R s) = D^l(R) Y_l(s)     for every unit vector s.

D^l is the projection of s -> Y_l(R s) onto Y_l:
D^l_{ab} = integral over the sphere of Y_{l,a}(R s) Y_{l,b}(s).  The
integrand is a polynomial of degree 2l on the sphere, so a product rule with
Gauss-Legendre nodes in cos(theta) (n >= l+1 nodes, exact to degree 2n-1)
times n_phi >= 2l+1 equally spaced azimuths (exact for trigonometric degree
< n_phi) integrates it exactly; the result is D^l up to rounding.
"""

from functools import lru_cache

import numpy as np
from numpy.polynomial import legendre as npleg

from .sh import real_sh


@lru_cache(maxsize=None)
def _product_quadrature(l_max: int):
    """Nodes s_q [Q, 3] and weights w_q [Q] exact for degree <= 2 l_max."""
    n_t = l_max + 1
    n_p = 2 * l_max + 1
    ct, wt = npleg.leggauss(n_t)
    ph = 2.0 * np.pi * np.arange(n_p) / n_p
    st = np.sqrt(1.0 - ct * ct)
    nodes = np.stack(
        [
            np.outer(st, np.cos(ph)).ravel(),
            np.outer(st, np.sin(ph)).ravel(),
            np.repeat(ct, n_p),
        ],
        axis=1,
    )
    weights = np.repeat(wt, n_p) * (2.0 * np.pi / n_p)
    nodes.flags.writeable = False
    weights.flags.writeable = False
    return nodes, weights


@lru_cache(maxsize=None)
def _sh_at_nodes(l_max: int):
    """Y(s_q) at the quadrature nodes: the same for every rotation, so it is
    evaluated once per l_max (read-only)."""
    y = real_sh(l_max, _product_quadrature(l_max)[0])
    y.flags.writeable = False
    return y


def wigner_d_blocks(l_max: int, R) -> list:
    """[D^0(R), ..., D^L(R)], each (2l+1) x (2l+1), rows/cols m = -l..l.

    R may also be a stack [E, 3, 3] of rotations; then every block is
    [E, 2l+1, 2l+1], entry e belonging to R[e]."""
    R = np.asarray(R, dtype=np.float64)
    single = R.ndim == 2
    rs = R.reshape(-1, 3, 3)
    nodes, w = _product_quadrature(l_max)
    y_s = _sh_at_nodes(l_max)  # Y(s_q)
    pts = np.einsum("eij,qj->eqi", rs, nodes)  # R s_q for every rotation
    y_rs = real_sh(l_max, pts.reshape(-1, 3)).reshape(rs.shape[0], nodes.shape[0], -1)  # Y(R s_q)
    blocks = []
    for l in range(l_max + 1):
        sl = slice(l * l, (l + 1) * (l + 1))
        b = np.einsum("eqa,q,qb->eab", y_rs[:, :, sl], w, y_s[:, sl])
        blocks.append(b[0] if single else b)
    return blocks


def rot_z(gamma: float) -> np.ndarray:
    """Rotation by gamma about z (counter-clockwise seen from +z)."""
    c, s = np.cos(gamma), np.sin(gamma)
    return np.array([[c, -s, 0.0], [s, c, 0.0], [0.0, 0.0, 1.0]])


def frame_rotation(rhat) -> np.ndarray:
    """A proper rotation R with R rhat = z_hat (Rodrigues about rhat x z_hat).

    rhat = +z gives the identity, rhat = -z the half turn about x.  Any
    other choice differs by a rotation about z after R (a gauge); the layer
    output does not depend on it (tested)."""
    r = np.asarray(rhat, dtype=np.float64)
    r = r / np.sqrt(np.sum(r * r))
    z = np.array([0.0, 0.0, 1.0])
    axis = np.cross(r, z)
    s = np.sqrt(np.sum(axis * axis))
    c = float(r @ z)
    if s == 0.0:
        return np.eye(3) if c > 0.0 else np.diag([1.0, -1.0, -1.0])
    k = axis / s
    kx = np.array([[0.0, -k[2], k[1]], [k[2], 0.0, -k[0]], [-k[1], k[0], 0.0]])
    ang = np.arctan2(s, c)
    return np.eye(3) + np.sin(ang) * kx + (1.0 - np.cos(ang)) * (kx @ kx)
