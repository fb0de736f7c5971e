"""Pins for the oracle's real spherical harmonics, Wigner-D blocks and edge
frame.  Each check is fixed by mathematics, not by the oracle itself:
textbook closed forms, orthonormality under an independent quadrature, the
addition theorem, the defining property Y(Rs) = D Y(s) at random points,
group structure, and the aligned-frame sparsity the E2Former-V2 summary
states (technical section 2.1, Lemma 4.1: on the edge axis only m = 0 is
non-zero)."""

from math import pi, sqrt

import numpy as np
import pytest
from scipy.special import eval_legendre, roots_legendre
from scipy.spatial.transform import Rotation

from oracle import frame_rotation, real_sh, rot_z, wigner_d_blocks


def _rand_unit(rng, n):
    v = rng.standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1)[:, None]


def _rand_rot(rng):
    return Rotation.random(random_state=int(rng.integers(1 << 31))).as_matrix()


def test_sh_textbook_closed_forms():
    rng = np.random.default_rng(0)
    v = _rand_unit(rng, 50)
    x, y, z = v.T
    Y = real_sh(3, v)
    expect = {
        0: np.full_like(x, 0.5 / sqrt(pi)),
        1: sqrt(3 / (4 * pi)) * y,
        2: sqrt(3 / (4 * pi)) * z,
        3: sqrt(3 / (4 * pi)) * x,
        4: 0.5 * sqrt(15 / pi) * x * y,
        5: 0.5 * sqrt(15 / pi) * y * z,
        6: 0.25 * sqrt(5 / pi) * (3 * z * z - 1),
        7: 0.5 * sqrt(15 / pi) * x * z,
        8: 0.25 * sqrt(15 / pi) * (x * x - y * y),
        9: 0.25 * sqrt(35 / (2 * pi)) * y * (3 * x * x - y * y),
        12: 0.25 * sqrt(7 / pi) * (5 * z**3 - 3 * z),
        15: 0.25 * sqrt(35 / (2 * pi)) * x * (x * x - 3 * y * y),
    }
    for idx, ref in expect.items():
        np.testing.assert_allclose(Y[:, idx], ref, atol=1e-14, err_msg=f"component {idx}")


def test_sh_orthonormal_independent_quadrature():
    L = 6
    n_t, n_p = 2 * L + 4, 4 * L + 5  # finer than, and different from, the oracle's rule
    ct, wt = roots_legendre(n_t)
    ph = 2 * pi * (np.arange(n_p) + 0.37) / n_p
    st = np.sqrt(1 - ct * ct)
    pts = np.stack(
        [np.outer(st, np.cos(ph)).ravel(), np.outer(st, np.sin(ph)).ravel(), np.repeat(ct, n_p)], 1
    )
    w = np.repeat(wt, n_p) * (2 * pi / n_p)
    Y = real_sh(L, pts)
    gram = (Y * w[:, None]).T @ Y
    np.testing.assert_allclose(gram, np.eye((L + 1) ** 2), atol=1e-13)


def test_sh_addition_theorem():
    rng = np.random.default_rng(1)
    a, b = _rand_unit(rng, 20), _rand_unit(rng, 20)
    L = 6
    Ya, Yb = real_sh(L, a), real_sh(L, b)
    cosg = np.sum(a * b, axis=1)
    for l in range(L + 1):
        sl = slice(l * l, (l + 1) ** 2)
        lhs = np.sum(Ya[:, sl] * Yb[:, sl], axis=1)
        rhs = (2 * l + 1) / (4 * pi) * eval_legendre(l, cosg)
        np.testing.assert_allclose(lhs, rhs, atol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_wigner_defining_property_at_random_points(seed):
    rng = np.random.default_rng(10 + seed)
    R = _rand_rot(rng)
    L = 6
    D = wigner_d_blocks(L, R)
    s = _rand_unit(rng, 40)
    Ys, Yrs = real_sh(L, s), real_sh(L, s @ R.T)
    for l in range(L + 1):
        sl = slice(l * l, (l + 1) ** 2)
        np.testing.assert_allclose(Yrs[:, sl], Ys[:, sl] @ D[l].T, atol=1e-13)


def test_wigner_orthogonal_and_homomorphism():
    rng = np.random.default_rng(2)
    A, B = _rand_rot(rng), _rand_rot(rng)
    L = 6
    DA, DB, DAB = wigner_d_blocks(L, A), wigner_d_blocks(L, B), wigner_d_blocks(L, A @ B)
    for l in range(L + 1):
        np.testing.assert_allclose(DA[l] @ DA[l].T, np.eye(2 * l + 1), atol=1e-13)
        np.testing.assert_allclose(DAB[l], DA[l] @ DB[l], atol=1e-13)
        assert abs(np.linalg.det(DA[l]) - 1.0) < 1e-12


def test_wigner_l1_is_the_rotation_in_yzx_order():
    rng = np.random.default_rng(3)
    R = _rand_rot(rng)
    P = np.array([[0, 1, 0], [0, 0, 1], [1, 0, 0]], dtype=float)  # (x,y,z) -> (y,z,x)
    np.testing.assert_allclose(wigner_d_blocks(1, R)[1], P @ R @ P.T, atol=1e-14)
    np.testing.assert_allclose(wigner_d_blocks(0, R)[0], [[1.0]], atol=1e-14)


def test_wigner_z_rotation_is_2x2_blocks():
    gamma = 0.7321
    L = 5
    D = wigner_d_blocks(L, rot_z(gamma))
    for l in range(L + 1):
        ref = np.zeros((2 * l + 1, 2 * l + 1))
        ref[l, l] = 1.0
        for m in range(1, l + 1):
            c, s = np.cos(m * gamma), np.sin(m * gamma)
            p, n = l + m, l - m
            ref[p, p], ref[p, n], ref[n, p], ref[n, n] = c, -s, s, c
        np.testing.assert_allclose(D[l], ref, atol=1e-13)


@pytest.mark.parametrize(
    "rhat",
    [
        None,
        (0.0, 0.0, 1.0),
        (0.0, 0.0, -1.0),
        (1e-9, 0.0, -1.0),
        (1.0, 0.0, 0.0),
        (0.3, -0.4, 0.5),
    ],
)
def test_edge_frame_maps_edge_to_z_and_only_m0_survives(rhat):
    rng = np.random.default_rng(4)
    r = _rand_unit(rng, 1)[0] if rhat is None else np.asarray(rhat, dtype=float)
    r = r / np.linalg.norm(r)
    R = frame_rotation(r)
    np.testing.assert_allclose(R @ R.T, np.eye(3), atol=1e-14)
    assert abs(np.linalg.det(R) - 1.0) < 1e-13
    np.testing.assert_allclose(R @ r, [0.0, 0.0, 1.0], atol=1e-14)
    L = 6
    D = wigner_d_blocks(L, R)
    Y = real_sh(L, r[None, :])[0]
    for l in range(L + 1):
        sl = slice(l * l, (l + 1) ** 2)
        e0 = np.zeros(2 * l + 1)
        e0[l] = sqrt((2 * l + 1) / (4 * pi))
        np.testing.assert_allclose(D[l] @ Y[sl], e0, atol=1e-13)
