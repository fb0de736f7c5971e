"""Pins of the SwiGLU-S2 oracle (CPU): the grid's exactness, a hand-worked
harmonic product, the L = 0 closed form and equivariance."""

import numpy as np
import pytest

from oracle import real_sh, wigner_d_blocks
from oracle.swiglu import s2_grid, silu, swiglu_s2_ref


@pytest.mark.parametrize("L", [0, 1, 2, 4, 6])
def test_grid_integrates_harmonic_products_exactly(L):
    """Orthonormality of Y_lm up to degree floor(3L/2) on the grid: the
    integrands reach degree 3L, the grid's design degree; plus the area 4 pi."""
    dirs, w = s2_grid(L)
    assert np.isclose(w.sum(), 4.0 * np.pi, rtol=0, atol=1e-12)
    lq = (3 * L) // 2
    Y = real_sh(lq, dirs)
    G = (Y * w[:, None]).T @ Y
    assert np.abs(G - np.eye(G.shape[0])).max() < 1e-12


def _unit(L, C):
    return np.stack([np.eye(C)] * (L + 1))


def test_y10_squared_by_hand():
    """x holds Y_10 in channel 0 and the scalar z0 in channel 1; A = B = O = 1
    on l >= 1 and 0 on l = 0, G maps channel 1 to the gate of channel 0.
    Then u = v = Y_10 and Y_10^2 = (3 / 4 pi) cos^2 = Y_00 / sqrt(4 pi) +
    Y_20 / sqrt(5 pi), so y_00 = SiLU(z0) / sqrt(4 pi), y_20 = SiLU(z0) /
    sqrt(5 pi) in channel 0 and every other entry is 0."""
    L, C, z0 = 2, 2, 0.7
    x = np.zeros((1, 9, C))
    x[0, 2, 0] = 1.0  # (l, m) = (1, 0)
    x[0, 0, 1] = z0
    A = _unit(L, C)
    A[0] = 0.0
    G = np.zeros((C, C))
    G[1, 0] = 1.0
    y = swiglu_s2_ref(x, A, A.copy(), G, _unit(L, C))
    want = np.zeros((1, 9, C))
    want[0, 0, 0] = silu(z0) / np.sqrt(4 * np.pi)
    want[0, 6, 0] = silu(z0) / np.sqrt(5 * np.pi)  # (2, 0)
    assert np.abs(y - want).max() < 1e-14


def test_l0_closed_form():
    """L = 0: Y_00 = 1 / sqrt(4 pi) everywhere, so h = u v / sqrt(4 pi) and
    y = (SiLU(x G) * (x A)(x B) / sqrt(4 pi)) O."""
    rng = np.random.default_rng(0)
    C = 5
    x = rng.standard_normal((7, 1, C))
    A, B, O = (rng.standard_normal((1, C, C)) for _ in range(3))
    G = rng.standard_normal((C, C))
    y = swiglu_s2_ref(x, A, B, G, O)
    x0 = x[:, 0, :]
    want = (silu(x0 @ G) * (x0 @ A[0]) * (x0 @ B[0]) / np.sqrt(4 * np.pi)) @ O[0]
    assert np.abs(y[:, 0, :] - want).max() < 1e-12


def _rotate(x, blocks):
    out = np.empty_like(x)
    for l, D in enumerate(blocks):
        sl = slice(l * l, (l + 1) * (l + 1))
        out[:, sl, :] = np.einsum("ij,njc->nic", D, x[:, sl, :])
    return out


def _random_rotation(rng):
    q = rng.standard_normal(4)
    q /= np.linalg.norm(q)
    a, b, c, d = q
    return np.array(
        [
            [a * a + b * b - c * c - d * d, 2 * (b * c - a * d), 2 * (b * d + a * c)],
            [2 * (b * c + a * d), a * a - b * b + c * c - d * d, 2 * (c * d - a * b)],
            [2 * (b * d - a * c), 2 * (c * d + a * b), a * a - b * b - c * c + d * d],
        ]
    )


@pytest.mark.parametrize("L", [1, 2, 4, 6])
def test_equivariance(L):
    rng = np.random.default_rng(L)
    C = 4
    x = rng.standard_normal((3, (L + 1) ** 2, C))
    A, B, O = (rng.standard_normal((L + 1, C, C)) for _ in range(3))
    G = rng.standard_normal((C, C))
    blocks = wigner_d_blocks(L, _random_rotation(rng))
    y = swiglu_s2_ref(x, A, B, G, O)
    y_rot = swiglu_s2_ref(_rotate(x, blocks), A, B, G, O)
    assert np.abs(y_rot - _rotate(y, blocks)).max() < 1e-10 * max(1.0, np.abs(y).max())


def test_grid_one_node_short_is_not_equivariant():
    """The same check on a grid with one Gauss-Legendre node fewer fails: the
    equivariance test sees the grid size."""
    L, C = 4, 4
    rng = np.random.default_rng(9)
    x = rng.standard_normal((2, 25, C))
    A, B, O = (rng.standard_normal((L + 1, C, C)) for _ in range(3))
    G = rng.standard_normal((C, C))
    short = s2_grid(L, n_theta=(3 * L + 2) // 2 - 1)
    blocks = wigner_d_blocks(L, _random_rotation(rng))
    y = swiglu_s2_ref(x, A, B, G, O, grid=short)
    y_rot = swiglu_s2_ref(_rotate(x, blocks), A, B, G, O, grid=short)
    assert np.abs(y_rot - _rotate(y, blocks)).max() > 1e-6 * np.abs(y).max()


def test_silu_values_and_identities():
    # SiLU(z) = z / (1 + e^-z) (the gate of SwiGLU); literal values of the
    # logistic function at 1 and 2 (1 / (1 + e^-1) = 0.731058578630004879...,
    # 2 / (1 + e^-2) = 1.761594155955764888...)
    assert silu(0.0) == 0.0
    assert silu(1.0) == pytest.approx(0.7310585786300049, rel=1e-15)
    assert silu(-1.0) == pytest.approx(-0.2689414213699951, rel=1e-14)
    assert silu(2.0) == pytest.approx(1.7615941559557649, rel=1e-15)
    z = np.linspace(-30.0, 30.0, 241)
    # silu(z) - silu(-z) = z (sigma(z) + sigma(-z) = 1); a plain sigmoid or
    # z sigma(-z) fails this
    np.testing.assert_allclose(silu(z) - silu(-z), z, atol=1e-12)
    # silu -> z for large z, -> 0 from below for very negative z, minimum
    # near z = -1.2785 with value -0.2784645...
    assert silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert -1e-15 < silu(-40.0) < 0.0
    zz = np.linspace(-2.0, -0.5, 300001)
    assert float(silu(zz).min()) == pytest.approx(-0.27846454276107, abs=1e-10)
    # slope 1/2 at the origin
    h = 1e-6
    assert (silu(h) - silu(-h)) / (2 * h) == pytest.approx(0.5, rel=1e-9)
