"""Pins of the merged RMS layer norm oracle ("EquiformerV3" technical
summary, section 2.B.1: one RMS statistic shared by all degrees).

Each check fixes the result by something other than the oracle's own
formula: the output's mean square, scale invariance, rotation
equivariance through independently computed Wigner-D blocks, the gain's
indexing by degree, the sharing of the statistic across degrees, and the
zero input."""

import numpy as np
import pytest
from scipy.spatial.transform import Rotation

from oracle import merged_rms_norm_ref, wigner_d_blocks


def _inputs(n=5, L=3, C=6, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, (L + 1) ** 2, C)) * rng.uniform(0.1, 10.0, size=(n, 1, 1))
    gamma = rng.uniform(0.5, 2.0, size=(L + 1, C))
    return x, gamma


def test_unit_mean_square_with_unit_gain():
    x, _ = _inputs()
    y = merged_rms_norm_ref(x, np.ones((4, 6)), eps=0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=(1, 2)), 1.0, rtol=1e-13)


def test_scale_invariance():
    x, g = _inputs()
    a = merged_rms_norm_ref(x, g, eps=0.0)
    b = merged_rms_norm_ref(37.5 * x, g, eps=0.0)
    np.testing.assert_allclose(a, b, rtol=1e-12)


@pytest.mark.parametrize("L", [1, 4, 6])
def test_rotation_equivariance(L):
    x, g = _inputs(n=3, L=L, C=4, seed=L)
    R = Rotation.random(random_state=5 + L).as_matrix()
    D = wigner_d_blocks(L, R)

    def rot(f):
        out = np.empty_like(f)
        for l in range(L + 1):
            sl = slice(l * l, (l + 1) ** 2)
            out[:, sl, :] = np.einsum("ab,nbc->nac", D[l], f[:, sl, :])
        return out

    np.testing.assert_allclose(merged_rms_norm_ref(rot(x), g), rot(merged_rms_norm_ref(x, g)), atol=1e-12)


def test_gain_acts_per_degree_and_channel():
    # gamma[l][c] scales exactly the 2l + 1 components of degree l in channel c
    x, _ = _inputs(n=2, L=3, C=5)
    base = merged_rms_norm_ref(x, np.ones((4, 5)), eps=1e-6)
    for l in range(4):
        for c in (0, 3):
            g = np.ones((4, 5))
            g[l, c] = 3.0
            y = merged_rms_norm_ref(x, g, eps=1e-6)
            ratio = np.ones_like(base)
            ratio[:, l * l : (l + 1) ** 2, c] = 3.0
            np.testing.assert_allclose(y, base * ratio, rtol=1e-13)


def test_one_statistic_shared_by_all_degrees():
    # changing only degree 3 changes the output of degree 0 (a per-degree
    # norm would leave it alone), by the ratio of the two node RMS values
    x, g = _inputs(n=1, L=3, C=4, seed=2)
    x2 = x.copy()
    x2[:, 9:16, :] *= 4.0
    y, y2 = merged_rms_norm_ref(x, g, eps=0.0), merged_rms_norm_ref(x2, g, eps=0.0)
    r1 = np.sqrt(np.sum(x * x) / x.size)
    r2 = np.sqrt(np.sum(x2 * x2) / x2.size)
    np.testing.assert_allclose(y2[:, 0:9, :], y[:, 0:9, :] * r1 / r2, rtol=1e-13)


def test_zero_node_stays_zero():
    x = np.zeros((2, 9, 3))
    x[1, 4, 2] = 2.0
    y = merged_rms_norm_ref(x, np.ones((3, 3)), eps=1e-5)
    assert np.all(y[0] == 0.0) and np.all(np.isfinite(y))
    # a single nonzero entry v among N entries: y = v / sqrt(v^2 / N + eps)
    np.testing.assert_allclose(y[1, 4, 2], 2.0 / np.sqrt(4.0 / 27 + 1e-5), rtol=1e-14)
