"""Pins for the oracle's attention layer.

No page prints an output value, so the layer is pinned by what the pages and
mathematics fix:
* hand-worked fixtures (tests/golden): a two-atom L = 1 case through the
  rotation, the per-m map and the rotation back (E2Former-V2 summary,
  technical section 2.1), and an L = 0 case for the envelope-gated softmax
  (EquiformerV3 summary, technical section 2.B.3);
* SO(3) equivariance, translation invariance, permutation equivariance,
  periodic-image invariance and gauge (frame roll) invariance;
* envelope boundary conditions and radial basis centres;
* special cases that reduce to independent formulas: L = 0 scalar attention
  via scipy's softmax, identity SO(2) weights (rotations cancel exactly),
  softmax weights summing to one, empty neighbourhoods;
* planted mistakes in the oracle must break at least one pin.
"""

import json
import os
from fractions import Fraction
from math import comb, exp

import numpy as np
import pytest
from scipy.spatial.transform import Rotation
from scipy.special import softmax

import oracle
import oracle.attention as oatt
from oracle import (
    envelope,
    neighbors_bruteforce,
    radial_gaussians,
    so2_attention_ref,
    so2_weight_count,
    unpack_so2,
    wigner_d_blocks,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _system(seed, n=12, side=6.0, rc=4.0, L=2, C=4, H=2, K=4, box=None):
    """Small random system whose pair distances stay away from the cutoff,
    so rotating it cannot change the fp32 neighbour test."""
    rng = np.random.default_rng(seed)
    while True:
        pos = rng.uniform(0.0, side, size=(n, 3))
        d = pos[:, None, :] - pos[None, :, :]
        if box is not None:
            d -= box * np.rint(d / box)
        r = np.sqrt((d * d).sum(-1))
        np.fill_diagonal(r, 1.0)
        if np.all(np.abs(r - rc) > 1e-3) and r.min() > 0.5:
            break
    nc = (L + 1) ** 2
    x = rng.standard_normal((n, nc, C))
    w_q = rng.standard_normal((C, C)) / np.sqrt(C)
    w_k = rng.standard_normal((C, C)) / np.sqrt(C)
    w_rad = rng.standard_normal((K, C)) / np.sqrt(K)
    w_so2 = rng.standard_normal(so2_weight_count(L, C)) / np.sqrt(C * (L + 1))
    return dict(pos=pos, x=x, w_q=w_q, w_k=w_k, w_rad=w_rad, w_so2=w_so2, L=L, H=H, rc=rc, box=box)


def _run(s, pos=None, x=None, **kw):
    pos = s["pos"] if pos is None else pos
    x = s["x"] if x is None else x
    box = s["box"]
    rp, col = neighbors_bruteforce(pos.astype(np.float32), s["rc"], box)
    return so2_attention_ref(
        pos, rp, col, x, s["w_q"], s["w_k"], s["w_rad"], s["w_so2"],
        l_max=s["L"], heads=s["H"], cutoff=s["rc"], box=box, **kw,
    )


def _rotate_features(x, R, L):
    D = wigner_d_blocks(L, R)
    out = np.empty_like(x)
    for l in range(L + 1):
        sl = slice(l * l, (l + 1) ** 2)
        out[:, sl, :] = np.einsum("ab,nbc->nac", D[l], x[:, sl, :])
    return out


# ---------------------------------------------------------------- fixtures


def test_golden_two_atoms_l1_hand_worked():
    g = _load("two_atoms_l1.json")
    pos = np.array(g["positions"], dtype=np.float32)
    rp, col = neighbors_bruteforce(pos, g["cutoff"])
    y = so2_attention_ref(
        pos, rp, col, np.array(g["x"]), np.array(g["w_q"]), np.array(g["w_k"]),
        np.array(g["w_rad"]), np.array(g["w_so2"]), l_max=g["l_max"], heads=g["heads"],
        cutoff=g["cutoff"], envelope_p=g["envelope_p"], flags=g["flags"],
    )
    np.testing.assert_allclose(y, np.array(g["expected_y"]), atol=1e-12)


def test_golden_three_atoms_envelope_softmax_l0():
    g = _load("three_atoms_softmax_l0.json")
    pos = np.array(g["positions"], dtype=np.float32)
    rp, col = neighbors_bruteforce(pos, g["cutoff"])
    assert list(col[rp[0] : rp[1]]) == [1, 2]
    y = so2_attention_ref(
        pos, rp, col, np.array(g["x"]), np.eye(1), np.eye(1), np.ones((2, 1)),
        np.array(g["w_so2"]), l_max=0, heads=1, cutoff=g["cutoff"], flags=oatt.FLAG_NO_RADIAL,
    )
    u1, u2 = g["u_target0"]
    z1, z2 = g["z_target0"]
    a1 = u1 * exp(z1) / (u1 * exp(z1) + u2 * exp(z2))
    a2 = 1.0 - a1
    assert abs(y[0, 0, 0] - 2.0 * (a1 * 0.5 + a2 * (-1.0))) < 1e-12
    np.testing.assert_allclose(envelope(np.array([0.2, 0.5]), 5), [u1, u2], atol=1e-15)


# ---------------------------------------------------------------- pieces


@pytest.mark.parametrize("p", [3, 5, 6, 8])
def test_envelope_boundary_conditions(p):
    assert envelope(0.0, p) == 1.0
    s = np.linspace(0.5, 0.999, 40)
    poly = np.polynomial.Polynomial.fit(s, envelope(s, p), p + 2).convert()
    for order in range(3):
        assert abs(poly.deriv(order)(1.0)) < 1e-7, (p, order)
    assert envelope(1.0, p) == 0.0 and envelope(1.3, p) == 0.0
    assert np.all(np.diff(envelope(np.linspace(0, 1, 200), p)) <= 1e-15)


def test_envelope_p5_published_form():
    s = np.linspace(0, 0.99, 17)
    np.testing.assert_allclose(envelope(s, 5), 1 - 21 * s**5 + 35 * s**6 - 15 * s**7, atol=1e-14)


def _envelope_exact(s, p):
    """The expanded polynomial 1 - (p+1)(p+2)/2 s^p + p(p+2) s^(p+1) -
    p(p+1)/2 s^(p+2) in exact rational arithmetic at the double s."""
    q = Fraction(s)
    return 1 - Fraction((p + 1) * (p + 2), 2) * q**p + p * (p + 2) * q ** (p + 1) - Fraction(p * (p + 1), 2) * q ** (p + 2)


@pytest.mark.parametrize("p", [3, 5, 6, 8])
def test_envelope_relative_precision_up_to_the_cutoff(p):
    # the oracle against the exact value of the same polynomial, relatively,
    # from the middle of the range to within 1e-12 of the cutoff: the
    # expanded form in fp64 is pure rounding noise there (a wrong cofactor or
    # a dropped term fails at every point)
    pts = [0.05, 0.3, 0.5, 0.9, 0.99, 1 - 1e-3, 1 - 1e-5, 1 - 1e-8, 1 - 1e-10, 1 - 1e-12]
    for s in pts:
        exact = _envelope_exact(s, p)
        assert exact > 0
        got = Fraction(float(envelope(s, p)))
        assert abs(got - exact) <= Fraction(1, 10**13) * exact, (p, s, float(got), float(exact))


@pytest.mark.parametrize("p", [3, 5, 6, 8])
def test_envelope_positive_inside_and_triple_root_at_the_cutoff(p):
    s = np.concatenate([np.linspace(0.0, 1.0, 2001)[:-1], 1.0 - np.logspace(-15, -1, 57)])
    u = envelope(s, p)
    assert np.all(u > 0.0)
    # u ~ C(p+2, 3) (1 - s)^3 as s -> 1: the cofactor at s = 1 is the sum of
    # the first p triangular numbers (the tetrahedral number)
    t = 1e-9
    assert abs(float(envelope(1.0 - t, p)) / t**3 - comb(p + 2, 3)) < 1e-6 * comb(p + 2, 3)


def test_envelope_p5_factored_cofactor():
    # at p = 5: u = (1 - s)^3 (1 + 3 s + 6 s^2 + 10 s^3 + 15 s^4), checked
    # against the printed polynomial on exact rationals
    for s in (0.1, 0.37, 0.8, 0.999):
        q = Fraction(s)
        assert (1 - q) ** 3 * (1 + 3 * q + 6 * q**2 + 10 * q**3 + 15 * q**4) == _envelope_exact(s, 5)


def test_radial_basis_centres_and_width():
    rc, K = 5.0, 8
    sigma = rc / (K - 1)
    for k in (0, 3, K - 1):
        mu = k * rc / (K - 1)
        assert abs(radial_gaussians(mu, rc, K)[k] - 1.0) < 1e-15
        np.testing.assert_allclose(radial_gaussians(mu + sigma, rc, K)[k], exp(-0.5), rtol=1e-14)


@pytest.mark.parametrize("L", [0, 1, 2, 4, 6])
def test_weight_count_closed_form(L):
    C = 3
    assert so2_weight_count(L, C) == C * C * ((L + 1) ** 2 + L * (L + 1) * (2 * L + 1) // 3)
    w0, w1, w2 = unpack_so2(np.arange(so2_weight_count(L, C)), L, C)
    assert w0.shape == ((L + 1) * C,) * 2
    assert all(w1[m].shape == ((L + 1 - m) * C,) * 2 for m in w1)


# ---------------------------------------------------------------- the parity metric


def test_max_rel_error_normalises_per_atom():
    # atom 0 has entries of order 1, atom 1 of order 1e-3; an error of 1e-4
    # on atom 1 is 10 % of that atom's scale (a global normaliser would
    # report 1e-4)
    ref = np.array([[[1.0, -0.5], [0.25, 0.0]], [[1e-3, 0.0], [-5e-4, 2e-4]]])
    test = ref.copy()
    test[1, 0, 0] += 1e-4
    assert oracle.max_rel_error(test, ref) == pytest.approx(0.1, rel=1e-12)
    # the same absolute error on atom 0 is 1e-4 of its scale
    test = ref.copy()
    test[0, 1, 1] -= 1e-4
    assert oracle.max_rel_error(test, ref) == pytest.approx(1e-4, rel=1e-9)


def test_max_rel_error_groups_by_the_first_axis():
    # [T, (L+1)^2, C] with T = 3: errors are grouped per target row, whatever
    # the trailing shape; a reshape over the wrong axis would mix the scales
    ref = np.zeros((3, 4, 2))
    ref[0] = 100.0
    ref[1] = 1.0
    ref[2, 3, 1] = -2.0
    test = ref.copy()
    test[1, 2, 0] += 0.5
    assert oracle.max_rel_error(test, ref) == pytest.approx(0.5, rel=1e-12)
    test[2, 0, 0] += 0.5
    assert oracle.max_rel_error(test, ref) == pytest.approx(0.5, rel=1e-12)
    test[2, 3, 1] -= 1.5
    assert oracle.max_rel_error(test, ref) == pytest.approx(0.75, rel=1e-12)
    assert oracle.max_rel_error(test.reshape(3, 8), ref.reshape(3, 8)) == pytest.approx(0.75, rel=1e-12)


def test_max_rel_error_floor_and_degenerate_cases():
    # an all-zero reference atom is measured against 1e-6 of the global scale
    ref = np.array([[[2.0, 0.0]], [[0.0, 0.0]]])
    test = ref.copy()
    test[1, 0, 1] = 3e-9
    assert oracle.max_rel_error(test, ref) == pytest.approx(3e-9 / 2e-6, rel=1e-12)
    # an all-zero reference: absolute error
    assert oracle.max_rel_error(np.full((2, 1, 1), 0.25), np.zeros((2, 1, 1))) == pytest.approx(0.25)
    assert oracle.max_rel_error(np.zeros((0, 4, 2)), np.zeros((0, 4, 2))) == 0.0
    assert oracle.max_rel_error(ref, ref) == 0.0
    # symmetric in the sign of the error
    assert oracle.max_rel_error(ref + 0.1, ref) == oracle.max_rel_error(ref - 0.1, ref)


# ---------------------------------------------------------------- symmetry


@pytest.mark.parametrize("seed", [0, 1])
def test_rotation_equivariance(seed):
    s = _system(seed, L=3, C=3, H=1)
    R = Rotation.random(random_state=seed + 7).as_matrix()
    center = s["pos"].mean(axis=0)
    pos_r = (s["pos"] - center) @ R.T + center
    y = _run(s)
    y_r = _run(s, pos=pos_r, x=_rotate_features(s["x"], R, s["L"]))
    np.testing.assert_allclose(y_r, _rotate_features(y, R, s["L"]), atol=1e-11)


def test_rotation_equivariance_periodic_cubic_symmetry():
    box = np.array([7.0, 7.0, 7.0])
    s = _system(3, n=14, side=7.0, rc=3.0, box=box)
    R = np.array([[0.0, -1.0, 0.0], [1.0, 0.0, 0.0], [0.0, 0.0, 1.0]])  # maps the cube to itself
    y = _run(s)
    y_r = _run(s, pos=s["pos"] @ R.T, x=_rotate_features(s["x"], R, s["L"]))
    np.testing.assert_allclose(y_r, _rotate_features(y, R, s["L"]), atol=1e-11)


def test_translation_invariance():
    s = _system(4)
    y = _run(s)
    np.testing.assert_allclose(_run(s, pos=s["pos"] + np.array([3.25, -1.5, 0.75])), y, atol=1e-11)


def test_periodic_image_shift_invariance():
    box = np.array([7.0, 7.0, 7.0])
    s = _system(5, n=14, side=7.0, rc=3.0, box=box)
    shift = np.zeros_like(s["pos"])
    shift[::3] = box * np.array([1.0, -2.0, 1.0])
    np.testing.assert_allclose(_run(s, pos=s["pos"] + shift), _run(s), atol=1e-11)


def test_permutation_equivariance():
    s = _system(6)
    perm = np.random.default_rng(0).permutation(s["pos"].shape[0])
    y = _run(s)
    y_p = _run(s, pos=s["pos"][perm], x=s["x"][perm])
    np.testing.assert_allclose(y_p, y[perm], atol=1e-12)


def test_gauge_invariance_frame_roll():
    s = _system(7, L=3, C=3, H=3)
    rng = np.random.default_rng(3)
    angles = {}

    def gauge(i, e):
        return angles.setdefault((i, e), rng.uniform(0, 2 * np.pi))

    np.testing.assert_allclose(_run(s, gauge=gauge), _run(s), atol=1e-12)


# ---------------------------------------------------------------- special cases


def test_softmax_weights_sum_to_one_per_head():
    s = _system(8, C=4, H=2)
    _, wts = _run(s, return_weights=True)
    for i, a in wts.items():
        np.testing.assert_allclose(a.sum(axis=0), 1.0, atol=1e-14)
        assert np.all(a > 0)


def test_l0_reduces_to_scalar_attention():
    s = _system(9, L=0, C=4, H=2)
    y = _run(s)
    rp, col = neighbors_bruteforce(s["pos"].astype(np.float32), s["rc"])
    C, H = 4, 2
    d = C // H
    x0 = s["x"][:, 0, :]
    q, k = x0 @ s["w_q"], x0 @ s["w_k"]
    W0 = s["w_so2"].reshape(C, C)
    for i in range(len(rp) - 1):
        js = col[rp[i] : rp[i + 1]]
        if js.size == 0:
            assert np.all(y[i] == 0)
            continue
        r = s["pos"][js] - s["pos"][i]
        rho = np.sqrt((r * r).sum(1))
        u = envelope(rho / s["rc"])
        g = radial_gaussians(rho[:, None], s["rc"], 4) @ s["w_rad"]
        msg = (g * x0[js]) @ W0.T  # [deg, C]
        for h in range(H):
            logits = (q[i, h * d : (h + 1) * d] * k[js, h * d : (h + 1) * d]).sum(1) / np.sqrt(d)
            a = softmax(logits + np.log(u))
            np.testing.assert_allclose(y[i, 0, h * d : (h + 1) * d], a @ msg[:, h * d : (h + 1) * d], atol=1e-12)


@pytest.mark.parametrize("L", [1, 3])
def test_identity_so2_weights_cancel_rotations(L):
    s = _system(10, L=L, C=2, H=1)
    C = 2
    blocks = [np.eye((L + 1) * C).ravel()]
    for m in range(1, L + 1):
        km = (L + 1 - m) * C
        blocks += [np.eye(km).ravel(), np.zeros(km * km)]
    s["w_so2"] = np.concatenate(blocks)
    y, wts = _run(s, return_weights=True)
    rp, col = neighbors_bruteforce(s["pos"].astype(np.float32), s["rc"])
    for i in range(len(rp) - 1):
        js = col[rp[i] : rp[i + 1]]
        if js.size == 0:
            continue
        r = s["pos"][js] - s["pos"][i]
        g = radial_gaussians(np.sqrt((r * r).sum(1))[:, None], s["rc"], 4) @ s["w_rad"]
        ref = np.einsum("e,ec,enc->nc", wts[i][:, 0], g, s["x"][js])
        np.testing.assert_allclose(y[i], ref, atol=1e-12)


def test_empty_neighbourhood_gives_zero():
    s = _system(11)
    s["pos"][0] = [100.0, 100.0, 100.0]
    y = _run(s)
    assert np.all(y[0] == 0.0)


def test_rbf_envelope_flag_scales_the_gate():
    s = _system(12, L=0, C=2, H=1)
    y0 = _run(s, flags=oatt.FLAG_NO_RADIAL)
    y1 = _run(s, flags=oatt.FLAG_RBF_ENVELOPE)
    assert not np.allclose(y0, y1)


# ---------------------------------------------------------------- planted mistakes


def _golden_passes():
    try:
        test_golden_two_atoms_l1_hand_worked()
        test_golden_three_atoms_envelope_softmax_l0()
        return True
    except AssertionError:
        return False


def _equivariance_passes():
    try:
        test_rotation_equivariance(0)
        return True
    except AssertionError:
        return False


def test_planted_mistakes_are_caught(monkeypatch):
    good_map, good_rot = oatt._so2_map, oatt._rotate
    assert _golden_passes() and _equivariance_passes()

    def wrong_sign(xt, w0, w1, w2, L):
        return good_map(xt, w0, w1, {m: -w for m, w in w2.items()}, L)

    monkeypatch.setattr(oatt, "_so2_map", wrong_sign)
    assert not _golden_passes()
    monkeypatch.setattr(oatt, "_so2_map", good_map)

    def no_transpose(blocks, feat, L, transpose=False):
        return good_rot(blocks, feat, L, transpose=False)

    monkeypatch.setattr(oatt, "_rotate", no_transpose)
    assert not _equivariance_passes()
    monkeypatch.setattr(oatt, "_rotate", good_rot)

    good_env = oatt.envelope
    calls = {"n": 0}

    def env_numerator_only(s, p=5):  # envelope dropped: u == 1
        calls["n"] += 1
        return np.where(np.asarray(s) < 1.0, 1.0, 0.0)

    monkeypatch.setattr(oatt, "envelope", env_numerator_only)
    assert not _golden_passes()
    monkeypatch.setattr(oatt, "envelope", good_env)
    assert calls["n"] > 0
    assert _golden_passes() and _equivariance_passes()
