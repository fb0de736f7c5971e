"""Pins for the oracle's gradients (oracle/attention_grad.py).

* its PyTorch forward reproduces the numpy oracle so2_attention_ref;
* every gradient (x, positions, W_q, W_k, W_rad, the SO(2) weights) equals
  the central finite difference of the numpy oracle along random
  directions, with and without a periodic box and for both flags;
* forces sum to zero (the layer depends on position differences only);
* rotation covariance: rotating positions, features and the upstream
  gradient rotates the position gradient by R and the feature gradient by
  D(R);
* a planted mistake in the forward (a dropped envelope derivative, through a
  cutoff-free envelope) breaks the finite-difference pin."""

import numpy as np
import pytest
from scipy.spatial.transform import Rotation

import oracle.attention_grad as og
from oracle import neighbors_bruteforce, so2_attention_ref, so2_weight_count, wigner_d_blocks


def _system(seed, n=10, side=5.5, rc=4.0, L=2, C=4, H=2, K=5, box=None):
    rng = np.random.default_rng(seed)
    while True:
        pos = rng.uniform(0.0, side, size=(n, 3))
        dd = pos[:, None, :] - pos[None, :, :]
        if box is not None:
            dd -= box * np.rint(dd / box)
        r = np.sqrt((dd * dd).sum(-1))
        np.fill_diagonal(r, 1.0)
        if np.all(np.abs(r - rc) > 5e-3) and r.min() > 0.7:
            break
    nc = (L + 1) ** 2
    return dict(
        pos=pos, x=rng.standard_normal((n, nc, C)), w_q=rng.standard_normal((C, C)) / np.sqrt(C),
        w_k=rng.standard_normal((C, C)) / np.sqrt(C), w_rad=rng.standard_normal((K, C)) / np.sqrt(K),
        w_so2=rng.standard_normal(so2_weight_count(L, C)) / np.sqrt(C * (L + 1)), L=L, H=H, rc=rc, box=box,
        dy=rng.standard_normal((n, nc, C)),
    )


def _graph(s):
    return neighbors_bruteforce(s["pos"].astype(np.float32), s["rc"], s["box"])


def _kw(s, flags=0):
    return dict(l_max=s["L"], heads=s["H"], cutoff=s["rc"], box=s["box"], flags=flags)


def _loss(s, rp, col, flags=0, **over):
    a = {k: over.get(k, s[k]) for k in ("pos", "x", "w_q", "w_k", "w_rad", "w_so2")}
    y = so2_attention_ref(a["pos"], rp, col, a["x"], a["w_q"], a["w_k"], a["w_rad"], a["w_so2"], **_kw(s, flags))
    return float((s["dy"] * y).sum())


def _grads(s, rp, col, flags=0):
    return og.so2_attention_grad_ref(s["pos"], rp, col, s["x"], s["w_q"], s["w_k"], s["w_rad"], s["w_so2"], s["dy"],
                                     **_kw(s, flags))


def test_torch_forward_matches_numpy_oracle():
    for box in (None, np.array([8.5, 8.5, 8.5])):
        s = _system(0, L=3, C=3, H=1, box=box)
        rp, col = _graph(s)
        y_np = so2_attention_ref(s["pos"], rp, col, s["x"], s["w_q"], s["w_k"], s["w_rad"], s["w_so2"], **_kw(s))
        g = _grads(s, rp, col)
        np.testing.assert_allclose(g["y"], y_np, atol=1e-12)


@pytest.mark.parametrize("flags,box", [(0, None), (0, 8.5), (1, None), (2, 8.5)])
def test_gradients_match_finite_differences(flags, box):
    s = _system(1 + flags, box=None if box is None else np.array([box] * 3))
    rp, col = _graph(s)
    g = _grads(s, rp, col, flags)
    rng = np.random.default_rng(7)
    h = 1e-5
    for name, key in (("x", "dx"), ("pos", "dpos"), ("w_q", "dw_q"), ("w_k", "dw_k"), ("w_rad", "dw_rad"),
                      ("w_so2", "dw_so2")):
        for _ in range(2):
            d = rng.standard_normal(s[name].shape)
            fd = (_loss(s, rp, col, flags, **{name: s[name] + h * d}) - _loss(s, rp, col, flags, **{name: s[name] - h * d})) / (2 * h)
            an = float((g[key] * d).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    if flags & og.FLAG_NO_RADIAL:
        assert np.all(g["dw_rad"] == 0.0)


def test_forces_sum_to_zero_and_rotate_covariantly():
    s = _system(5, L=3, C=3, H=3)
    rp, col = _graph(s)
    g = _grads(s, rp, col)
    assert np.abs(g["dpos"].sum(0)).max() < 1e-12 * max(1.0, np.abs(g["dpos"]).max()) + 1e-13
    R = Rotation.random(random_state=3).as_matrix()
    D = wigner_d_blocks(s["L"], R)

    def rot(f):
        out = np.empty_like(f)
        for l in range(s["L"] + 1):
            sl = slice(l * l, (l + 1) ** 2)
            out[:, sl] = np.einsum("ab,nbc->nac", D[l], f[:, sl])
        return out

    c = s["pos"].mean(0)
    s2 = dict(s, pos=(s["pos"] - c) @ R.T + c, x=rot(s["x"]), dy=rot(s["dy"]))
    rp2, col2 = _graph(s2)
    assert np.array_equal(rp2, rp) and np.array_equal(col2, col)
    g2 = _grads(s2, rp2, col2)
    np.testing.assert_allclose(g2["dpos"], g["dpos"] @ R.T, atol=1e-11)
    np.testing.assert_allclose(g2["dx"], rot(g["dx"]), atol=1e-11)
    for key in ("dw_q", "dw_k", "dw_rad", "dw_so2"):
        np.testing.assert_allclose(g2[key], g[key], atol=1e-11)


def test_planted_mistake_breaks_the_pin(monkeypatch):
    # an envelope without its cutoff polynomial (u = 1 inside) changes the
    # forward of the torch copy only, so the finite differences of the numpy
    # oracle no longer match its position gradient
    s = _system(9)
    rp, col = _graph(s)
    good = og.envelope_torch
    monkeypatch.setattr(og, "envelope_torch", lambda s_, p: good(s_, p) * 0.0 + (s_ < 1.0).to(s_.dtype))
    g = _grads(s, rp, col)
    monkeypatch.setattr(og, "envelope_torch", good)
    d = np.random.default_rng(1).standard_normal(s["pos"].shape)
    h = 1e-5
    fd = (_loss(s, rp, col, pos=s["pos"] + h * d) - _loss(s, rp, col, pos=s["pos"] - h * d)) / (2 * h)
    assert abs(fd - float((g["dpos"] * d).sum())) > 1e-4
