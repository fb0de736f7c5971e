"""Pins for the oracle's variants of the value path and the logits
(so2_attention_ref's m_max, w_logit, n_focus / w_focus):

* m_max = L is the base layer; m_max < L equals the base layer with the
  weight blocks of the orders above m_max set to zero (a different code
  path: the full packing), and stays rotation equivariant;
* the radial logit bias at L = 0 is textbook scalar attention with logits
  z + sum_k phi_k w_logit[k] and weights u e^z (scipy's softmax);
* multi-focus: one stream is the base layer; with w_focus = 0 every stream
  gets weight 1/F, which equals the base layer with block-diagonal weights
  divided by F; at L = 0 the cross-focus softmax matches a direct formula;
  rotation equivariance with F = 2."""

import numpy as np
import pytest
from scipy.spatial.transform import Rotation
from scipy.special import softmax

from oracle import (
    envelope,
    neighbors_bruteforce,
    radial_gaussians,
    so2_attention_ref,
    so2_weight_count,
    unpack_so2,
    wigner_d_blocks,
)


def _system(seed, n=12, side=6.0, rc=4.0, L=2, C=4, H=2, K=4):
    rng = np.random.default_rng(seed)
    while True:
        pos = rng.uniform(0.0, side, size=(n, 3))
        d = pos[:, None, :] - pos[None, :, :]
        r = np.sqrt((d * d).sum(-1))
        np.fill_diagonal(r, 1.0)
        if np.all(np.abs(r - rc) > 1e-3) and r.min() > 0.5:
            break
    nc = (L + 1) ** 2
    return dict(pos=pos, x=rng.standard_normal((n, nc, C)), w_q=rng.standard_normal((C, C)) / np.sqrt(C),
                w_k=rng.standard_normal((C, C)) / np.sqrt(C), w_rad=rng.standard_normal((K, C)) / np.sqrt(K),
                L=L, H=H, rc=rc, C=C, K=K, rng=rng)


def _run(s, w_so2, pos=None, x=None, **kw):
    pos = s["pos"] if pos is None else pos
    x = s["x"] if x is None else x
    rp, col = neighbors_bruteforce(pos.astype(np.float32), s["rc"])
    return so2_attention_ref(pos, rp, col, x, s["w_q"], s["w_k"], s["w_rad"], w_so2, l_max=s["L"], heads=s["H"],
                             cutoff=s["rc"], **kw)


def _rot(x, R, L):
    D = wigner_d_blocks(L, R)
    out = np.empty_like(x)
    for l in range(L + 1):
        sl = slice(l * l, (l + 1) ** 2)
        out[:, sl] = np.einsum("ab,nbc->nac", D[l], x[:, sl])
    return out


def _pack(w0, w1, w2, L):
    parts = [w0.ravel()]
    for m in range(1, L + 1):
        parts += [w1[m].ravel(), w2[m].ravel()]
    return np.concatenate(parts)


def test_m_max_equals_zeroed_high_orders():
    s = _system(0, L=3, C=3, H=1)
    L, C = s["L"], s["C"]
    full = s["rng"].standard_normal(so2_weight_count(L, C)) / np.sqrt(C * (L + 1))
    np.testing.assert_array_equal(_run(s, full, m_max=L), _run(s, full))
    for m_max in (0, 1, 2):
        w0, w1, w2 = unpack_so2(full, L, C)
        trunc = _pack(w0, {m: w1[m] for m in range(1, m_max + 1)}, {m: w2[m] for m in range(1, m_max + 1)}, m_max)
        assert trunc.size == so2_weight_count(L, C, m_max)
        zeroed = _pack(w0, {m: (w1[m] if m <= m_max else 0 * w1[m]) for m in w1},
                       {m: (w2[m] if m <= m_max else 0 * w2[m]) for m in w2}, L)
        np.testing.assert_allclose(_run(s, trunc, m_max=m_max), _run(s, zeroed), atol=1e-13)


def test_m_max_equivariance():
    s = _system(1, L=3, C=3, H=1)
    w = s["rng"].standard_normal(so2_weight_count(3, 3, 1))
    R = Rotation.random(random_state=2).as_matrix()
    c = s["pos"].mean(0)
    y = _run(s, w, m_max=1)
    y_r = _run(s, w, pos=(s["pos"] - c) @ R.T + c, x=_rot(s["x"], R, 3), m_max=1)
    np.testing.assert_allclose(y_r, _rot(y, R, 3), atol=1e-11)


def test_logit_bias_l0_scalar_attention():
    s = _system(2, L=0, C=4, H=2, K=5)
    C, H, K = 4, 2, 5
    d = C // H
    w0 = s["rng"].standard_normal((C, C))
    wl = s["rng"].standard_normal((K, H))
    y = _run(s, w0.ravel(), w_logit=wl)
    rp, col = neighbors_bruteforce(s["pos"].astype(np.float32), s["rc"])
    x0 = s["x"][:, 0, :]
    q, k = x0 @ s["w_q"], x0 @ s["w_k"]
    for i in range(len(rp) - 1):
        js = col[rp[i] : rp[i + 1]]
        if js.size == 0:
            continue
        r = s["pos"][js] - s["pos"][i]
        rho = np.sqrt((r * r).sum(1))
        phi = radial_gaussians(rho[:, None], s["rc"], K)
        msg = ((phi @ s["w_rad"]) * x0[js]) @ w0.T
        for h in range(H):
            z = (q[i, h * d : (h + 1) * d] * k[js, h * d : (h + 1) * d]).sum(1) / np.sqrt(d) + phi @ wl[:, h]
            a = softmax(z + np.log(envelope(rho / s["rc"])))
            np.testing.assert_allclose(y[i, 0, h * d : (h + 1) * d], a @ msg[:, h * d : (h + 1) * d], atol=1e-12)


def test_single_focus_is_the_base_layer():
    s = _system(3, C=4)
    w = s["rng"].standard_normal(so2_weight_count(2, 4))
    np.testing.assert_array_equal(_run(s, w, n_focus=1, w_focus=np.ones(4)), _run(s, w))


def test_uniform_focus_weights_give_block_diagonal_map_over_f():
    s = _system(4, L=2, C=6, H=3)
    L, C, F = 2, 6, 3
    cf = C // F
    per = so2_weight_count(L, cf)
    w = s["rng"].standard_normal(F * per)
    stacks = [unpack_so2(w[f * per : (f + 1) * per], L, cf) for f in range(F)]

    def blockdiag(mats, nblk):
        # stream f's [(L+1-m) cf]^2 block placed on channels f cf .. (f+1) cf of each degree
        km = mats[0].shape[0] // cf
        out = np.zeros((km * C, km * C))
        for f, M in enumerate(mats):
            for a in range(km):
                for b in range(km):
                    out[a * C + f * cf : a * C + (f + 1) * cf, b * C + f * cf : b * C + (f + 1) * cf] = \
                        M[a * cf : (a + 1) * cf, b * cf : (b + 1) * cf]
        return out

    w0 = blockdiag([st[0] for st in stacks], F)
    w1 = {m: blockdiag([st[1][m] for st in stacks], F) for m in range(1, L + 1)}
    w2 = {m: blockdiag([st[2][m] for st in stacks], F) for m in range(1, L + 1)}
    y = _run(s, w, n_focus=F, w_focus=np.zeros(C))
    np.testing.assert_allclose(y, _run(s, _pack(w0, w1, w2, L)) / F, atol=1e-13)


def test_focus_softmax_l0_direct_formula():
    s = _system(5, L=0, C=4, H=1, K=4)
    C, F = 4, 2
    cf = C // F
    w = s["rng"].standard_normal(F * cf * cf)
    wf = s["rng"].standard_normal(C)
    y = _run(s, w, n_focus=F, w_focus=wf)
    rp, col = neighbors_bruteforce(s["pos"].astype(np.float32), s["rc"])
    x0 = s["x"][:, 0, :]
    q, k = x0 @ s["w_q"], x0 @ s["w_k"]
    W = [w[f * cf * cf : (f + 1) * cf * cf].reshape(cf, cf) for f in range(F)]
    for i in range(len(rp) - 1):
        js = col[rp[i] : rp[i + 1]]
        if js.size == 0:
            continue
        r = s["pos"][js] - s["pos"][i]
        rho = np.sqrt((r * r).sum(1))
        xt = (radial_gaussians(rho[:, None], s["rc"], 4) @ s["w_rad"]) * x0[js]
        msg = np.concatenate([xt[:, f * cf : (f + 1) * cf] @ W[f].T for f in range(F)], axis=1)
        score = np.stack([(msg[:, f * cf : (f + 1) * cf] * wf[f * cf : (f + 1) * cf]).sum(1) for f in range(F)], 1)
        pi = softmax(score, axis=1)
        msg = msg * np.repeat(pi, cf, axis=1)
        a = softmax((q[i] * k[js]).sum(1) / np.sqrt(C) + np.log(envelope(rho / s["rc"])))
        np.testing.assert_allclose(y[i, 0], a @ msg, atol=1e-12)


def test_multi_focus_equivariance():
    s = _system(6, L=3, C=4, H=2)
    F = 2
    w = s["rng"].standard_normal(so2_weight_count(3, 4, n_focus=F))
    wf = s["rng"].standard_normal(4)
    R = Rotation.random(random_state=9).as_matrix()
    c = s["pos"].mean(0)
    y = _run(s, w, n_focus=F, w_focus=wf)
    y_r = _run(s, w, pos=(s["pos"] - c) @ R.T + c, x=_rot(s["x"], R, 3), n_focus=F, w_focus=wf)
    np.testing.assert_allclose(y_r, _rot(y, R, 3), atol=1e-11)


def test_variant_argument_errors():
    s = _system(7)
    w = np.zeros(so2_weight_count(2, 4))
    with pytest.raises(ValueError):
        _run(s, w, m_max=3)
    with pytest.raises(ValueError):
        _run(s, w, n_focus=2)  # w_focus missing
    with pytest.raises(ValueError):
        _run(s, w, n_focus=3, w_focus=np.ones(4))  # 3 does not divide 4
