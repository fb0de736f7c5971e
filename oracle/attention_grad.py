"""Gradients of the SO(2) attention layer, fp64: the forward of
oracle/attention.py written again in PyTorch CPU ops and differentiated by
autograd.  Test infrastructure (see oracle/__init__).

What it differentiates ("E2Former-V2: On-the-Fly Equivariant Attention with
Linear Activation Memory", technical summary, section 4: the Conservative
variant takes forces as derivatives of the energy through this layer;
"DPA4: Pushing the Accuracy-Cost Frontier of Interatomic Potentials with EMFA
SO(2) Convolution", technical summary, section 2.2: conservative training
differentiates the energy-to-force path): for a scalar loss L whose gradient
with respect to the layer output y is dy, the gradients of L with respect to
the node features x, the positions, W_q, W_k, W_rad and the packed SO(2)
weights.

The forward is the same sequence of steps as so2_attention_ref (O2-O12 of
oracle/attention.py), per target with its edges stacked:

  q, k         projections of the l = 0 slice
  r, rho       minimum-image edge vector r_ij = p_j - p_i and its length
  u            envelope (1 - s)^3 sum_{k<p} (k+1)(k+2)/2 s^k, s = rho / rc
  z, a         logits per head and the envelope-gated softmax (two-pass)
  g            Gaussian radial basis times W_rad
  R            Rodrigues frame with R r_hat = z_hat, written as
               I + [w] + [w]^2 / (1 + c) with w = r_hat x z_hat, c = r_hat . z_hat
               (the same rotation as frame_rotation, smooth away from
               r_hat = -z_hat)
  D            Wigner-D blocks by the exact quadrature of oracle/wigner.py
  xt, yt, v    rotate and gate, per-m map, rotate back
  y            sum_j a_ij v_ij

and L = sum(dy * y).  Autograd supplies every derivative; the tests pin them
to central finite differences of the numpy oracle, so this module checks
itself against an implementation it shares no code with."""

from math import factorial, pi, sqrt

import numpy as np
import torch
from numpy.polynomial import legendre as npleg
from numpy.polynomial import polynomial as nppoly

from .wigner import _product_quadrature

FLAG_RBF_ENVELOPE = 1
FLAG_NO_RADIAL = 2

_T = torch.float64


def _legendre_power_coeffs(l: int, m: int) -> np.ndarray:
    """Power-series coefficients of d^m/dx^m P_l (lowest degree first)."""
    c = npleg.leg2poly(npleg.Legendre.basis(l).coef)
    for _ in range(m):
        c = nppoly.polyder(c)
    return np.atleast_1d(c)


def real_sh_torch(l_max: int, v: torch.Tensor) -> torch.Tensor:
    """Real spherical harmonics of oracle/sh.py (no Condon-Shortley phase, z
    polar, index l^2 + l + m) for v [n, 3], differentiable; [n, (L+1)^2]."""
    r = torch.sqrt((v * v).sum(-1))
    u = v / r[:, None]
    ct = u[:, 2]
    st = torch.sqrt(u[:, 0] * u[:, 0] + u[:, 1] * u[:, 1])
    ph = torch.atan2(u[:, 1], u[:, 0])
    cols = [None] * ((l_max + 1) ** 2)
    for l in range(l_max + 1):
        for m in range(l + 1):
            nlm = sqrt((2 * l + 1) / (4.0 * pi) * factorial(l - m) / factorial(l + m))
            coef = _legendre_power_coeffs(l, m)
            poly = torch.zeros_like(ct)
            for cf in coef[::-1]:  # Horner
                poly = poly * ct + float(cf)
            plm = st**m * poly
            if m == 0:
                cols[l * l + l] = nlm * plm
            else:
                cols[l * l + l + m] = sqrt(2.0) * nlm * plm * torch.cos(m * ph)
                cols[l * l + l - m] = sqrt(2.0) * nlm * plm * torch.sin(m * ph)
    return torch.stack(cols, dim=1)


def wigner_blocks_torch(l_max: int, R: torch.Tensor) -> list:
    """D^l(R) for a stack R [E, 3, 3] by the quadrature D^l = sum_q w_q
    Y_l(R s_q) Y_l(s_q)^T; returns [E, 2l+1, 2l+1] per degree."""
    nodes_np, w_np = _product_quadrature(l_max)
    nodes = torch.tensor(nodes_np, dtype=_T)
    w = torch.tensor(w_np, dtype=_T)
    y_s = real_sh_torch(l_max, nodes)
    pts = torch.einsum("eij,qj->eqi", R, nodes)
    n_e, n_q = R.shape[0], nodes.shape[0]
    y_rs = real_sh_torch(l_max, pts.reshape(-1, 3)).reshape(n_e, n_q, -1)
    out = []
    for l in range(l_max + 1):
        sl = slice(l * l, (l + 1) * (l + 1))
        out.append(torch.einsum("eqa,q,qb->eab", y_rs[:, :, sl], w, y_s[:, sl]))
    return out


def frame_torch(rhat: torch.Tensor) -> torch.Tensor:
    """Rotations [E, 3, 3] with R rhat = z_hat: I + [w] + [w]^2 / (1 + c),
    w = rhat x z_hat, c = rhat . z_hat (Rodrigues about w)."""
    zero = torch.zeros_like(rhat[:, 0])
    w = torch.stack([rhat[:, 1], -rhat[:, 0], zero], dim=1)  # rhat x (0, 0, 1)
    c = rhat[:, 2]
    K = torch.zeros(rhat.shape[0], 3, 3, dtype=rhat.dtype)
    K[:, 0, 1], K[:, 0, 2] = -w[:, 2], w[:, 1]
    K[:, 1, 0], K[:, 1, 2] = w[:, 2], -w[:, 0]
    K[:, 2, 0], K[:, 2, 1] = -w[:, 1], w[:, 0]
    eye = torch.eye(3, dtype=rhat.dtype).expand_as(K)
    return eye + K + (K @ K) / (1.0 + c)[:, None, None]


def envelope_torch(s: torch.Tensor, p: int) -> torch.Tensor:
    t = 1.0 - s
    q = torch.zeros_like(s)
    for k in range(p - 1, -1, -1):
        q = q * s + (k + 1) * (k + 2) / 2.0
    return torch.where(s < 1.0, t * t * t * q, torch.zeros_like(s))


def _unpack(w_so2, l_max, C):
    off = 0
    k0 = (l_max + 1) * C
    w0 = w_so2[off : off + k0 * k0].reshape(k0, k0)
    off += k0 * k0
    w1, w2 = {}, {}
    for m in range(1, l_max + 1):
        km = (l_max + 1 - m) * C
        w1[m] = w_so2[off : off + km * km].reshape(km, km)
        off += km * km
        w2[m] = w_so2[off : off + km * km].reshape(km, km)
        off += km * km
    return w0, w1, w2


def _so2_map(xt, w0, w1, w2, l_max):
    n_e, nc, C = xt.shape
    rows = [None] * nc
    rows0 = [l * l + l for l in range(l_max + 1)]
    y0 = (xt[:, rows0].reshape(n_e, -1) @ w0.T).reshape(n_e, l_max + 1, C)
    for a, r in enumerate(rows0):
        rows[r] = y0[:, a]
    for m in range(1, l_max + 1):
        rp = [l * l + l + m for l in range(m, l_max + 1)]
        rm = [l * l + l - m for l in range(m, l_max + 1)]
        xp = xt[:, rp].reshape(n_e, -1)
        xm = xt[:, rm].reshape(n_e, -1)
        yp = (xp @ w1[m].T - xm @ w2[m].T).reshape(n_e, -1, C)
        ym = (xp @ w2[m].T + xm @ w1[m].T).reshape(n_e, -1, C)
        for a, r in enumerate(rp):
            rows[r] = yp[:, a]
        for a, r in enumerate(rm):
            rows[r] = ym[:, a]
    return torch.stack(rows, dim=1)


def so2_attention_torch(pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2, *, l_max, heads, cutoff, envelope_p=5,
                        box=None, flags=0, targets=None):
    """The forward of so2_attention_ref on torch fp64 tensors (differentiable
    in pos, x and the weights).  Returns y [T, (L+1)^2, C]."""
    n_atoms, nc, C = x.shape
    d = C // heads
    K = w_rad.shape[0]
    rc = float(np.float32(cutoff))
    w0, w1, w2 = _unpack(w_so2, l_max, C)
    q = x[:, 0, :] @ w_q
    k = x[:, 0, :] @ w_k
    mu = torch.arange(K, dtype=_T) * rc / (K - 1)
    sigma = rc / (K - 1)
    head_of = torch.arange(C) // d
    b = None if box is None else torch.tensor(np.asarray(box, dtype=np.float32).astype(np.float64), dtype=_T)
    if targets is None:
        targets = range(n_atoms)
    out = []
    for i in targets:
        js = torch.as_tensor(np.asarray(col[row_ptr[i] : row_ptr[i + 1]], dtype=np.int64))
        if js.numel() == 0:
            out.append(torch.zeros(nc, C, dtype=_T))
            continue
        r = pos[js] - pos[i]
        if b is not None:
            r = r - b * torch.round(r / b)
        rho = torch.sqrt((r * r).sum(-1))
        u = envelope_torch(rho / rc, envelope_p)
        z = (q[i][None, :] * k[js]).reshape(-1, heads, d).sum(-1) / sqrt(d)
        if flags & FLAG_NO_RADIAL:
            g = torch.ones(js.numel(), C, dtype=_T)
        else:
            phi = torch.exp(-((rho[:, None] - mu[None, :]) ** 2) / (2.0 * sigma * sigma))
            if flags & FLAG_RBF_ENVELOPE:
                phi = phi * u[:, None]
            g = phi @ w_rad
        R = frame_torch(r / rho[:, None])
        blocks = wigner_blocks_torch(l_max, R)
        xj = x[js]
        xt = torch.cat([torch.einsum("eab,ebc->eac", blocks[l], xj[:, l * l : (l + 1) ** 2]) for l in range(l_max + 1)],
                       dim=1) * g[:, None, :]
        yt = _so2_map(xt, w0, w1, w2, l_max)
        v = torch.cat([torch.einsum("eba,ebc->eac", blocks[l], yt[:, l * l : (l + 1) ** 2]) for l in range(l_max + 1)],
                      dim=1)
        zmax = z.max(dim=0).values.detach()
        ew = u[:, None] * torch.exp(z - zmax[None, :])
        den = ew.sum(0)
        a = ew / den[None, :]
        out.append(torch.einsum("ec,enc->nc", a[:, head_of], v))
    return torch.stack(out)


def so2_attention_grad_ref(pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2, dy, *, l_max, heads, cutoff, envelope_p=5,
                           box=None, flags=0, targets=None):
    """Gradients of L = sum(dy * y) with y = so2_attention_ref(...) for the
    targets (default all atoms; dy has one row per target).  Returns a dict
    of fp64 numpy arrays: y, dx [N, (L+1)^2, C], dpos [N, 3], dw_q, dw_k,
    dw_rad, dw_so2.  Targets whose softmax normaliser is 0 (all envelopes 0)
    are not supported (the layer is not differentiable there)."""
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), dtype=_T, requires_grad=True)
    P, X, WQ, WK, WR, WS = (t(a) for a in (np.asarray(pos).astype(np.float64), x, w_q, w_k, w_rad, w_so2))
    y = so2_attention_torch(P, np.asarray(row_ptr), np.asarray(col), X, WQ, WK, WR, WS, l_max=l_max, heads=heads,
                            cutoff=cutoff, envelope_p=envelope_p, box=box, flags=flags, targets=targets)
    G = torch.tensor(np.asarray(dy, dtype=np.float64), dtype=_T)
    loss = (G * y).sum()
    grads = torch.autograd.grad(loss, [X, P, WQ, WK, WR, WS], allow_unused=True)
    names = ["dx", "dpos", "dw_q", "dw_k", "dw_rad", "dw_so2"]
    shapes = [X.shape, P.shape, WQ.shape, WK.shape, WR.shape, WS.shape]
    out = {"y": y.detach().numpy()}
    for n, gr, sh in zip(names, grads, shapes):
        out[n] = np.zeros(tuple(sh)) if gr is None else gr.detach().numpy()
    return out
