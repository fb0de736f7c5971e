"""The on-the-fly SO(2) equivariant graph attention forward pass as a plain
per-edge loop in fp64.  Test infrastructure (see oracle/__init__).

Sources (page titles; the pages print no equations, so each step below is a
reading of their prose):

* "E2Former-V2: On-the-Fly Equivariant Attention with Linear Activation
  Memory", technical summary
  - section 2.1 (EAAS): rotate each neighbour's irreps into the frame aligned
    with the edge vector, apply sparse block-wise linear maps (one complex
    linear map per |m|, mixing all degrees l >= |m| and all channels), rotate
    back;
  - section 2.2: query and key are SO(3)-invariant scalar projections (its
    "Eq. 6"), geometry enters only through the value path, a softmax runs
    over the neighbours j in N(i), value updates are accumulated per atom.
* "EquiformerV3: Scaling Efficient, Expressive, and General
  SE(3)-Equivariant Graph Attention Transformers", technical summary,
  section 2.B.3: the envelope of the smooth radius cutoff multiplies the
  attention terms in the numerator and in the softmax denominator.
* "DPA4: Pushing the Accuracy-Cost Frontier of Interatomic Potentials with
  EMFA SO(2) Convolution", technical summary, section 2.1 A3:
  envelope-gated attention with weights from the invariant l = 0 section
  (corroborates the above).

The softmax here is two-pass (max, then normalised sum); the streaming GPU
kernel reaches the same numbers by a different schedule.

Steps for each target atom i and each neighbour j (r_ij = mic(p_j - p_i)):

  O2  q_i = x_i[l=0] @ W_q,  k_j = x_j[l=0] @ W_k                 (fp64)
  O3  z_ij^h = q_i^h . k_j^h / sqrt(d),  d = C / H, head h owns channels
      [h d, (h+1) d)
  O4  u_ij = envelope(rho / rc), the polynomial envelope of exponent p
  O5  a_ij^h = u_ij exp(z_ij^h - M_i^h) / sum_k u_ik exp(z_ik^h - M_i^h)
  O6  g_ij[c] = sum_k phi_k(rho) W_rad[k][c], Gaussian radial basis
  O7  R_ij proper rotation with R_ij r_hat = z_hat
  O8  D^l(R_ij) Wigner-D blocks
  O9  xt = D(R_ij) x_j (per degree), then xt[:, c] *= g_ij[c]
  O10 SO(2) map per m: m = 0 real (W0), m >= 1 complex (W1 + i W2)
  O11 v_ij = D(R_ij)^T yt
  O12 y_i = sum_j a_ij^{h(c)} v_ij[:, c];  y_i = 0 when N(i) is empty
"""

from math import sqrt

import numpy as np

from .sh import n_comp
from .wigner import frame_rotation, rot_z, wigner_d_blocks

FLAG_RBF_ENVELOPE = 1  # alternative reading: phi_k(rho) is also multiplied by u
FLAG_NO_RADIAL = 2  # g_ij == 1 (used by special-case tests)


def so2_weight_count(l_max: int, channels: int, m_max=None, n_focus: int = 1) -> int:
    """C^2 [(L+1)^2 + 2 sum_{m=1..m_max} (L+1-m)^2] for one stack over C
    channels (m_max = L by default); with F focus streams, F stacks over C/F
    channels each."""
    m_max = l_max if m_max is None else m_max
    cf = channels // n_focus
    total = (l_max + 1) ** 2
    for m in range(1, m_max + 1):
        total += 2 * (l_max + 1 - m) ** 2
    return n_focus * total * cf * cf


def unpack_so2(w_so2, l_max: int, channels: int, m_max=None):
    """Split one stack of packed SO(2) weights.

    Packing: W0 [(L+1)C x (L+1)C], then for m = 1..m_max (L by default) the
    pair W1_m, W2_m, each [(L+1-m)C x (L+1-m)C]; every block row-major
    [out][in] with row and column index (l - m) C + c.  Returns (W0,
    {m: W1_m}, {m: W2_m})."""
    m_max = l_max if m_max is None else m_max
    w = np.asarray(w_so2, dtype=np.float64).ravel()
    C = channels
    off = 0
    k0 = (l_max + 1) * C
    w0 = w[off : off + k0 * k0].reshape(k0, k0)
    off += k0 * k0
    w1, w2 = {}, {}
    for m in range(1, m_max + 1):
        km = (l_max + 1 - m) * C
        w1[m] = w[off : off + km * km].reshape(km, km)
        off += km * km
        w2[m] = w[off : off + km * km].reshape(km, km)
        off += km * km
    if off != w.size:
        raise ValueError(f"w_so2 has {w.size} entries, expected {off}")
    return w0, w1, w2


def envelope(s, p: int = 5):
    """u(s) = 1 - (p+1)(p+2)/2 s^p + p(p+2) s^(p+1) - p(p+1)/2 s^(p+2) for
    0 <= s < 1, else 0 (the polynomial cutoff envelope; with p = 5 it reads
    1 - 21 s^5 + 35 s^6 - 15 s^7).

    u(1) = u'(1) = u''(1) = 0, so (1 - s)^3 divides u, and since u = 1 +
    O(s^p) the cofactor is the degree p-1 truncation of 1 / (1 - s)^3:
        u(s) = (1 - s)^3 sum_{k=0}^{p-1} (k+1)(k+2)/2 s^k.
    That form is evaluated here: every term is positive on [0, 1), so it
    keeps its relative precision up to the cutoff, where the expanded sum
    cancels to rounding noise."""
    s = np.asarray(s, dtype=np.float64)
    t = 1.0 - s
    q = np.zeros_like(s)
    for k in range(p - 1, -1, -1):  # Horner, highest power first
        q = q * s + (k + 1) * (k + 2) / 2.0
    u = t * t * t * q
    return np.where(s < 1.0, u, 0.0)


def radial_gaussians(rho, cutoff: float, n_rbf: int):
    """phi_k(rho) = exp(-(rho - mu_k)^2 / (2 sigma^2)), mu_k = k rc/(K-1),
    sigma = rc/(K-1), k = 0..K-1 (centres include both ends of [0, rc])."""
    rc = float(np.float32(cutoff))
    mu = np.arange(n_rbf, dtype=np.float64) * rc / (n_rbf - 1)
    sigma = rc / (n_rbf - 1)
    return np.exp(-((rho - mu) ** 2) / (2.0 * sigma * sigma))


def _mic(r, box):
    if box is None:
        return r
    b = np.asarray(box, dtype=np.float32).astype(np.float64)
    return r - b * np.rint(r / b)


def _rotate(blocks, feat, l_max, transpose=False):
    """Apply blockdiag(D^l) (or its transpose) to feat [(L+1)^2, C]."""
    out = np.empty_like(feat)
    for l in range(l_max + 1):
        sl = slice(l * l, (l + 1) * (l + 1))
        d = blocks[l].T if transpose else blocks[l]
        out[sl] = d @ feat[sl]
    return out


def _so2_map(xt, w0, w1, w2, l_max):
    """O10, the per-m map in the edge frame, for a stack of edges
    xt [E, (L+1)^2, C] (the same map for every edge; each edge's rows form
    a row vector, so W v is written v W^T):

    m = 0:  yt[(l,0)]  = sum_{l'} W0[(l,.),(l',.)] xt[(l',0)]
    m >= 1: yt_+ = W1 xt_+ - W2 xt_-,  yt_- = W2 xt_+ + W1 xt_-
    with xt_{+/-} the rows (l, +/-m), l = m..L, stacked as (l - m) C + c."""
    n_e, _, C = xt.shape
    yt = np.zeros_like(xt)
    rows0 = [l * l + l for l in range(l_max + 1)]
    y0 = xt[:, rows0].reshape(n_e, -1) @ w0.T
    yt[:, rows0] = y0.reshape(n_e, l_max + 1, C)
    for m in sorted(w1):  # m = 1..m_max; rows with |m| > m_max stay 0
        rp = [l * l + l + m for l in range(m, l_max + 1)]
        rm = [l * l + l - m for l in range(m, l_max + 1)]
        xp = xt[:, rp].reshape(n_e, -1)
        xm = xt[:, rm].reshape(n_e, -1)
        yp = xp @ w1[m].T - xm @ w2[m].T
        ym = xp @ w2[m].T + xm @ w1[m].T
        yt[:, rp] = yp.reshape(n_e, -1, C)
        yt[:, rm] = ym.reshape(n_e, -1, C)
    return yt


def so2_attention_ref(
    pos,
    row_ptr,
    col,
    x,
    w_q,
    w_k,
    w_rad,
    w_so2,
    *,
    l_max: int,
    heads: int,
    cutoff: float,
    envelope_p: int = 5,
    box=None,
    flags: int = 0,
    targets=None,
    gauge=None,
    return_weights: bool = False,
    m_max=None,
    w_logit=None,
    n_focus: int = 1,
    w_focus=None,
):
    """y[t] for each target t (default: all atoms), shape [T, (L+1)^2, C].

    pos     [N,3] positions (fp32 is widened exactly to fp64)
    row_ptr, col   CSR of N(i)
    x       [N,(L+1)^2,C] features (bf16 inputs are passed as their exact
            values); W_q, W_k [C][C] (in, out); W_rad [K][C]; w_so2 packed
    gauge   optional callable (target, edge_index) -> angle; the edge frame
            becomes rot_z(angle) @ R_ij (the output must not change)
    return_weights  also return {target: a [deg, H]}

    Variants of the value path and the logits (readings V1-V3):
    m_max   the per-m maps stop at |m| = m_max (default L): the rows with
            |m| > m_max of the edge-frame message are 0, and w_so2 holds the
            blocks for m = 0..m_max only
    w_logit [K][H]: a radial logit bias, z_ij^h += sum_k phi_k(rho) w_logit[k][h]
            (the same Gaussian basis as the gate, without the envelope)
    n_focus F > 1: the channels form F contiguous streams of C/F; each
            stream has its own stack of per-m maps (w_so2 is the F stacks
            back to back, stack f acting on channels [f C/F, (f+1) C/F)),
            and the streams of one edge are weighted by pi = softmax over f
            of score_f = sum_{c in f} w_focus[c] yt[(0,0), c], the invariant
            l = 0 part of the stream's edge-frame message (DPA4's
            cross-focus competition); w_focus [C] is required
    """
    # fp32 positions are widened exactly; fp64 positions (symmetry tests)
    # are used as they are.
    pos = np.asarray(pos).astype(np.float64)
    x = np.asarray(x, dtype=np.float64)
    n_atoms, nc, C = x.shape
    if nc != n_comp(l_max):
        raise ValueError("x has the wrong number of irreps components")
    if C % heads:
        raise ValueError("channels must split evenly into heads")
    d = C // heads
    w_q = np.asarray(w_q, dtype=np.float64)
    w_k = np.asarray(w_k, dtype=np.float64)
    w_rad = np.asarray(w_rad, dtype=np.float64)
    n_rbf = w_rad.shape[0]
    m_max = l_max if m_max is None else int(m_max)
    if not 0 <= m_max <= l_max:
        raise ValueError("m_max must lie in 0..l_max")
    if C % n_focus or (n_focus > 1 and w_focus is None):
        raise ValueError("n_focus must divide C, and w_focus is required with several streams")
    cf = C // n_focus
    w_flat = np.asarray(w_so2, dtype=np.float64).ravel()
    per = so2_weight_count(l_max, cf, m_max)
    if w_flat.size != n_focus * per:
        raise ValueError(f"w_so2 has {w_flat.size} entries, expected {n_focus * per}")
    stacks = [unpack_so2(w_flat[f * per : (f + 1) * per], l_max, cf, m_max) for f in range(n_focus)]
    w_logit = None if w_logit is None else np.asarray(w_logit, dtype=np.float64)
    w_focus = None if w_focus is None else np.asarray(w_focus, dtype=np.float64)
    rc = float(np.float32(cutoff))
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col = np.asarray(col, dtype=np.int64)

    q = x[:, 0, :] @ w_q  # O2
    k = x[:, 0, :] @ w_k
    head_of = np.arange(C) // d

    if targets is None:
        targets = range(n_atoms)
    targets = list(targets)
    y = np.zeros((len(targets), nc, C), dtype=np.float64)
    weights = {}
    for ti, i in enumerate(targets):
        js = col[row_ptr[i] : row_ptr[i + 1]]
        deg = js.size
        if deg == 0:
            continue
        z = np.empty((deg, heads))
        u = np.empty(deg)
        g = np.empty((deg, C))
        frames = np.empty((deg, 3, 3))
        for e, j in enumerate(js):
            r = _mic(pos[j] - pos[i], box)
            rho = sqrt(float(r @ r))
            u[e] = envelope(rho / rc, envelope_p)  # O4
            for h in range(heads):  # O3
                z[e, h] = q[i, h * d : (h + 1) * d] @ k[j, h * d : (h + 1) * d] / sqrt(d)
            if w_logit is not None:  # V2, radial logit bias
                z[e] += radial_gaussians(rho, cutoff, n_rbf) @ w_logit
            if flags & FLAG_NO_RADIAL:  # O6
                g[e] = 1.0
            else:
                phi = radial_gaussians(rho, cutoff, n_rbf)
                if flags & FLAG_RBF_ENVELOPE:
                    phi = phi * u[e]
                g[e] = phi @ w_rad
            frames[e] = frame_rotation(r / rho)  # O7
            if gauge is not None:
                frames[e] = rot_z(gauge(i, e)) @ frames[e]
        blocks = wigner_d_blocks(l_max, frames)  # O8, one [deg, 2l+1, 2l+1] stack per degree
        xt = np.empty((deg, nc, C))
        for e, j in enumerate(js):
            xt[e] = _rotate([b[e] for b in blocks], x[j], l_max) * g[e][None, :]  # O9
        yt = np.concatenate(  # O10, every edge of i through the same map, stream by stream (V1, V3)
            [_so2_map(xt[:, :, f * cf : (f + 1) * cf], *stacks[f], l_max) for f in range(n_focus)], axis=2
        )
        if n_focus > 1:  # V3, cross-focus softmax over the streams' invariant l = 0 message
            score = (yt[:, 0, :] * w_focus[None, :]).reshape(deg, n_focus, cf).sum(-1)
            pi = np.exp(score - score.max(axis=1, keepdims=True))
            pi /= pi.sum(axis=1, keepdims=True)
            yt = yt * np.repeat(pi, cf, axis=1)[:, None, :]
        v = np.empty((deg, nc, C))
        for e in range(deg):
            v[e] = _rotate([b[e] for b in blocks], yt[e], l_max, transpose=True)  # O11
        zmax = z.max(axis=0)  # O5, two-pass softmax
        ew = u[:, None] * np.exp(z - zmax[None, :])
        den = ew.sum(axis=0)
        a = np.where(den > 0.0, ew / np.where(den > 0.0, den, 1.0), 0.0)
        weights[i] = a
        y[ti] = np.einsum("ec,enc->nc", a[:, head_of], v)  # O12
    if return_weights:
        return y, weights
    return y


def max_rel_error(y_test, y_ref) -> float:
    """max_i max_{(l,m),c} |y_test - y_ref| / max(||y_ref,i||_inf,
    1e-6 ||y_ref||_inf): the error normalised per atom, since an
    elementwise relative error is undefined near zero."""
    yr = np.asarray(y_ref, dtype=np.float64)
    if yr.size == 0:
        return 0.0
    yt = np.asarray(y_test, dtype=np.float64).reshape(len(yr), -1)
    yr = yr.reshape(len(yr), -1)
    glob = np.abs(yr).max()
    per_atom = np.maximum(np.abs(yr).max(axis=1), 1e-6 * glob)
    per_atom = np.where(per_atom > 0.0, per_atom, 1.0)
    return float((np.abs(yt - yr).max(axis=1) / per_atom).max())
