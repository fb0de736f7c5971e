"""Parity of so2_attention_fwd_variant on the GPU against the oracle's
variants (m_max < L, radial logit bias, F focus streams with the
cross-focus softmax), through the C ABI:

* fp32 on the edge-batch path, every atom of the tiny workload, each
  variant alone and all together, at 1e-4; 128 heads and 128 focus streams
  at C = 256;
* targets whose edges take two and three batches (64 edges per target, at
  least 4096), with and without variants;
* bf16 inputs on the MFMA kernel at 2e-2: the logit bias (a small-molecule
  batch, and seeded targets of the L = 6 water box) and truncated orders
  (m_max = 0..3 at L = 4, m_max = L - 1 and 0 at every other degree, m_max =
  2 and 4 on seeded targets of the L = 6 water box) and 2, 4, 8 focus
  streams at L <= 4 (small molecules, every degree 1..3, seeded targets of a
  20,000-atom water box); focus streams with truncated orders or of 8
  channels on the edge-batch path (fp32 arithmetic, 1e-4);
* the base variant through the variant call is bitwise the base call;
  repeated calls on the edge-batch path are bitwise equal."""

import numpy as np
import pytest

from helpers import TOL, csr_to_device, device_inputs, say
from oracle import max_rel_error, neighbors_bruteforce, so2_attention_ref, so2_weight_count
from synth import make_workload, to_bf16_exact

pytestmark = pytest.mark.gpu


def _weights(w, m_max, n_focus, logit, seed=0):
    rng = np.random.default_rng(seed)
    L, C, H, K = w.l_max, w.channels, w.heads, w.n_rbf
    mm = L if m_max < 0 else m_max
    cf = C // n_focus
    ws = (rng.standard_normal(so2_weight_count(L, C, mm, n_focus)) / np.sqrt(cf * (L + 1))).astype(np.float32)
    wl = (rng.standard_normal((K, H)) * 0.5).astype(np.float32) if logit else None
    wf = (rng.standard_normal(C) / np.sqrt(cf)).astype(np.float32) if n_focus > 1 else None
    if w.dtype == "bf16":
        ws = to_bf16_exact(ws)
        wl = None if wl is None else to_bf16_exact(wl)
        wf = None if wf is None else to_bf16_exact(wf)
    return ws, wl, wf


def _run(w, m_max=-1, n_focus=1, logit=False, targets=None, n_targets=None, out=None):
    import torch

    import so_equivariant_graph_amd as sea

    ws, wl, wf = _weights(w, m_max, n_focus, logit)
    w.w_so2 = ws
    d = device_inputs(w)
    rp, col = neighbors_bruteforce(w.pos, w.cutoff, w.box, w.mol_id)
    rp_d, col_d = csr_to_device(rp, col)
    dt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    t = lambda a: None if a is None else torch.from_numpy(a).to(device="cuda", dtype=dt)
    y = sea.so2_attention_fwd_variant(
        d["pos"], rp_d, col_d, d["x"], d["w_q"], d["w_k"], d["w_rad"], d["w_so2"], l_max=w.l_max, heads=w.heads,
        cutoff=w.cutoff, envelope_p=w.envelope_p, box=w.box, m_max=m_max, n_focus=n_focus, w_logit=t(wl),
        w_focus=t(wf), n_targets=n_targets,
    )
    torch.cuda.synchronize()
    if out is not None:
        out.append(y.clone())
    nt = w.n_atoms if n_targets is None else n_targets
    tg = np.arange(nt) if targets is None else np.asarray(targets)
    y_ref = so2_attention_ref(w.pos, rp, col, w.x, w.w_q, w.w_k, w.w_rad, ws, l_max=w.l_max, heads=w.heads,
                              cutoff=w.cutoff, envelope_p=w.envelope_p, box=w.box, targets=tg,
                              m_max=None if m_max < 0 else m_max, w_logit=wl, n_focus=n_focus, w_focus=wf)
    err = max_rel_error(y.cpu().numpy()[tg], y_ref)
    say("variant m_max", m_max, "focus", n_focus, "logit", logit, "max rel err", err)
    return err


def _kind(w, m_max, n_focus):
    import ctypes

    import so_equivariant_graph_amd as sea

    d = sea.make_desc(n_atoms=w.n_atoms, n_targets=w.n_atoms, l_max=w.l_max, channels=w.channels, heads=w.heads,
                      n_rbf=w.n_rbf, envelope_p=w.envelope_p, cutoff=w.cutoff, flags=0,
                      dtype=sea.SO2_BF16 if w.dtype == "bf16" else sea.SO2_FP32)
    v = sea.AttnVariant(m_max, n_focus)
    return sea.load_library().so2_attention_variant_kernel_kind(ctypes.byref(d), ctypes.byref(v))


@pytest.mark.parametrize("m_max,n_focus,logit", [(1, 1, False), (0, 1, False), (-1, 2, False), (-1, 1, True),
                                                 (1, 4, True)])
def test_fp32_variants_every_atom(m_max, n_focus, logit):
    w = make_workload("tiny_fp32")
    assert _run(w, m_max, n_focus, logit) <= TOL["fp32"]


def test_fp32_many_heads_and_focus_streams():
    # C = 256 with 128 heads and 128 focus streams of 2 channels: the
    # statistics and the cross-focus softmax run over more than 64 entries
    w = make_workload("tiny_fp32", l_max=1, channels=256, heads=128)
    assert _run(w, 1, 128, True) <= TOL["fp32"]


def test_bf16_logit_bias_on_the_mfma_kernel():
    import so_equivariant_graph_amd as sea

    w = make_workload("small_molecules", geometry=dict(n_molecules=4))
    assert _kind(w, -1, 1) == sea.KERNEL_MFMA
    assert _run(w, logit=True) <= TOL["bf16"]


def test_bf16_logit_bias_l6_water_sampled():
    w = make_workload("water_l6")
    t = np.sort(np.random.default_rng(1).choice(w.n_atoms, 48, replace=False))
    assert _run(w, logit=True, targets=t) <= TOL["bf16"]


@pytest.mark.parametrize("n_focus,logit", [(2, False), (4, True), (8, False), (8, True)])
def test_bf16_focus_streams_on_the_mfma_kernel(n_focus, logit):
    import so_equivariant_graph_amd as sea

    w = make_workload("small_molecules", geometry=dict(n_molecules=3))
    assert _kind(w, -1, n_focus) == sea.KERNEL_MFMA
    assert _run(w, -1, n_focus, logit=logit) <= TOL["bf16"]


@pytest.mark.parametrize("L", [1, 2, 3])
def test_bf16_focus_streams_mfma_every_degree(L):
    import so_equivariant_graph_amd as sea

    w = make_workload("tiny_fp32", l_max=L, channels=128, heads=8, n_rbf=16, dtype="bf16")
    assert _kind(w, -1, 4) == sea.KERNEL_MFMA
    assert _run(w, -1, 4, logit=True) <= TOL["bf16"]


def test_bf16_focus_streams_mfma_water_sampled():
    import so_equivariant_graph_amd as sea

    w = make_workload("water_100k", geometry=dict(n_atoms=20000))
    assert _kind(w, -1, 4) == sea.KERNEL_MFMA
    t = np.sort(np.random.default_rng(3).choice(w.n_atoms, 48, replace=False))
    assert _run(w, -1, 4, logit=True, targets=t) <= TOL["bf16"]


@pytest.mark.parametrize("m_max,n_focus", [(3, 2), (0, 2), (-1, 16)])
def test_bf16_c128_focus_streams_on_the_batch_path(m_max, n_focus):
    import so_equivariant_graph_amd as sea

    w = make_workload("small_molecules", geometry=dict(n_molecules=2))
    assert _kind(w, m_max, n_focus) == sea.KERNEL_BATCH
    assert _run(w, m_max, n_focus, logit=True) <= 1e-4


@pytest.mark.parametrize("m_max,logit", [(0, False), (1, True), (2, False), (3, True)])
def test_bf16_truncated_orders_on_the_mfma_kernel(m_max, logit):
    import so_equivariant_graph_amd as sea

    w = make_workload("small_molecules", geometry=dict(n_molecules=3))
    assert _kind(w, m_max, 1) == sea.KERNEL_MFMA
    assert _run(w, m_max, 1, logit=logit) <= TOL["bf16"]


@pytest.mark.parametrize("L", [1, 2, 3, 5, 6])
def test_bf16_truncated_orders_every_degree(L):
    # m_max = L - 1 and m_max = 0 on the MFMA kernel of every degree (the
    # 32-edge chunks of L = 5, 6 included)
    import so_equivariant_graph_amd as sea

    w = make_workload("tiny_fp32", l_max=L, channels=128, heads=8, n_rbf=16, dtype="bf16")
    for mm in sorted({L - 1, 0}):
        assert _kind(w, mm, 1) == sea.KERNEL_MFMA
        assert _run(w, mm, 1, logit=mm == 0) <= TOL["bf16"]


def test_bf16_truncated_orders_l6_water_sampled():
    w = make_workload("water_l6")
    t = np.sort(np.random.default_rng(2).choice(w.n_atoms, 48, replace=False))
    for mm in (2, 4):
        assert _run(w, mm, 1, logit=True, targets=t) <= TOL["bf16"]


def test_base_variant_is_the_base_call():
    import torch

    import so_equivariant_graph_amd as sea

    w = make_workload("small_molecules", geometry=dict(n_molecules=3))
    d = device_inputs(w)
    rp, col = neighbors_bruteforce(w.pos, w.cutoff, w.box, w.mol_id)
    rp_d, col_d = csr_to_device(rp, col)
    kw = dict(l_max=w.l_max, heads=w.heads, cutoff=w.cutoff, envelope_p=w.envelope_p, box=w.box)
    a = sea.so2_attention_fwd(d["pos"], rp_d, col_d, d["x"], d["w_q"], d["w_k"], d["w_rad"], d["w_so2"], **kw)
    b = sea.so2_attention_fwd_variant(d["pos"], rp_d, col_d, d["x"], d["w_q"], d["w_k"], d["w_rad"], d["w_so2"],
                                      m_max=w.l_max, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("cutoff,batches,m_max,n_focus,logit", [(6.0, 2, -1, 1, False), (7.5, 3, 1, 2, True)])
def test_fp32_edge_batches(cutoff, batches, m_max, n_focus, logit):
    w = make_workload("water_l6", l_max=2, channels=16, heads=2, n_rbf=8, dtype="fp32", cutoff=cutoff)
    nt = 64  # batch capacity max(4096, 64 nt) = 4096 edges
    rp, _ = neighbors_bruteforce(w.pos, w.cutoff, w.box, w.mol_id)
    n_edges = int(rp[nt] - rp[0])
    assert (batches - 1) * 4096 < n_edges <= batches * 4096, n_edges
    assert _run(w, m_max, n_focus, logit, n_targets=nt) <= TOL["fp32"]


def test_batch_path_repeats_bitwise():
    import torch

    w = make_workload("tiny_fp32")
    outs = []
    _run(w, 1, 2, True, out=outs)
    _run(w, 1, 2, True, out=outs)
    assert torch.equal(outs[0], outs[1])
