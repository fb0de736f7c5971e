"""so2_attention_fwd_noalloc against so2_attention_fwd, through the C ABI:
the variant that keeps its workspace in the library's own device array
must give the same outputs as the entry point with a caller workspace, on
two calls in a row (the second on a smaller input, so stale scratch from the
first call would show), and refuse a size past the array's limit without
launching anything."""

import ctypes

import numpy as np
import pytest

from helpers import csr_to_device, device_inputs, say
from oracle import max_rel_error, neighbors_bruteforce
from synth import make_workload

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 128 << 20  # SO2_NOALLOC_SCRATCH_BYTES


def _desc(w, n_targets=None):
    import so_equivariant_graph_amd as sea

    return sea.make_desc(
        n_atoms=w.n_atoms, n_targets=w.n_atoms if n_targets is None else n_targets, l_max=w.l_max,
        channels=w.channels, heads=w.heads, n_rbf=w.n_rbf, envelope_p=w.envelope_p, cutoff=w.cutoff, flags=0,
        dtype=sea.SO2_BF16 if w.dtype == "bf16" else sea.SO2_FP32,
    )


def _call(w, d, rp, col, y, noalloc, n_targets=None):
    import torch

    import so_equivariant_graph_amd as sea

    lib = sea.load_library()
    desc = _desc(w, n_targets)
    keep, box_p = sea._host_box(w.box)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [sea._ptr(d["pos"]), box_p, sea._ptr(rp), sea._ptr(col), sea._ptr(d["x"]), sea._ptr(d["w_q"]),
            sea._ptr(d["w_k"]), sea._ptr(d["w_rad"]), sea._ptr(d["w_so2"]), sea._ptr(y)]
    if noalloc:
        return lib.so2_attention_fwd_noalloc(ctypes.byref(desc), *args, stream)
    ws_bytes = lib.so2_attention_workspace_bytes(ctypes.byref(desc))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    st = lib.so2_attention_fwd(ctypes.byref(desc), *args, sea._ptr(ws), ws_bytes, stream)
    torch.cuda.synchronize()
    return st


def _case(w, n_targets=None):
    import torch

    import so_equivariant_graph_amd as sea

    d = device_inputs(w)
    rp, col = neighbors_bruteforce(w.pos, w.cutoff, w.box, w.mol_id)
    rp_d, col_d = csr_to_device(rp, col)
    nt = w.n_atoms if n_targets is None else n_targets
    shape = (nt, (w.l_max + 1) ** 2, w.channels)
    y_ref = torch.full(shape, float("nan"), device="cuda")
    y_na = torch.full(shape, float("nan"), device="cuda")
    assert _call(w, d, rp_d, col_d, y_ref, False, n_targets) == sea.SO2_OK
    assert _call(w, d, rp_d, col_d, y_na, True, n_targets) == sea.SO2_OK
    torch.cuda.synchronize()
    a, b = y_na.cpu().numpy(), y_ref.cpu().numpy()
    assert np.all(np.isfinite(a))
    return max_rel_error(a, b), bool(np.array_equal(a, b))


@pytest.mark.parametrize("kind", ["bf16", "fp32"])
def test_noalloc_matches_the_workspace_entry_point_twice(kind):
    import so_equivariant_graph_amd as sea

    if kind == "bf16":
        first = make_workload("small_molecules", geometry=dict(n_molecules=48))
        second = make_workload("small_molecules", geometry=dict(n_molecules=5), seed=9)
    else:
        first = make_workload("tiny_fp32")
        second = make_workload("tiny_fp32", geometry=dict(n_atoms=40), seed=3)
    assert second.n_atoms < first.n_atoms
    for w in (first, second):
        need = sea.attention_workspace_bytes(_desc(w))
        assert 0 < need <= SCRATCH_BYTES
        say("noalloc", kind, "atoms", w.n_atoms, "workspace", need)
        err, same = _case(w)
        say("noalloc vs workspace entry point: max rel err", err, "bitwise", same)
        assert err <= (2e-2 if kind == "bf16" else 1e-4)
    # partial targets on the smaller input
    err, _ = _case(second, n_targets=second.n_atoms // 2)
    assert err <= (2e-2 if kind == "bf16" else 1e-4)


def test_noalloc_refuses_inputs_past_its_scratch():
    import so_equivariant_graph_amd as sea

    lib = sea.load_library()
    w = make_workload("water_100k", with_features=False)
    desc = _desc(w)
    assert lib.so2_attention_workspace_bytes(ctypes.byref(desc)) > SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 30)  # never touched: the size check comes first
    args = [fake, ctypes.c_void_p(0)] + [fake] * 8  # pos, box (open), row_ptr .. y
    st = lib.so2_attention_fwd_noalloc(ctypes.byref(desc), *args, ctypes.c_void_p(0))
    assert st == sea.SO2_ERR_WORKSPACE
