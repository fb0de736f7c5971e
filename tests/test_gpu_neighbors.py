"""Neighbour-list parity on the GPU: the cell-list CSR from build_neighbors
must equal the brute-force oracle bit for bit (whole graph where the oracle
is quick, seeded sampled rows plus whole-graph properties at 100k atoms),
and the adversarial cases the exact fp64 test has to get right."""

import numpy as np
import pytest

from helpers import say
from oracle import neighbors_bruteforce
from synth import make_workload

pytestmark = pytest.mark.gpu


def _gpu_csr(pos, cutoff, box=None, mol=None, capacity=None):
    import torch

    import so_equivariant_graph_amd as sea

    p = torch.from_numpy(np.ascontiguousarray(pos, dtype=np.float32)).cuda()
    m = None if mol is None else torch.from_numpy(np.asarray(mol, dtype=np.int32)).cuda()
    rp, col = sea.build_neighbors(p, cutoff, box=box, mol_id=m, capacity=capacity)
    torch.cuda.synchronize()
    return rp.cpu().numpy(), col.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny_fp32", "small_molecules", "water_l6", "solvated_protein"])
def test_workload_graph_bit_exact(name):
    say("neighbors full", name)
    w = make_workload(name, with_features=False)
    rp, col = _gpu_csr(w.pos, w.cutoff, w.box, w.mol_id)
    rp_ref, col_ref = neighbors_bruteforce(w.pos, w.cutoff, w.box, w.mol_id)
    assert np.array_equal(rp, rp_ref)
    assert np.array_equal(col, col_ref)


def test_water_100k_sampled_rows_and_properties():
    say("neighbors water_100k sampled")
    w = make_workload("water_100k", with_features=False)
    rp, col = _gpu_csr(w.pos, w.cutoff, w.box)
    n = w.n_atoms
    assert rp[0] == 0 and rp[-1] == col.size and np.all(np.diff(rp) >= 0)
    rows = np.random.default_rng(0).choice(n, size=384, replace=False)
    rows = np.concatenate([rows, [0, n - 1]])
    ref = neighbors_bruteforce(w.pos, w.cutoff, w.box, rows=rows)
    for i, r in zip(rows, ref):
        assert np.array_equal(col[rp[i] : rp[i + 1]], r), i
    # whole graph: sorted rows, no self pairs, symmetric
    deg = np.diff(rp)
    owner = np.repeat(np.arange(n), deg)
    assert np.all(col != owner)
    same = owner[1:] == owner[:-1]
    assert np.all(col[1:][same] > col[:-1][same])
    fwd = owner.astype(np.int64) * n + col
    bwd = col.astype(np.int64) * n + owner
    assert np.array_equal(np.sort(fwd), np.sort(bwd))


def test_cutoff_boundary_and_cell_faces():
    say("neighbors boundary")
    rc = np.float32(2.5)
    inside = np.nextafter(np.float32(2.5), np.float32(0))
    pts = [[0, 0, 0], [2.5, 0, 0], [0, inside, 0], [0, 0, -2.5], [5.0, 5.0, 5.0], [7.5, 5.0, 5.0]]
    # atoms on exact multiples of the cell size, and duplicates
    g = np.arange(0.0, 12.6, 2.5)
    grid = np.stack(np.meshgrid(g, g, g, indexing="ij"), -1).reshape(-1, 3)
    pos = np.vstack([pts, grid, grid[:5]]).astype(np.float32)
    rp, col = _gpu_csr(pos, rc)
    rp_ref, col_ref = neighbors_bruteforce(pos, rc)
    assert np.array_equal(rp, rp_ref) and np.array_equal(col, col_ref)


@pytest.mark.parametrize("side", [5.05, 7.4, 12.0, 40.0])
def test_periodic_small_and_large_boxes(side):
    say("neighbors periodic side", side)
    rng = np.random.default_rng(int(side * 10))
    rc = 2.5
    box = np.array([side, side * 1.07, side * 0.93], dtype=np.float32)
    box = np.maximum(box, 2 * rc + 0.01).astype(np.float32)
    n = 600
    pos = rng.uniform(-2 * side, 3 * side, size=(n, 3)).astype(np.float32)
    # pairs at exactly half a box apart (rint ties) and on the box faces
    pos[:4] = [[0, 0, 0], [box[0] / 2, 0, 0], [-box[0] / 2, 0, 0], [box[0], box[1], box[2]]]
    rp, col = _gpu_csr(pos, rc, box)
    rp_ref, col_ref = neighbors_bruteforce(pos, rc, box)
    assert np.array_equal(rp, rp_ref) and np.array_equal(col, col_ref)


def test_open_boundaries_spread_out_and_molecules():
    say("neighbors sparse open")
    rng = np.random.default_rng(3)
    pos = np.vstack([rng.uniform(-1000, 1000, size=(300, 3)), rng.uniform(0, 6, size=(300, 3))]).astype(np.float32)
    mol = (np.arange(600) // 7).astype(np.int32)
    for m in (None, mol):
        rp, col = _gpu_csr(pos, 3.0, None, m)
        rp_ref, col_ref = neighbors_bruteforce(pos, 3.0, None, m)
        assert np.array_equal(rp, rp_ref) and np.array_equal(col, col_ref)


def test_single_atom_and_coincident_atoms():
    say("neighbors degenerate")
    rp, col = _gpu_csr(np.zeros((1, 3), np.float32), 1.0)
    assert list(rp) == [0, 0] and col.size == 0
    pos = np.zeros((5, 3), np.float32)
    rp, col = _gpu_csr(pos, 1.0)
    rp_ref, col_ref = neighbors_bruteforce(pos, 1.0)
    assert np.array_equal(rp, rp_ref) and np.array_equal(col, col_ref)


def test_long_rows_are_sorted():
    say("neighbors long rows")
    rng = np.random.default_rng(4)
    v = rng.standard_normal((1500, 3))
    pos = (v / np.linalg.norm(v, axis=1)[:, None] * rng.uniform(0, 1.0, size=(1500, 1))).astype(np.float32)
    pos = np.vstack([pos, rng.uniform(10, 30, size=(200, 3)).astype(np.float32)])
    rp, col = _gpu_csr(pos, 2.5)
    assert np.diff(rp).max() > 1024
    rp_ref, col_ref = neighbors_bruteforce(pos, 2.5)
    assert np.array_equal(rp, rp_ref) and np.array_equal(col, col_ref)


def test_capacity_error_reports_required_size():
    say("neighbors capacity")
    import so_equivariant_graph_amd as sea

    w = make_workload("tiny_fp32", with_features=False)
    with pytest.raises(sea.SO2Error) as ei:
        _gpu_csr_capacity_once(w.pos, w.cutoff, capacity=10)
    assert ei.value.status == sea.SO2_ERR_CAPACITY
    rp, col = _gpu_csr(w.pos, w.cutoff, capacity=10)  # the binding retries with the reported size
    rp_ref, col_ref = neighbors_bruteforce(w.pos, w.cutoff)
    assert np.array_equal(col, col_ref)


def _gpu_csr_capacity_once(pos, cutoff, capacity):
    import ctypes

    import torch

    import so_equivariant_graph_amd as sea

    lib = sea.load_library()
    p = torch.from_numpy(np.ascontiguousarray(pos)).cuda()
    n = p.shape[0]
    ws = torch.empty(lib.so2_neighbors_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    rp = torch.empty(n + 1, dtype=torch.int32, device="cuda")
    col = torch.empty(capacity, dtype=torch.int32, device="cuda")
    ne = ctypes.c_int64(0)
    st = lib.build_neighbors(
        ctypes.c_void_p(p.data_ptr()), n, None, None, ctypes.c_float(cutoff), ctypes.c_void_p(rp.data_ptr()),
        ctypes.c_void_p(col.data_ptr()), capacity, ctypes.byref(ne), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
        sea._stream_handle(p.device),
    )
    torch.cuda.synchronize()
    rp_ref, col_ref = neighbors_bruteforce(pos, cutoff)
    assert ne.value == col_ref.size
    assert np.array_equal(rp.cpu().numpy(), rp_ref)
    sea._check(st, "build_neighbors")


def test_non_finite_position_is_rejected():
    say("neighbors non-finite")
    import so_equivariant_graph_amd as sea

    pos = np.zeros((10, 3), np.float32)
    pos[3, 1] = np.nan
    with pytest.raises(sea.SO2Error) as ei:
        _gpu_csr(pos, 1.0)
    assert ei.value.status == sea.SO2_ERR_INVALID_ARGUMENT
