"""Forward parity on the GPU: so2_attention_fwd (through the C ABI) against
the fp64 oracle, element by element.

* tiny_fp32: every atom, max relative error (normalised per atom) <= 1e-4;
* bf16 workloads: a small batch of the same kind (several kernel tiles and a
  ragged tail) on every atom at <= 2e-2 (the oracle gets the same
  bf16-rounded inputs); the full-size workloads are in
  test_gpu_x_full_parity.py;
* edges just inside the cutoff, where the envelope is a few 1e-9 and
  decides the softmax;
* edge cases: empty neighbourhoods, n_targets < n_atoms, L = 0 and L = 6,
  odd channel counts, both flags;
* GPU-side invariants: softmax weights summing to one, rotation
  equivariance, bitwise determinism of repeated calls."""

import numpy as np
import pytest

from helpers import TOL, csr_to_device, device_inputs, gpu_attention, oracle_attention, say
from oracle import max_rel_error, neighbors_bruteforce, so2_weight_count, wigner_d_blocks
from synth import make_workload

pytestmark = pytest.mark.gpu


def _run_pair(w, targets=None, use_gpu_graph=False, **kw):
    import torch

    import so_equivariant_graph_amd as sea

    d = device_inputs(w)
    rp, col = neighbors_bruteforce(w.pos, w.cutoff, w.box, w.mol_id)
    if use_gpu_graph:
        rp_d, col_d = sea.build_neighbors(d["pos"], w.cutoff, box=w.box, mol_id=d["mol"])
    else:
        rp_d, col_d = csr_to_device(rp, col)
    y = gpu_attention(w, d, rp_d, col_d, **kw)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    t = np.arange(w.n_atoms) if targets is None else np.asarray(targets)
    y_ref = oracle_attention(w, rp, col, targets=t, **kw)
    return y[t], y_ref


def test_tiny_fp32_every_atom():
    say("attention tiny_fp32 full")
    w = make_workload("tiny_fp32")
    y, y_ref = _run_pair(w, use_gpu_graph=True)
    err = max_rel_error(y, y_ref)
    say("max rel err", err)
    assert err <= TOL["fp32"]


@pytest.mark.parametrize("flags", [1, 2])
def test_tiny_fp32_flags(flags):
    say("attention tiny flags", flags)
    w = make_workload("tiny_fp32")
    y, y_ref = _run_pair(w, flags=flags)
    assert max_rel_error(y, y_ref) <= TOL["fp32"]


def test_small_molecules_batch_every_atom_bf16():
    say("attention small_molecules batch of 4")
    w = make_workload("small_molecules", geometry=dict(n_molecules=4))
    y, y_ref = _run_pair(w, use_gpu_graph=True)
    err = max_rel_error(y, y_ref)
    say("max rel err", err)
    assert err <= TOL["bf16"]


def test_empty_neighbourhood_and_partial_targets():
    say("attention empty rows, n_targets < n_atoms")
    w = make_workload("tiny_fp32")
    w.pos[5] = [500.0, 500.0, 500.0]  # isolated atom
    y, y_ref = _run_pair(w)
    assert np.all(y[5] == 0.0)
    assert max_rel_error(y, y_ref) <= TOL["fp32"]
    import torch

    d = device_inputs(w)
    rp, col = neighbors_bruteforce(w.pos, w.cutoff)
    rp_d, col_d = csr_to_device(rp, col)
    y_part = gpu_attention(w, d, rp_d, col_d, n_targets=17)
    torch.cuda.synchronize()
    assert y_part.shape[0] == 17
    assert max_rel_error(y_part.cpu().numpy(), y_ref[:17]) <= TOL["fp32"]


@pytest.mark.parametrize("L,C,H,dtype", [(0, 8, 2, "fp32"), (6, 8, 1, "fp32"), (3, 3, 3, "fp32"), (2, 16, 4, "bf16")])
def test_shapes(L, C, H, dtype):
    say("attention shape", L, C, H, dtype)
    w = make_workload("tiny_fp32", l_max=L, channels=C, heads=H, dtype=dtype)
    y, y_ref = _run_pair(w)
    assert max_rel_error(y, y_ref) <= TOL[dtype]


def test_softmax_weights_sum_to_one_on_gpu():
    say("attention softmax sum trick")
    import torch

    w = make_workload("small_molecules", geometry=dict(n_molecules=3), dtype="bf16")
    L, C = w.l_max, w.channels
    w.x[:] = 0.0
    w.x[:, 0, :] = 1.0
    blocks = [np.eye((L + 1) * C).ravel()]
    for m in range(1, L + 1):
        km = (L + 1 - m) * C
        blocks += [np.eye(km).ravel(), np.zeros(km * km)]
    w.w_so2 = np.concatenate(blocks).astype(np.float32)
    assert w.w_so2.size == so2_weight_count(L, C)
    d = device_inputs(w)
    rp, col = neighbors_bruteforce(w.pos, w.cutoff, w.box, w.mol_id)
    rp_d, col_d = csr_to_device(rp, col)
    y = gpu_attention(w, d, rp_d, col_d, flags=2)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    has = np.diff(rp) > 0
    np.testing.assert_allclose(y[has, 0, :], 1.0, atol=2e-2)
    assert np.abs(y[has, 1:, :]).max() < 2e-2


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_rotation_equivariance_on_gpu(dtype):
    say("attention equivariance", dtype)
    import torch
    from scipy.spatial.transform import Rotation

    from synth import to_bf16_exact

    w = make_workload("tiny_fp32", l_max=3, channels=16, heads=2, dtype=dtype)
    R = Rotation.random(random_state=11).as_matrix()
    D = wigner_d_blocks(w.l_max, R)

    def rot(feat):
        out = np.empty_like(feat)
        for l in range(w.l_max + 1):
            sl = slice(l * l, (l + 1) ** 2)
            out[:, sl, :] = np.einsum("ab,nbc->nac", D[l], feat[:, sl, :])
        return out

    def run(pos, x):
        w2 = make_workload("tiny_fp32", l_max=3, channels=16, heads=2, dtype=dtype)
        w2.pos, w2.x = pos.astype(np.float32), x.astype(np.float32)
        d = device_inputs(w2)
        rp, col = neighbors_bruteforce(w2.pos, w2.cutoff)
        y = gpu_attention(w2, d, *csr_to_device(rp, col))
        torch.cuda.synchronize()
        return y.cpu().numpy().astype(np.float64)

    c = w.pos.mean(0)
    x_r = rot(w.x)
    if dtype == "bf16":
        x_r = to_bf16_exact(x_r.astype(np.float32))
    y = run(w.pos, w.x)
    y_r = run((w.pos - c) @ R.T + c, x_r)
    assert max_rel_error(y_r, rot(y)) <= TOL[dtype]


def test_repeated_calls_are_bitwise_identical():
    say("attention determinism")
    import torch

    w = make_workload("small_molecules", geometry=dict(n_molecules=3))
    d = device_inputs(w)
    rp, col = neighbors_bruteforce(w.pos, w.cutoff, w.box, w.mol_id)
    rp_d, col_d = csr_to_device(rp, col)
    a = gpu_attention(w, d, rp_d, col_d).clone()
    b = gpu_attention(w, d, rp_d, col_d)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---------------------------------------------------------------- bf16 MFMA kernel


def _kind(w):
    import so_equivariant_graph_amd as sea

    d = sea.make_desc(n_atoms=w.n_atoms, n_targets=w.n_atoms, l_max=w.l_max,
                      channels=w.channels, heads=w.heads, n_rbf=w.n_rbf, envelope_p=w.envelope_p,
                      cutoff=w.cutoff, flags=0, dtype=sea.SO2_BF16 if w.dtype == "bf16" else sea.SO2_FP32)
    return sea.attention_kernel_kind(d)


@pytest.mark.parametrize("name", ["small_molecules", "water_l6", "solvated_protein", "water_100k"])
def test_bf16_workloads_run_on_the_mfma_kernel(name):
    import so_equivariant_graph_amd as sea

    w = make_workload(name, with_features=False)
    assert _kind(w) == sea.KERNEL_MFMA


@pytest.mark.parametrize("L", [1, 2, 3, 4, 5, 6])
def test_mfma_every_degree(L):
    say("mfma L", L)
    import so_equivariant_graph_amd as sea

    w = make_workload("tiny_fp32", l_max=L, channels=128, heads=8, n_rbf=16, dtype="bf16")
    assert _kind(w) == sea.KERNEL_MFMA
    y, y_ref = _run_pair(w)
    err = max_rel_error(y, y_ref)
    say("max rel err", err)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("L,K", [(1, 8), (2, 8), (2, 12), (2, 24), (3, 8), (3, 20), (5, 8), (6, 24)])
def test_mfma_degree_and_rbf_counts(L, K):
    """Degrees below 4 leave some of the five component-pair slots of a lane
    unused and basis counts other than 16 change the gate and rotation data
    next to the Wigner-D rows (32-edge chunks for L = 5, 6): every output
    must stay finite and match."""
    say("mfma L", L, "n_rbf", K)
    w = make_workload("tiny_fp32", l_max=L, channels=128, heads=8, n_rbf=K, dtype="bf16")
    y, y_ref = _run_pair(w)
    assert np.isfinite(y).all()
    err = max_rel_error(y, y_ref)
    say("max rel err", err)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("heads", [1, 4, 16])
def test_mfma_head_counts(heads):
    say("mfma heads", heads)
    w = make_workload("tiny_fp32", l_max=2, channels=128, heads=heads, n_rbf=8, dtype="bf16")
    y, y_ref = _run_pair(w)
    assert max_rel_error(y, y_ref) <= TOL["bf16"]


@pytest.mark.parametrize("flags", [1, 2])
def test_mfma_flags(flags):
    say("mfma flags", flags)
    w = make_workload("small_molecules", geometry=dict(n_molecules=2))
    y, y_ref = _run_pair(w, flags=flags)
    assert max_rel_error(y, y_ref) <= TOL["bf16"]


@pytest.mark.parametrize("L", [4, 6])
def test_mfma_ragged_degrees_and_split_targets(L):
    """Degrees 0, 1, 2 and > 64 (one target spanning several 64- or 32-edge
    chunks), a target count that is not a multiple of the 16-target group,
    and n_targets < n_atoms."""
    say("mfma ragged degrees, L", L)
    import torch

    rng = np.random.default_rng(7)
    chunk = 64 if L <= 4 else 32
    # a dense cluster: neighbours within rc = 5 well above one chunk per target
    dense = rng.uniform(0, 4.0, size=(90 if L <= 4 else 50, 3))
    sparse = np.array([[50, 0, 0], [53, 0, 0], [50, 4, 0], [80, 0, 0], [90, 0, 0], [93.5, 0, 0], [150, 0, 0]], float)
    pos = np.vstack([dense, sparse, rng.uniform(200, 210, size=(40, 3))])
    w = make_workload("tiny_fp32", l_max=L, channels=128, heads=8, n_rbf=16, dtype="bf16")
    from synth import to_bf16_exact

    n = pos.shape[0]
    w.pos = pos.astype(np.float32)
    w.x = to_bf16_exact(rng.standard_normal((n, (L + 1) ** 2, 128)).astype(np.float32))
    rp, col = neighbors_bruteforce(w.pos, w.cutoff)
    deg = np.diff(rp)
    assert deg.max() > chunk and (deg == 0).any() and (deg == 1).any()
    y, y_ref = _run_pair(w)
    err = max_rel_error(y, y_ref)
    say("max rel err", err, "max deg", deg.max())
    assert err <= TOL["bf16"]
    assert np.all(y[deg == 0] == 0.0)
    d = device_inputs(w)
    nt = n - 36  # 101 (L = 4) or 61 (L = 6) targets, not a multiple of 16
    y_part = gpu_attention(w, d, *csr_to_device(rp, col), n_targets=nt)
    torch.cuda.synchronize()
    assert y_part.shape[0] == nt
    assert max_rel_error(y_part.cpu().numpy(), y_ref[:nt]) <= TOL["bf16"]


def test_mfma_hub_target_keeps_estimated_runs():
    """One target with 250 neighbours (4 chunks of 64 edges) among
    300 targets of degree 19: the chunk cap one below the largest estimated
    run cannot hold the hub, so the estimated runs stay; every target is
    checked against the oracle."""
    say("mfma hub target")
    from synth import to_bf16_exact

    rng = np.random.default_rng(11)
    g = np.arange(-4, 5) * 1.2
    lat = np.array(np.meshgrid(g, g, g, indexing="ij")).reshape(3, -1).T
    shell = lat[(np.linalg.norm(lat, axis=1) > 0) & (np.linalg.norm(lat, axis=1) < 4.8)]
    cube = np.array(np.meshgrid(*(np.arange(3) * 1.2,) * 3, indexing="ij")).reshape(3, -1).T[:20]
    groups = [cube + [100.0 + 30.0 * k, 0.0, 0.0] for k in range(15)]
    pos = np.vstack([[[0.0, 0.0, 0.0]], *groups, shell])
    nt = 1 + 15 * 20
    n = pos.shape[0]
    w = make_workload("tiny_fp32", l_max=2, channels=128, heads=8, n_rbf=16, dtype="bf16")
    w.pos = pos.astype(np.float32)
    w.x = to_bf16_exact(rng.standard_normal((n, 9, 128)).astype(np.float32))
    rp, col = neighbors_bruteforce(w.pos, w.cutoff)
    deg = np.diff(rp)
    assert deg[0] > 3 * 64 and np.all(deg[1:nt] == 19)
    import torch

    d = device_inputs(w)
    y = gpu_attention(w, d, *csr_to_device(rp, col), n_targets=nt)
    torch.cuda.synchronize()
    y_ref = oracle_attention(w, rp, col, targets=np.arange(nt))
    err = max_rel_error(y.cpu().numpy(), y_ref)
    say("max rel err", err, "hub degree", deg[0])
    assert err <= TOL["bf16"]


def test_mfma_exact_schedule_with_isolated_targets():
    """96 small molecules with 1923 isolated atoms mixed into the index order
    (5769 targets, a third without neighbours): the run schedule takes the
    exact refinement (a cap of 8 chunks, 229 runs), with runs that start and
    end next to targets without neighbours.  Every row is compared with the
    fp32 VALU kernel on the same bf16-exact inputs (one workgroup per target,
    no run schedule), and 40 seeded targets with the oracle."""
    import copy

    import torch

    from synth import to_bf16_exact

    say("mfma exact schedule, isolated targets mixed in")
    w = make_workload("small_molecules", geometry=dict(n_molecules=96))
    rng = np.random.default_rng(3)
    n0 = w.n_atoms
    n_iso = n0 // 2
    iso = np.stack([np.full(n_iso, -500.0), np.arange(n_iso) * 20.0, np.zeros(n_iso)], 1)
    perm = rng.permutation(n0 + n_iso)
    w.pos = np.vstack([w.pos, iso])[perm].astype(np.float32)
    w.mol_id = np.concatenate([w.mol_id, 100000 + np.arange(n_iso)])[perm].astype(np.int32)
    x_iso = to_bf16_exact(rng.standard_normal((n_iso,) + w.x.shape[1:]).astype(np.float32))
    w.x = np.concatenate([w.x, x_iso])[perm]
    rp, col = neighbors_bruteforce(w.pos, w.cutoff, w.box, w.mol_id)
    deg = np.diff(rp)
    assert (deg == 0).sum() > w.n_atoms // 4
    y = gpu_attention(w, device_inputs(w), *csr_to_device(rp, col))
    w32 = copy.copy(w)
    w32.dtype = "fp32"
    y32 = gpu_attention(w32, device_inputs(w32), *csr_to_device(rp, col))
    torch.cuda.synchronize()
    y, y32 = y.cpu().numpy(), y32.cpu().numpy()
    assert np.all(np.isfinite(y)) and np.all(y[deg == 0] == 0.0)
    err_all = max_rel_error(y, y32)
    t = np.sort(rng.choice(w.n_atoms, size=40, replace=False))
    err_ref = max_rel_error(y[t], oracle_attention(w, rp, col, targets=t))
    say("vs fp32 kernel", err_all, "vs oracle", err_ref)
    assert err_all <= TOL["bf16"] and err_ref <= TOL["bf16"]


def _near_cutoff_system(L, C, H, K, dtype, seed=5):
    """Groups far apart: in each, a target with one or two neighbours at
    distance rc (1 - delta), delta in [1e-5, 1e-3] (the pair of neighbours on
    opposite sides, 2 rc apart), so every atom of a group sees only edges
    whose envelope is 1e-15..1e-7; plus a small uniform cluster of ordinary
    atoms, so that chunks mix both kinds of edges."""
    from synth import to_bf16_exact

    w = make_workload("tiny_fp32", l_max=L, channels=C, heads=H, n_rbf=K, dtype=dtype)
    rng = np.random.default_rng(seed)
    rc = w.cutoff
    pos = [w.pos[:24].astype(np.float64)]
    deltas = np.geomspace(1e-5, 1e-3, 12)
    for g, delta in enumerate(deltas):
        # group centres 16 A apart (> 3 rc: atoms of different groups are more
        # than rc apart), coordinates
        # below 80 A so that fp32 positions move a distance by < 1e-5 A
        c = np.array([30.0 + 16.0 * (g % 3), 16.0 * ((g // 3) % 2), 16.0 * (g // 6)])
        u = rng.standard_normal(3)
        u /= np.linalg.norm(u)
        r = rc * (1.0 - delta)
        group = [c, c + r * u]
        if g % 2 == 0:
            group.append(c - r * u)
        pos.append(np.array(group))
    w.pos = np.vstack(pos).astype(np.float32)
    n = w.pos.shape[0]
    w.x = rng.standard_normal((n, (L + 1) ** 2, C)).astype(np.float32)
    if dtype == "bf16":
        w.x = to_bf16_exact(w.x)
    return w, deltas


@pytest.mark.parametrize("L,C,H,K,dtype", [(2, 16, 2, 8, "fp32"), (4, 128, 8, 16, "bf16"), (6, 128, 8, 16, "bf16")])
def test_neighbours_just_inside_the_cutoff(L, C, H, K, dtype):
    """Atoms whose only neighbours sit within 1e-3 rc of the cutoff: the
    envelope (about 35 (1 - s)^3 there) weighs the softmax, so an envelope
    evaluated by cancellation, or from a length rounded to fp32, would give
    weights of the wrong size or sign.  fp32 (VALU kernel) and bf16 (MFMA
    kernel at L = 4 and 6) against the oracle, every atom."""
    say("attention near-cutoff edges", L, C, dtype)
    import so_equivariant_graph_amd as sea

    w, deltas = _near_cutoff_system(L, C, H, K, dtype)
    rp, col = neighbors_bruteforce(w.pos, w.cutoff, w.box, w.mol_id)
    deg = np.diff(rp)
    far = np.arange(24, w.n_atoms)
    assert np.all(deg[far] >= 1)
    for i in far:  # every edge of a group atom is just inside the cutoff
        r = w.pos[col[rp[i] : rp[i + 1]]].astype(np.float64) - w.pos[i].astype(np.float64)
        s = np.sqrt((r * r).sum(1)) / w.cutoff
        assert np.all((s > 1 - 1.2e-3) & (s < 1.0)), (i, s)
    assert _kind(w) == (sea.KERNEL_BATCH if dtype == "fp32" else sea.KERNEL_MFMA)
    y, y_ref = _run_pair(w)
    err = max_rel_error(y, y_ref)
    err_far = max_rel_error(y[far], y_ref[far])
    say("max rel err", err, "near-cutoff atoms", err_far)
    assert np.all(np.abs(y_ref[far]).max(axis=(1, 2)) > 0)
    assert err <= TOL[dtype] and err_far <= TOL[dtype]
