"""Backward parity on the GPU: so2_attention_bwd (through the C ABI) against
the fp64 oracle's gradients (oracle/attention_grad.py), element by element,
for the node features, the positions and every weight.

Tolerance: max relative error, normalised per atom for dx and dpos (the
parity metric of the forward) and by the largest entry for the weight
gradients.  fp32 inputs take fp32 arithmetic and the fp32 bound, 1e-4.
bf16 inputs run the per-m maps on bf16 matrix-core operands (each fp32
operand split into two bf16 parts, fp32 accumulation) and take the bf16
bound, 2e-2; the measured errors are 5e-6 to 3e-4 (plain bf16 operands,
without the split, reach 0.36 on the position gradient of the multi-batch
case).  Cases: the tiny fp32 workload (every atom, both flags),
a small periodic water box, a bf16 batch at L = 4, C = 128, bf16 inputs at
C = 16 and 48 (partial GEMM tiles in every dimension), L = 6, 128
heads at C = 256, empty
neighbourhoods with n_targets < n_atoms, targets whose edges take two and
three batches (64 edges per target, at least 4096: the second pass then
recomputes every batch but the last of the first); on the GPU's own output,
forces that sum to zero and rotate with the system."""

import numpy as np
import pytest

from helpers import csr_to_device, device_inputs, say
from oracle import max_rel_error, neighbors_bruteforce, so2_attention_grad_ref, wigner_d_blocks
from synth import make_workload

pytestmark = pytest.mark.gpu

TOL = 1e-4
TOL_BF16 = 2e-2


def _gpu(w, rp, col, dy, n_targets=None, flags=0, weights=True):
    import torch

    import so_equivariant_graph_amd as sea

    d = device_inputs(w)
    rp_d, col_d = csr_to_device(rp, col)
    g = sea.so2_attention_bwd(
        d["pos"], rp_d, col_d, d["x"], d["w_q"], d["w_k"], d["w_rad"], d["w_so2"],
        torch.from_numpy(np.ascontiguousarray(dy, dtype=np.float32)).cuda(), l_max=w.l_max, heads=w.heads,
        cutoff=w.cutoff, envelope_p=w.envelope_p, box=w.box, flags=flags, n_targets=n_targets, weights=weights,
    )
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().astype(np.float64) for k, v in g.items()}


def _ref(w, rp, col, dy, n_targets=None, flags=0):
    t = None if n_targets is None else range(n_targets)
    return so2_attention_grad_ref(w.pos, rp, col, w.x, w.w_q, w.w_k, w.w_rad, w.w_so2, dy, l_max=w.l_max,
                                  heads=w.heads, cutoff=w.cutoff, envelope_p=w.envelope_p, box=w.box, flags=flags,
                                  targets=t)


def _compare(g, r, weights=True):
    errs = {
        "dx": max_rel_error(g["dx"], r["dx"]),
        "dpos": max_rel_error(g["dpos"][:, None, :], r["dpos"][:, None, :]),
    }
    if weights:
        for k in ("dw_q", "dw_k", "dw_rad", "dw_so2"):
            scale = np.abs(r[k]).max()
            errs[k] = float(np.abs(g[k] - r[k]).max() / scale) if scale > 0 else float(np.abs(g[k]).max())
    say("backward max rel err", {k: f"{v:.2e}" for k, v in errs.items()})
    return errs


def _case(w, flags=0, n_targets=None, seed=0):
    rp, col = neighbors_bruteforce(w.pos, w.cutoff, w.box, w.mol_id)
    nt = w.n_atoms if n_targets is None else n_targets
    dy = np.random.default_rng(seed).standard_normal((nt,) + w.x.shape[1:]).astype(np.float32)
    g = _gpu(w, rp, col, dy, n_targets, flags)
    r = _ref(w, rp, col, dy.astype(np.float64), n_targets, flags)
    return g, r, rp, col


@pytest.mark.parametrize("flags", [0, 1, 2])
def test_tiny_fp32_every_gradient(flags):
    say("backward tiny_fp32 flags", flags)
    w = make_workload("tiny_fp32")
    g, r, _, _ = _case(w, flags)
    errs = _compare(g, r)
    if flags == 2:
        assert np.all(g["dw_rad"] == 0.0)
        errs.pop("dw_rad")
    assert max(errs.values()) <= TOL


def test_periodic_water_box():
    say("backward periodic water box, 300 atoms")
    w = make_workload("water_100k", geometry=dict(n_atoms=300), l_max=2, channels=16, heads=2, n_rbf=8, dtype="fp32")
    assert w.box is not None
    g, r, _, _ = _case(w)
    assert max(_compare(g, r).values()) <= TOL


def test_bf16_inputs_l4_c128():
    say("backward bf16 small molecules, L = 4, C = 128")
    w = make_workload("small_molecules", geometry=dict(n_molecules=2))
    assert w.dtype == "bf16" and w.channels == 128
    g, r, _, _ = _case(w)
    assert max(_compare(g, r).values()) <= TOL_BF16


@pytest.mark.parametrize("L,C,H", [(2, 16, 2), (3, 48, 4)])
def test_bf16_inputs_ragged_gemm_tiles(L, C, H):
    # bf16 inputs take the split-bf16 GEMMs; with these widths every per-m
    # block (3C, 2(L+1-m)C columns) leaves partial 128-column tiles and
    # partial 32-wide K stages, and the edge counts partial row tiles
    say("backward bf16 ragged GEMM tiles", L, C, H)
    w = make_workload("tiny_fp32", l_max=L, channels=C, heads=H, dtype="bf16")
    g, r, _, _ = _case(w, seed=5)
    assert max(_compare(g, r).values()) <= TOL_BF16


def test_l6():
    say("backward L = 6")
    w = make_workload("tiny_fp32", l_max=6, channels=8, heads=2)
    g, r, _, _ = _case(w)
    assert max(_compare(g, r).values()) <= TOL


def test_many_heads_wide_channels():
    # 128 heads of 2 channels at C = 256: the per-(target, head) statistics
    # and head sums hold heads lane and lane + 64 of each wave
    say("backward C = 256, H = 128")
    w = make_workload("tiny_fp32", l_max=1, channels=256, heads=128)
    g, r, _, _ = _case(w)
    assert max(_compare(g, r).values()) <= TOL


def test_empty_rows_and_partial_targets():
    say("backward empty rows, n_targets < n_atoms")
    w = make_workload("tiny_fp32")
    w.pos[5] = [500.0, 500.0, 500.0]
    g, r, rp, _ = _case(w, n_targets=40)
    assert np.all(g["dx"][5] == 0.0) and np.all(g["dpos"][5] == 0.0)
    assert max(_compare(g, r).values()) <= TOL


@pytest.mark.parametrize("cutoff,batches,L,C,dtype", [(6.0, 2, 2, 16, "fp32"), (7.5, 3, 2, 16, "fp32"),
                                                      (6.0, 2, 4, 128, "bf16")])
def test_edges_in_several_batches(cutoff, batches, L, C, dtype):
    say("backward edge batches", cutoff, batches, L, C, dtype)
    w = make_workload("water_l6", l_max=L, channels=C, heads=2, n_rbf=8, dtype=dtype, cutoff=cutoff)
    nt = 64  # batch capacity max(4096, 64 nt) = 4096 edges
    g, r, rp, _ = _case(w, n_targets=nt)
    n_edges = int(rp[nt] - rp[0])
    assert (batches - 1) * 4096 < n_edges <= batches * 4096, n_edges
    assert max(_compare(g, r).values()) <= (TOL if dtype == "fp32" else TOL_BF16)


def test_force_only_path_matches():
    say("backward without weight gradients")
    w = make_workload("tiny_fp32")
    rp, col = neighbors_bruteforce(w.pos, w.cutoff)
    dy = np.random.default_rng(4).standard_normal(w.x.shape).astype(np.float32)
    a = _gpu(w, rp, col, dy)
    b = _gpu(w, rp, col, dy, weights=False)
    assert set(b) == {"dx", "dpos"}
    assert max_rel_error(b["dx"], a["dx"]) <= 1e-5 and max_rel_error(b["dpos"][:, None], a["dpos"][:, None]) <= 1e-5


def test_gpu_forces_sum_to_zero_and_rotate():
    say("backward force invariants on the GPU")
    from scipy.spatial.transform import Rotation

    w = make_workload("tiny_fp32", l_max=3, channels=16, heads=2)
    rp, col = neighbors_bruteforce(w.pos, w.cutoff)
    dy = np.random.default_rng(2).standard_normal(w.x.shape).astype(np.float64)
    g = _gpu(w, rp, col, dy)
    scale = np.abs(g["dpos"]).max()
    assert np.abs(g["dpos"].sum(0)).max() <= 1e-5 * scale * np.sqrt(w.n_atoms)
    R = Rotation.random(random_state=5).as_matrix()
    D = wigner_d_blocks(w.l_max, R)

    def rot(f):
        out = np.empty_like(f)
        for l in range(w.l_max + 1):
            sl = slice(l * l, (l + 1) ** 2)
            out[:, sl] = np.einsum("ab,nbc->nac", D[l], f[:, sl])
        return out

    c = w.pos.mean(0)
    w2 = make_workload("tiny_fp32", l_max=3, channels=16, heads=2)
    w2.pos = ((w.pos - c) @ R.T + c).astype(np.float32)
    w2.x = rot(w.x.astype(np.float64)).astype(np.float32)
    rp2, col2 = neighbors_bruteforce(w2.pos, w2.cutoff)
    assert np.array_equal(rp2, rp) and np.array_equal(col2, col)
    g2 = _gpu(w2, rp2, col2, rot(dy))
    assert max_rel_error(g2["dpos"][:, None], (g["dpos"] @ R.T)[:, None]) <= 1e-4
    assert max_rel_error(g2["dx"], rot(g["dx"])) <= 1e-4
