"""Merged RMS layer norm on the GPU (so2_merged_rms_norm through the C ABI)
against the fp64 oracle ("EquiformerV3" technical summary, section 2.B.1).
The shapes reach every kernel path: values kept in registers (up to 8 or
16 vectors per lane), the two-read path for larger nodes, and the
element-wise path for odd channel counts and unaligned buffers.

Tolerances: fp32 output, max relative error (normalised per node) <= 1e-5
(fp32 sums of up to 12,544 squares); bf16 output, every element within one
bf16 rounding (2^-8 relative) of the oracle plus 1e-6 of the node's largest
value (the oracle gets the same bf16-rounded input)."""

import numpy as np
import pytest

from helpers import say
from oracle import max_rel_error, merged_rms_norm_ref
from synth import make_workload, to_bf16_exact

pytestmark = pytest.mark.gpu


def _run(x_np, gamma_np, dtype, eps=1e-5, inplace=False, offset=0):
    import torch

    import so_equivariant_graph_amd as sea

    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    n, nc, C = x_np.shape
    flat = torch.zeros(n * nc * C + offset, dtype=dt, device=dev)
    x = flat[offset:].view(n, nc, C)
    x.copy_(torch.from_numpy(x_np).to(dt))
    g = torch.from_numpy(gamma_np.astype(np.float32)).to(dev)
    y = sea.merged_rms_norm(x, g, eps=eps, out=x if inplace else None)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def _check(y, ref, dtype):
    if dtype == "fp32":
        assert max_rel_error(y, ref) <= 1e-5
    else:
        scale = np.abs(ref).max(axis=(1, 2), keepdims=True)
        assert np.all(np.abs(y - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * scale)


def _inputs(n, L, C, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, (L + 1) ** 2, C)).astype(np.float32)
    x *= rng.uniform(0.01, 30.0, size=(n, 1, 1)).astype(np.float32)
    x[0] = 0.0  # a zero node stays zero
    gamma = rng.uniform(0.5, 2.0, size=(L + 1, C))
    return x, gamma


@pytest.mark.parametrize(
    "dtype,L,C,offset",
    [("bf16", 4, 128, 0), ("bf16", 6, 128, 0), ("fp32", 4, 128, 0), ("bf16", 2, 6, 0), ("fp32", 3, 5, 0),
     ("bf16", 4, 128, 3), ("fp32", 1, 16, 1), ("bf16", 6, 256, 0), ("fp32", 6, 128, 0)],
)
def test_norm_matches_oracle(dtype, L, C, offset):
    say("norm", dtype, L, C, "offset", offset)
    x, gamma = _inputs(301, L, C, seed=L + C)
    if dtype == "bf16":
        x = to_bf16_exact(x)
    y = _run(x, gamma, dtype, offset=offset)
    ref = merged_rms_norm_ref(x, gamma)
    assert np.all(y[0] == 0.0)
    _check(y, ref, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_norm_in_place(dtype):
    say("norm in place", dtype)
    x, gamma = _inputs(67, 4, 128, seed=9)
    if dtype == "bf16":
        x = to_bf16_exact(x)
    y = _run(x, gamma, dtype, inplace=True)
    _check(y, merged_rms_norm_ref(x, gamma), dtype)


def test_norm_full_size_water_box_sampled_nodes():
    """The 100k-atom water box's features (bf16, L = 4, C = 128), the
    launch the benchmark times; sampled nodes against the oracle."""
    say("norm water_100k")
    import torch

    import so_equivariant_graph_amd as sea

    w = make_workload("water_100k")
    rng = np.random.default_rng(3)
    gamma = rng.uniform(0.5, 2.0, size=(w.l_max + 1, w.channels))
    x = torch.from_numpy(w.x).to(device="cuda:0", dtype=torch.bfloat16)
    y = sea.merged_rms_norm(x, torch.from_numpy(gamma.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    t = np.unique(np.concatenate([rng.choice(w.n_atoms, size=64, replace=False), [0, w.n_atoms - 1]]))
    yt = y[torch.from_numpy(t).cuda()].float().cpu().numpy().astype(np.float64)
    _check(yt, merged_rms_norm_ref(w.x[t], gamma), "bf16")
