"""Shared helpers for the GPU tests: move a seeded workload to the device,
run the HIP path through the C ABI, and print what names each case before
it runs (so a failing GPU step is identifiable from the log alone)."""

import sys

import numpy as np


def say(*args):
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def device_inputs(w, device="cuda"):
    import torch

    dt = torch.float32 if w.dtype == "fp32" else torch.bfloat16

    def t(a, d=dt):
        # float32 -> bfloat16 is exact here: the workload's values are bf16-exact
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=d)

    out = dict(
        pos=t(w.pos, torch.float32),
        x=t(w.x),
        w_q=t(w.w_q),
        w_k=t(w.w_k),
        w_rad=t(w.w_rad),
        w_so2=t(w.w_so2),
        mol=None if w.mol_id is None else torch.from_numpy(w.mol_id.astype(np.int32)).to(device),
    )
    return out


def csr_to_device(row_ptr, col, device="cuda"):
    import torch

    return (
        torch.from_numpy(np.ascontiguousarray(row_ptr, dtype=np.int32)).to(device),
        torch.from_numpy(np.ascontiguousarray(col, dtype=np.int32)).to(device),
    )


def gpu_attention(w, d, row_ptr, col, **kw):
    import so_equivariant_graph_amd as sea

    return sea.so2_attention_fwd(
        d["pos"], row_ptr, col, d["x"], d["w_q"], d["w_k"], d["w_rad"], d["w_so2"],
        l_max=w.l_max, heads=w.heads, cutoff=w.cutoff, envelope_p=w.envelope_p, box=w.box, **kw,
    )


def oracle_attention(w, row_ptr, col, targets=None, **kw):
    from oracle import so2_attention_ref

    return so2_attention_ref(
        w.pos, row_ptr, col, w.x, w.w_q, w.w_k, w.w_rad, w.w_so2, l_max=w.l_max, heads=w.heads,
        cutoff=w.cutoff, envelope_p=w.envelope_p, box=w.box, targets=targets, **kw,
    )


TOL = {"fp32": 1e-4, "bf16": 2e-2}
