#!/usr/bin/env python3
"""Benchmark of the hot path: neighbour-pair messages/s of the fused SO(2)
equivariant graph attention forward on one MI355X.

One step = the whole hot path over one batch of seeded synthetic input:
build_neighbors (cell list, a1) + so2_attention_fwd (q/k projection, the
fused kernel's prologue and the fused kernel, a2-a11).  Inputs are resident
in device memory before the timed region starts.  Prints ONE JSON line.
The default workload is the 100,000-atom periodic water box (L = 4,
C = 128, bf16), the largest system of the set that runs on one GPU.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload water_100k]
    python bench.py --memory-sweep [--steps 5 --warmup 2]   (peak bytes against N)
    python bench.py --norm                                  (merged RMS layer norm, HBM roofline)
    python bench.py --swiglu                                (SwiGLU-S2 activation, vector-unit roofline)
    python bench.py --backward 32 --steps 3 --warmup 1      (the backward on 32 small molecules)

value          messages (edges) per second of the whole step
roofline       the fused attention kernel against the dense bf16 MFMA peak:
               algorithmic flops per launch (E * 2C^2[(L+1)^2 + 2/3 L(L+1)(2L+1)])
               over its mean duration, timed with torch (HIP) events on the
               stream the library launches on, around the fused stage alone
cpu_baseline   the fp64 oracle (never tuned) on a bounded sample of the same
               workload, on this host's cores, in worker processes forked before
               the GPU is touched
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "neighbor-pair messages/sec, fused SO(2) attention fwd; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (vendor figure, no sparsity)
PEAK_HBM_GBS = 8000.0

# HBM bytes moved by one launch of the fused kernel, from two rocprofv3 --pmc
# passes over this benchmark (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch),
# each multiplied by the factor that maps the same counter's reading for a plain
# device copy of known size (--copy-probe) onto that size.  A figure holds only
# for the kernel sources it was taken on: their digest is stored with it and a
# mismatch reports null.
MEASURED_TRAFFIC = {
    # FETCH_SIZE 115172382 KiB x 1.99994 (a 1 GiB copy reads as 524305 KiB), WRITE_SIZE
    # 1272532 KiB x 1.00 (the copy writes read exactly 1048576 KiB); mean of 5 launches.
    "water_100k": {
        "sources_sha256": "35406eaaa9784c95ad6c2ec4230f665fea339553945b7f0074fa800b99033e19",
        "fetch_bytes": 235865480513,
        "write_bytes": 1303072379,
    },
}
# the files that hold the fused kernel's device code
KERNEL_SOURCES = ("attention_mfma.hip", "wigner.h", "common.h")


def flops_per_edge(L, C):
    """2 C^2 [(L+1)^2 + 2/3 L (L+1)(2L+1)]: the per-m map, 4 real products per m >= 1."""
    return 2 * C * C * ((L + 1) ** 2 + (2 * L * (L + 1) * (2 * L + 1)) // 3)


def kernel_digest():
    """sha256 over the fused kernel's source files, in a fixed order."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "so_equivariant_graph_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(d, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    rec = MEASURED_TRAFFIC.get(workload)
    if rec is None or rec["sources_sha256"] != kernel_digest():
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def copy_probe(mib):
    """A plain device-to-device copy of `mib` MiB, three times: the reference
    reading for FETCH_SIZE / WRITE_SIZE (each copy reads and writes mib MiB)."""
    import torch

    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    ok = bool(torch.equal(a[:: 1 << 16], b[:: 1 << 16]))
    print(json.dumps({"copy_probe_bytes": n * 4, "copies": 3, "ok": ok}), flush=True)


# ------------------------------------------------------------------ CPU leg


def _subsystem(w, targets, rows):
    """The atoms the oracle needs for `targets` (the targets first, then their
    neighbours) and the CSR of the targets' rows in that numbering: the
    oracle's result for a target depends on nothing else."""
    import numpy as np

    extra = np.setdiff1d(np.concatenate([r for r in rows] + [np.zeros(0, np.int64)]), targets)
    atoms = np.concatenate([np.asarray(targets, dtype=np.int64), extra.astype(np.int64)])
    index = {int(a): k for k, a in enumerate(atoms)}
    row_ptr = np.zeros(atoms.size + 1, dtype=np.int64)
    row_ptr[1 : len(targets) + 1] = np.cumsum([r.size for r in rows])
    row_ptr[len(targets) + 1 :] = row_ptr[len(targets)]
    col = np.array([index[int(j)] for r in rows for j in r], dtype=np.int64)
    return atoms, row_ptr, col


def _oracle_worker(args):
    """Time the fp64 oracle on `targets` (in batches of 8, so that the time
    budget can end it) for about `seconds`; returns (edges, targets, seconds)."""
    targets, seconds = args
    from threadpoolctl import threadpool_limits

    from oracle import neighbors_bruteforce, so2_attention_ref

    w = _WORKLOAD
    done_edges, done_targets, busy = 0, 0, 0.0
    with threadpool_limits(limits=1):
        for b0 in range(0, len(targets), 8):
            batch = targets[b0 : b0 + 8]
            rows = neighbors_bruteforce(w.pos, w.cutoff, w.box, w.mol_id, rows=batch)
            atoms, row_ptr, col = _subsystem(w, batch, rows)
            t0 = time.perf_counter()
            so2_attention_ref(
                w.pos[atoms], row_ptr, col, w.x[atoms], w.w_q, w.w_k, w.w_rad, w.w_so2, l_max=w.l_max,
                heads=w.heads, cutoff=w.cutoff, envelope_p=w.envelope_p, box=w.box, targets=range(len(batch)),
            )
            busy += time.perf_counter() - t0
            done_edges += int(row_ptr[len(batch)])
            done_targets += len(batch)
            if busy > seconds:
                break
    return done_edges, done_targets, busy


_WORKLOAD = None


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, seconds, max_workers=16):
    """Oracle messages/s on this host, before the GPU is touched: first one
    worker alone (the single-process rate), then one forked single-threaded
    worker per usable core (at most max_workers, the CPU share of one GPU),
    each timing the per-edge oracle on its own seeded share of targets for
    about `seconds`.  The oracle runs on the sub-system of each batch's
    targets and their neighbours, which gives the same outputs."""
    import multiprocessing as mp

    import numpy as np

    global _WORKLOAD
    _WORKLOAD = w
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    workers = max(1, min(avail, max_workers))
    order = np.random.default_rng(1234).permutation(w.n_atoms)
    ctx = mp.get_context("fork")
    with ctx.Pool(1) as pool:
        e1, t1, b1 = pool.map(_oracle_worker, [(order[:400].tolist(), seconds / 3)])[0]
    shares = [order[400 + k :: workers][:400].tolist() for k in range(workers)]
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        res = pool.map(_oracle_worker, [(s, seconds) for s in shares])
    wall = time.perf_counter() - t0
    edges = sum(r[0] for r in res)
    targets = sum(r[1] for r in res)
    busy = max(r[2] for r in res)
    return {
        "value": edges / busy,
        "unit": "messages/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{targets} seeded target atoms of {w.name} ({edges} edges), fp64 per-edge oracle on each "
        f"batch's sub-system, {workers} forked single-threaded workers, ~{seconds:.0f} s each "
        f"(wall {wall:.1f} s incl. graph rows)",
        "single_process_value": e1 / b1,
        "single_process_sample": f"{t1} target atoms ({e1} edges) in {b1:.1f} s, one single-threaded worker",
        "host_cores_available": avail,
        "cpu_model": _cpu_model(),
    }


# ------------------------------------------------------------------ GPU leg


def run_gpu(w, steps, warmup):
    """Warm-up, then `steps` timed steps (neighbour build + attention forward)
    between device synchronisations; the fused kernel of every timed step is
    bracketed by torch events on the stream the library launches on (torch's
    current stream), by calling the prologue and the fused kernel as two
    stages."""
    import numpy as np
    import torch

    import so_equivariant_graph_amd as sea

    dev = torch.device("cuda:0")
    dt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    t = lambda a, d=dt: torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=d)
    pos = t(w.pos, torch.float32)
    x, w_q, w_k, w_rad, w_so2 = (t(a) for a in (w.x, w.w_q, w.w_k, w.w_rad, w.w_so2))
    mol = None if w.mol_id is None else torch.from_numpy(w.mol_id.astype(np.int32)).to(dev)
    del w.x  # the host copy is not needed any more

    nb_ws = torch.empty(sea.neighbors_workspace_bytes(w.n_atoms), dtype=torch.uint8, device=dev)
    row_ptr, col = sea.build_neighbors(pos, w.cutoff, box=w.box, mol_id=mol, workspace=nb_ws)
    E = int(col.numel())
    nc = (w.l_max + 1) ** 2
    desc = sea.make_desc(
        n_atoms=w.n_atoms, n_targets=w.n_atoms, l_max=w.l_max, channels=w.channels, heads=w.heads,
        n_rbf=w.n_rbf, envelope_p=w.envelope_p, cutoff=w.cutoff, flags=0,
        dtype=sea.SO2_BF16 if w.dtype == "bf16" else sea.SO2_FP32,
    )
    kind = sea.attention_kernel_kind(desc)
    attn_ws = torch.empty(sea.attention_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    y = torch.empty((w.n_atoms, nc, w.channels), dtype=torch.float32, device=dev)
    cap = E
    kw = dict(l_max=w.l_max, heads=w.heads, cutoff=w.cutoff, envelope_p=w.envelope_p, box=w.box, out=y,
              workspace=attn_ws)

    def step(ev=None):
        rp, cl = sea.build_neighbors(pos, w.cutoff, box=w.box, mol_id=mol, capacity=cap, workspace=nb_ws)
        sea.so2_attention_fwd(pos, rp, cl, x, w_q, w_k, w_rad, w_so2, stages=sea.STAGE_PREPARE, **kw)
        if ev is not None:
            ev[0].record()
        sea.so2_attention_fwd(pos, rp, cl, x, w_q, w_k, w_rad, w_so2, stages=sea.STAGE_FUSED, **kw)
        if ev is not None:
            ev[1].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(events[k])
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in events]
    peak_bytes = torch.cuda.max_memory_allocated(dev)

    # attention-only rate (both stages, no neighbour build)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        sea.so2_attention_fwd(pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2, **kw)
    torch.cuda.synchronize()
    attn_total = time.perf_counter() - t1
    return dict(
        E=E, total_s=total, kern_ms=kern_ms, peak_bytes=int(peak_bytes), kind=kind,
        attn_ms=attn_total / steps * 1e3, finite=bool(torch.isfinite(y).all().item()),
    )


NORM_TRAFFIC = {
    # HBM bytes of one launch of merged_rms_norm_reg_kernel<bf16, 8> on the 100k-atom water
    # box's features: FETCH_SIZE 312574 KiB x 2.00, WRITE_SIZE 625000 KiB x 1.00 (the same
    # copy calibration as the fused kernel's figure); mean of 4 launches.
    "water_100k": {
        "sources_sha256": "0bba6f27ba07289078f31ce07f3de142738b052cd1fe948e0466e06a7fac618b",
        "fetch_bytes": 640131645,
        "write_bytes": 640000032,
    },
}
NORM_SOURCES = ("norm.hip", "norm.h", "common.h")


def norm_bench(steps, warmup):
    """The merged RMS layer norm of the 100k-atom water box's node features
    (bf16, L = 4, C = 128): nodes/s and the HBM roofline.  Algorithmic bytes
    per node: read x once and write y once, 2 (L+1)^2 C x 2 B, plus the
    gains (read once per launch).  Kernel time from torch events on the
    stream the library launches on (torch's current stream)."""
    import numpy as np
    import torch

    import so_equivariant_graph_amd as sea
    from synth import make_workload

    w = make_workload("water_100k")
    dev = torch.device("cuda:0")
    x = torch.from_numpy(w.x).to(device=dev, dtype=torch.bfloat16)
    del w.x
    gamma = torch.from_numpy(np.random.default_rng(0).uniform(0.5, 2.0, size=(w.l_max + 1, w.channels))
                             .astype(np.float32)).to(dev)
    y = torch.empty_like(x)
    for _ in range(warmup):
        sea.merged_rms_norm(x, gamma, out=y)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record()
        sea.merged_rms_norm(x, gamma, out=y)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    mean = sum(ms) / len(ms)
    n, nc, C = x.shape
    algo = 2 * n * nc * C * 2 + gamma.numel() * 4
    h = hashlib.sha256()
    for f in NORM_SOURCES:
        h.update(open(os.path.join(ROOT, "so_equivariant_graph_amd", "csrc", f), "rb").read())
    rec = NORM_TRAFFIC.get("water_100k")
    traffic = rec["fetch_bytes"] + rec["write_bytes"] if rec and rec["sources_sha256"] == h.hexdigest() else None
    print(json.dumps({
        "metric": "merged RMS layer norm nodes/s", "value": n / (mean * 1e-3), "unit": "nodes/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": mean, "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "water_100k node features", "n_atoms": n, "l_max": int(round(nc ** 0.5)) - 1,
                   "channels": C},
        "roofline": {"bound": "hbm", "achieved": algo / (mean * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": algo / (mean * 1e-3) / 1e9 / PEAK_HBM_GBS, "traffic": traffic},
        "detail": {"algorithmic_bytes": algo, "ms_min": ms[0], "ms_median": ms[len(ms) // 2],
                   "kernel_sources_sha256": h.hexdigest()},
    }), flush=True)


PEAK_FP32_VALU_TFLOPS = 157.3  # published vector fp32 (with packed FMA; single-issue FMA is half)
PEAK_FP32_MFMA_TFLOPS = 157.3  # published dense fp32 matrix-core figure


def swiglu_flops(L, C):
    """Algorithmic flops per node of the SwiGLU-S2 activation.  Matrix cores:
    the three per-degree maps and the gate map, 2 C^2 (3 (L+1)^2 + 1).  Vector
    units, per channel, the grid step as the kernel runs it (rings paired at
    +-cos(theta), meridians paired at +-phi): the even/odd harmonic sums of u
    and v, 2 (L+1)^2 multiply-adds per ring pair or middle ring (R of them);
    per ring, 6L multiply-adds for each of the Q = (n_f - 1) // 2 meridian
    pairs and 3 (L + 1) for phi = pi when n_f is even; (L+1)^2 per ring pair
    for the projection back; plus one product per grid point."""
    nc, nt, nf = (L + 1) ** 2, (3 * L + 2) // 2, 3 * L + 1
    mfma = 2 * C * C * (3 * nc + 1)
    r, q, e = (nt + 1) // 2, (nf - 1) // 2, 1 if nf % 2 == 0 else 0
    fma = r * 2 * nc + nt * (q * 6 * L + e * 3 * (L + 1)) + r * nc
    grid = C * (2 * fma + nt * nf)
    return mfma, grid


def swiglu_bench(steps, warmup):
    """The SwiGLU-S2 activation of the 100k-atom water box's node features
    (bf16, L = 4, C = 128) with seeded weights: nodes/s of the whole call,
    which runs the fused kernel (maps, grid step and output map per group of
    8 nodes; a 5-us weight repack before it), timed with torch events on the
    stream the library launches on.  Roofline: the vector-unit flops of the
    grid step over the call's time against the fp32 vector peak (the maps'
    matrix-core flops run in the same time and are reported beside it, as are
    the HBM bytes, x read and y written).  The same call in its three steps
    (maps, grid kernel, output map: three kernels through the workspace) is
    timed after it for comparison."""
    import numpy as np
    import torch

    import so_equivariant_graph_amd as sea
    from synth import make_workload

    w = make_workload("water_100k")
    dev = torch.device("cuda:0")
    x = torch.from_numpy(w.x).to(device=dev, dtype=torch.bfloat16)
    del w.x
    n, nc, C = x.shape
    L = int(round(nc ** 0.5)) - 1
    rng = np.random.default_rng(5)
    s = 1.0 / np.sqrt(C)
    mk = lambda *shape: torch.from_numpy((rng.standard_normal(shape) * s).astype(np.float32)).to(dev, torch.bfloat16)
    A, B, O, G = mk(L + 1, C, C), mk(L + 1, C, C), mk(L + 1, C, C), mk(C, C)
    y = torch.empty((n, nc, C), dtype=torch.float32, device=dev)
    ws = torch.empty(sea.load_library().so2_swiglu_s2_workspace_bytes(n, L, C, sea.SO2_BF16), dtype=torch.uint8,
                     device=dev)
    for _ in range(warmup):
        sea.swiglu_s2(x, A, B, G, O, out=y, workspace=ws)
    torch.cuda.synchronize()
    mk_ev = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    ev = [mk_ev() for _ in range(steps)]
    for a, b in ev:
        a.record()
        sea.swiglu_s2(x, A, B, G, O, out=y, workspace=ws)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    mean = sum(ms) / len(ms)
    finite = bool(torch.isfinite(y).all())
    # the three-step path, for comparison
    ev3 = [mk_ev() for _ in range(steps)]
    gev = [mk_ev() for _ in range(steps)]
    for (a, b), (ga, gb) in zip(ev3, gev):
        a.record()
        sea.swiglu_s2(x, A, B, G, O, out=y, workspace=ws, stages=sea.STAGE_SW_MAPS)
        ga.record()
        sea.swiglu_s2(x, A, B, G, O, out=y, workspace=ws, stages=sea.STAGE_SW_GRID)
        gb.record()
        sea.swiglu_s2(x, A, B, G, O, out=y, workspace=ws, stages=sea.STAGE_SW_OUT)
        b.record()
    torch.cuda.synchronize()
    ms3 = [a.elapsed_time(b) for a, b in ev3]
    grid_ms = [ga.elapsed_time(gb) for ga, gb in gev]
    mean3, gmean = sum(ms3) / len(ms3), sum(grid_ms) / len(grid_ms)
    f_mfma, f_grid = swiglu_flops(L, C)
    achieved = n * f_grid / (mean * 1e-3) / 1e12
    hbm_bytes = n * nc * C * (2 + 4)  # x in bf16 read, y in fp32 written
    print(json.dumps({
        "metric": "SwiGLU-S2 activation nodes/s", "value": n / (mean * 1e-3), "unit": "nodes/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": mean, "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "water_100k node features", "n_atoms": n, "l_max": L, "channels": C},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_VALU_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP32_VALU_TFLOPS, "traffic": None},
        "detail": {"kernel": "swiglu_fused_kernel (after sw_pack_kernel)", "grid_flop_per_node": f_grid,
                   "mfma_flop_per_node": f_mfma, "mfma_tflops_same_time": n * f_mfma / (mean * 1e-3) / 1e12,
                   "hbm_bytes": hbm_bytes, "hbm_tbps": hbm_bytes / (mean * 1e-3) / 1e12,
                   "ms_min": ms[0], "ms_median": ms[len(ms) // 2], "outputs_finite": finite,
                   "three_step_ms": mean3, "three_step_grid_kernel_ms": gmean,
                   "three_step_grid_tflops": n * f_grid / (gmean * 1e-3) / 1e12},
    }), flush=True)


def backward_bench(steps, warmup, n_molecules):
    """The backward of the attention layer (so2_attention_bwd) on a batch of
    the small-molecule workload (bf16 inputs, L = 4, C = 128): messages/s of
    the force-only call (dx, dpos) and of the full call (every weight
    gradient too), timed with torch events on the stream the library
    launches on.  Algorithmic flops per edge: the forward per-m map
    (recomputed) and its transpose, plus the SO(2) weight gradient in the
    full call, each the forward map's count; for bf16 inputs the three run
    as bf16-operand GEMMs on the matrix cores (fp32 operands split into two
    bf16 parts, fp32 accumulation), so the roofline is the bf16 MFMA peak."""
    import numpy as np
    import torch

    import so_equivariant_graph_amd as sea
    from synth import make_workload

    w = make_workload("small_molecules", geometry={"n_molecules": n_molecules})
    dev = torch.device("cuda:0")
    t = lambda a, d=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=d)
    pos = t(w.pos, torch.float32)
    x, w_q, w_k, w_rad, w_so2 = (t(a) for a in (w.x, w.w_q, w.w_k, w.w_rad, w.w_so2))
    mol = torch.from_numpy(w.mol_id.astype(np.int32)).to(dev)
    row_ptr, col = sea.build_neighbors(pos, w.cutoff, box=w.box, mol_id=mol)
    E = int(col.numel())
    dy = torch.randn((w.n_atoms, (w.l_max + 1) ** 2, w.channels), generator=torch.Generator().manual_seed(0)).to(dev)
    kw = dict(l_max=w.l_max, heads=w.heads, cutoff=w.cutoff, envelope_p=w.envelope_p, box=w.box)
    res = {}
    for name, weights in (("forces", False), ("full", True)):
        for _ in range(warmup):
            sea.so2_attention_bwd(pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2, dy, weights=weights, **kw)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record()
            g = sea.so2_attention_bwd(pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2, dy, weights=weights, **kw)
            b.record()
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in ev]
        res[name] = (sum(ms) / len(ms), bool(all(torch.isfinite(v).all() for v in g.values())))
    F = flops_per_edge(w.l_max, w.channels)
    ms_f, ok_f = res["forces"]
    ms_w, ok_w = res["full"]
    achieved = E * 3 * F / (ms_w * 1e-3) / 1e12
    print(json.dumps({
        "metric": "backward neighbor-pair messages/sec (so2_attention_bwd, all gradients)",
        "value": E / (ms_w * 1e-3), "unit": "messages/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_w, "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"small_molecules batch of {n_molecules}", "n_atoms": w.n_atoms, "n_edges": E,
                   "l_max": w.l_max, "channels": w.channels, "heads": w.heads},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None},
        "detail": {"forces_only_ms": ms_f, "forces_only_messages_per_s": E / (ms_f * 1e-3),
                   "forces_only_tflops": E * 2 * F / (ms_f * 1e-3) / 1e12, "full_ms": ms_w,
                   "flop_per_edge_full": 3 * F, "flop_per_edge_forces": 2 * F,
                   "outputs_finite": ok_f and ok_w},
    }), flush=True)


def variant_flops(L, C, m_max, n_focus):
    """Algorithmic flops per edge of a variant's per-m maps: F streams of C/F
    channels, orders up to m_max, 4 real products per m >= 1."""
    cf = C // n_focus
    return n_focus * 2 * cf * cf * ((L + 1) ** 2 + 4 * sum((L + 1 - m) ** 2 for m in range(1, m_max + 1)))


def variant_bench(steps, warmup, spec, workload):
    """so2_attention_fwd_variant on a workload with the radial logit bias and
    the orders and focus streams of spec ("M_MAX:N_FOCUS", M_MAX -1 = every
    order), seeded weights of the variant's shapes in the workload's dtype:
    messages/s of the whole call (torch events around each call), against
    the peak of the path it runs on (the fp32 matrix peak for the edge-batch
    path, whose per-m maps are fp32 GEMMs; the bf16 peak for the MFMA
    kernel), with the variant's algorithmic flops (variant_flops)."""
    import ctypes

    import numpy as np
    import torch

    import so_equivariant_graph_amd as sea
    from synth import make_workload, to_bf16_exact

    m_max, n_focus = (int(v) for v in spec.split(":"))
    w = make_workload(workload)
    L, C, H, K = w.l_max, w.channels, w.heads, w.n_rbf
    mm = L if m_max < 0 else m_max
    rng = np.random.default_rng(11)
    cf = C // n_focus
    ws = (rng.standard_normal(sea.load_library().so2_weight_count_variant(L, C, m_max, n_focus)) /
          np.sqrt(cf * (L + 1))).astype(np.float32)
    wl = (rng.standard_normal((K, H)) * 0.5).astype(np.float32)
    wf = (rng.standard_normal(C) / np.sqrt(cf)).astype(np.float32)
    if w.dtype == "bf16":
        ws, wl, wf = to_bf16_exact(ws), to_bf16_exact(wl), to_bf16_exact(wf)
    dev = torch.device("cuda:0")
    dt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    t = lambda a, d=dt: torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=d)
    pos = t(w.pos, torch.float32)
    x, w_q, w_k, w_rad = (t(a) for a in (w.x, w.w_q, w.w_k, w.w_rad))
    w_so2, w_logit, w_focus = t(ws), t(wl), t(wf) if n_focus > 1 else None
    mol = None if w.mol_id is None else torch.from_numpy(w.mol_id.astype(np.int32)).to(dev)
    row_ptr, col = sea.build_neighbors(pos, w.cutoff, box=w.box, mol_id=mol)
    E = int(col.numel())
    desc = sea.make_desc(n_atoms=w.n_atoms, n_targets=w.n_atoms, l_max=L, channels=C, heads=H, n_rbf=K,
                         envelope_p=w.envelope_p, cutoff=w.cutoff, flags=0,
                         dtype=sea.SO2_BF16 if w.dtype == "bf16" else sea.SO2_FP32)
    var = sea.AttnVariant(m_max, n_focus)
    lib = sea.load_library()
    kind = int(lib.so2_attention_variant_kernel_kind(ctypes.byref(desc), ctypes.byref(var)))
    ws_t = torch.empty(lib.so2_attention_variant_workspace_bytes(ctypes.byref(desc), ctypes.byref(var)),
                       dtype=torch.uint8, device=dev)
    y = torch.empty((w.n_atoms, (L + 1) ** 2, C), dtype=torch.float32, device=dev)
    kw = dict(l_max=L, heads=H, cutoff=w.cutoff, envelope_p=w.envelope_p, box=w.box, m_max=m_max, n_focus=n_focus,
              w_logit=w_logit, w_focus=w_focus, out=y, workspace=ws_t)
    for _ in range(warmup):
        sea.so2_attention_fwd_variant(pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2, **kw)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record()
        sea.so2_attention_fwd_variant(pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2, **kw)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    mean = sum(ms) / len(ms)
    F = variant_flops(L, C, mm, n_focus)
    peak = PEAK_BF16_TFLOPS if kind == 2 else PEAK_FP32_MFMA_TFLOPS
    achieved = E * F / (mean * 1e-3) / 1e12
    print(json.dumps({
        "metric": "neighbor-pair messages/sec, so2_attention_fwd_variant (logit bias, m_max, focus streams)",
        "value": E / (mean * 1e-3), "unit": "messages/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": mean, "higher_is_better": True,
        "dtype": ("bf16" if kind == 2 else f"{w.dtype} inputs, fp32 arithmetic"), "data": "synthetic",
        "config": {"workload": workload, "n_atoms": w.n_atoms, "n_edges": E, "l_max": L, "channels": C, "heads": H,
                   "m_max": mm, "n_focus": n_focus, "logit_bias": True},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": None},
        "detail": {"kernel_kind": kind, "flop_per_edge": F, "ms_min": ms[0], "ms_median": ms[len(ms) // 2],
                   "outputs_finite": bool(torch.isfinite(y).all().item())},
    }), flush=True)


SWEEP_ATOMS = (12_500, 25_000, 50_000, 100_000, 200_000)


def memory_sweep(steps, warmup):
    """Peak device bytes and throughput of the whole step against atom count:
    the periodic water box at 0.1 atoms/A^3 with a 5 A cutoff (the 100k-atom
    workload's recipe) at every size in SWEEP_ATOMS.  Prints one JSON line
    per size, then a least-squares line bytes = a + b N with its largest
    relative residual.  Every buffer of the step is a torch allocation (the
    library allocates nothing), so torch's peak counter covers them all."""
    import numpy as np
    import torch

    from synth import make_workload

    pts = []
    for n in SWEEP_ATOMS:
        w = make_workload("water_100k", geometry={"n_atoms": n})
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        g = run_gpu(w, steps, warmup)
        kern = sum(g["kern_ms"]) / len(g["kern_ms"])
        rec = {
            "n_atoms": n, "n_edges": g["E"], "peak_device_bytes": g["peak_bytes"],
            "peak_bytes_per_atom": g["peak_bytes"] / n, "ms_per_step": g["total_s"] / steps * 1e3,
            "messages_per_s": g["E"] * steps / g["total_s"], "attention_kernel_ms_mean": kern,
            "attention_tflops": g["E"] * flops_per_edge(w.l_max, w.channels) / (kern * 1e-3) / 1e12,
            "outputs_finite": g["finite"],
        }
        pts.append(rec)
        print(json.dumps(rec), flush=True)
        del w, g
    n = np.array([p["n_atoms"] for p in pts], dtype=np.float64)
    b = np.array([p["peak_device_bytes"] for p in pts], dtype=np.float64)
    slope, icpt = np.polyfit(n, b, 1)
    resid = np.abs(b - (icpt + slope * n)) / b
    print(json.dumps({"fit": "peak_device_bytes = a + b * n_atoms", "a_bytes": icpt, "b_bytes_per_atom": slope,
                      "max_relative_residual": float(resid.max())}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="water_100k",
                    help="water_100k (default, the largest single-GPU system), solvated_protein, small_molecules, "
                    "water_l6 or tiny_fp32")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, metavar="MIB", default=0,
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--swiglu", action="store_true",
                    help="the SwiGLU-S2 activation of the 100k-atom water box's features instead of the attention step")
    ap.add_argument("--norm", action="store_true",
                    help="only time the merged RMS layer norm on the 100k-atom water box's features")
    ap.add_argument("--backward", type=int, metavar="N_MOLECULES", default=0,
                    help="only time so2_attention_bwd on a batch of N small molecules")
    ap.add_argument("--variant", metavar="M_MAX:N_FOCUS", default=None,
                    help="only time so2_attention_fwd_variant (with the radial logit bias) on --workload")
    ap.add_argument("--memory-sweep", action="store_true",
                    help="only run the water box at 12.5k-200k atoms: peak device bytes against N")
    args = ap.parse_args()
    if args.gpus != 1:
        print(
            f"bench.py runs on one GPU only (--gpus {args.gpus} requested); the multi-GPU "
            "sharding of this path is a design, not a measured configuration.",
            file=sys.stderr,
        )
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.memory_sweep:
        memory_sweep(args.steps, args.warmup)
        return
    if args.backward:
        backward_bench(args.steps, args.warmup, args.backward)
        return
    if args.variant:
        variant_bench(args.steps, args.warmup, args.variant, args.workload)
        return
    if args.norm:
        norm_bench(args.steps, args.warmup)
        return
    if args.swiglu:
        swiglu_bench(args.steps, args.warmup)
        return

    from synth import make_workload

    w = make_workload(args.workload)
    L, C = w.l_max, w.channels
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_seconds)
    g = run_gpu(w, args.steps, args.warmup)

    E = g["E"]
    F = flops_per_edge(L, C)
    ms_step = g["total_s"] / args.steps * 1e3
    kern = sorted(g["kern_ms"])
    kern_mean = sum(kern) / len(kern)
    achieved = E * F / (kern_mean * 1e-3) / 1e12
    # the MFMA kernel runs bf16 operands; the edge-batch path's per-m maps are fp32 GEMMs
    peak = PEAK_BF16_TFLOPS if g["kind"] == 2 else PEAK_FP32_MFMA_TFLOPS
    traffic = measured_traffic(w.name) if g["kind"] == 2 else None
    line = {
        "metric": METRIC,
        "value": E * args.steps / g["total_s"],
        "unit": "messages/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "n_atoms": w.n_atoms,
            "n_edges": E,
            "l_max": L,
            "channels": C,
            "heads": w.heads,
            "n_rbf": w.n_rbf,
            "cutoff": w.cutoff,
            "periodic": w.box is not None,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
        "detail": {
            "attention_kernel": {1: "valu_fp32", 2: "mfma_bf16"}.get(g["kind"], "none"),
            "attention_kernel_ms_mean": kern_mean,
            "attention_kernel_ms_min": kern[0],
            "attention_kernel_ms_median": kern[len(kern) // 2],
            "attention_call_ms": g["attn_ms"],
            "attention_messages_per_s": E / (kern_mean * 1e-3),
            "neighbors_plus_overhead_ms": ms_step - kern_mean,
            "flop_per_edge": F,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "traffic_GBps": None if traffic is None else traffic / (kern_mean * 1e-3) / 1e9,
            "kernel_sources_sha256": kernel_digest(),
            "peak_device_bytes": g["peak_bytes"],
            "peak_device_bytes_per_atom": g["peak_bytes"] / w.n_atoms,
            "outputs_finite": g["finite"],
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
