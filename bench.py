#!/usr/bin/env python3
"""Benchmark of the hot path: neighbour-pair messages/s of the fused SO(2)
equivariant graph attention forward on one MI355X.

One step = the whole hot path over one batch of seeded synthetic input:
build_neighbors (cell list, a1) + so2_attention_fwd (q/k projection and the
fused kernel, a2-a11).  Inputs are resident in device memory before the
timed region starts.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload small_molecules]
    python bench.py --memory-sweep [--steps 5 --warmup 2]   (peak bytes against N)
    python bench.py --norm                                  (merged RMS layer norm, HBM roofline)
    python bench.py --swiglu                                (SwiGLU-S2 activation, vector-unit roofline)

value          messages (edges) per second of the whole step
roofline       the fused attention kernel against the dense bf16 MFMA peak:
               algorithmic flops per launch (E * 2C^2[(L+1)^2 + 2/3 L(L+1)(2L+1)])
               over its mean duration, timed with HIP events the library records
               around that kernel on its own stream
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
    # FETCH_SIZE 2588185 KiB x 2.00 (a 1 GiB copy reads as 524302 KiB), WRITE_SIZE
    # 147800 KiB x 1.00 (the copy writes read exactly 1048576 KiB); mean of 7 launches.
    "small_molecules": {
        "sources_sha256": "e94fe024fc58d120beb9358742307a2e9d96a629bfedec38354fb490bc40181f",
        "fetch_bytes": 5300458768,
        "write_bytes": 151347200,
    },
}
KERNEL_SOURCES = ("attention_mfma.hip", "wigner.h", "common.h", "launch.h")


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


def _oracle_worker(args):
    name, targets, seconds = args
    from threadpoolctl import threadpool_limits

    import numpy as np

    from oracle import neighbors_bruteforce, so2_attention_ref

    w = _WORKLOAD
    with threadpool_limits(limits=1):
        rows = neighbors_bruteforce(w.pos, w.cutoff, w.box, w.mol_id, rows=targets)
        row_ptr = np.zeros(w.n_atoms + 1, dtype=np.int64)
        deg = np.zeros(w.n_atoms, dtype=np.int64)
        for t, r in zip(targets, rows):
            deg[t] = r.size
        np.cumsum(deg, out=row_ptr[1:])
        col = np.zeros(row_ptr[-1], dtype=np.int32)
        for t, r in zip(targets, rows):
            col[row_ptr[t] : row_ptr[t + 1]] = r
        done_edges, done_targets = 0, 0
        t0 = time.perf_counter()
        for t in targets:
            so2_attention_ref(
                w.pos, row_ptr, col, w.x, w.w_q, w.w_k, w.w_rad, w.w_so2, l_max=w.l_max,
                heads=w.heads, cutoff=w.cutoff, envelope_p=w.envelope_p, box=w.box, targets=[t],
            )
            done_edges += int(deg[t])
            done_targets += 1
            if time.perf_counter() - t0 > seconds:
                break
        return done_edges, done_targets, time.perf_counter() - t0


_WORKLOAD = None


def cpu_baseline(w, seconds):
    """Oracle messages/s on this host: fork one worker per core, each timing the
    per-edge oracle on its own seeded share of targets for about `seconds`."""
    import multiprocessing as mp

    import numpy as np

    global _WORKLOAD
    _WORKLOAD = w
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))
    order = np.random.default_rng(1234).permutation(w.n_atoms)
    shares = [order[k::cores][:400].tolist() for k in range(cores)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        res = pool.map(_oracle_worker, [(w.name, s, seconds) for s in shares])
    wall = time.perf_counter() - t0
    edges = sum(r[0] for r in res)
    targets = sum(r[1] for r in res)
    busy = max(r[2] for r in res)
    return {
        "value": edges / busy,
        "unit": "messages/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{targets} seeded target atoms of {w.name} ({edges} edges), fp64 per-edge oracle, "
        f"{cores} forked single-threaded workers, ~{seconds:.0f} s each (wall {wall:.1f} s incl. graph rows)",
    }


# ------------------------------------------------------------------ GPU leg


def run_gpu(w, steps, warmup):
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
        n_atoms=w.n_atoms, n_targets=w.n_atoms, n_edges=E, l_max=w.l_max, channels=w.channels,
        heads=w.heads, n_rbf=w.n_rbf, envelope_p=w.envelope_p, cutoff=w.cutoff, flags=0,
        dtype=sea.SO2_BF16 if w.dtype == "bf16" else sea.SO2_FP32,
    )
    kind = sea.attention_kernel_kind(desc)
    attn_ws = torch.empty(sea.attention_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    y = torch.empty((w.n_atoms, nc, w.channels), dtype=torch.float32, device=dev)
    cap = E

    def step():
        rp, cl = sea.build_neighbors(pos, w.cutoff, box=w.box, mol_id=mol, capacity=cap, workspace=nb_ws)
        sea.so2_attention_fwd(
            pos, rp, cl, x, w_q, w_k, w_rad, w_so2, l_max=w.l_max, heads=w.heads, cutoff=w.cutoff,
            envelope_p=w.envelope_p, box=w.box, out=y, workspace=attn_ws,
        )

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    timer = sea.KernelTimer(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        timer.arm()
        step()
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    timer.disarm()
    kern_ms = timer.elapsed_ms()
    timer.close()
    peak_bytes = torch.cuda.max_memory_allocated(dev)

    # attention-only rate (same kernel, no neighbour build)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        sea.so2_attention_fwd(
            pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2, l_max=w.l_max, heads=w.heads,
            cutoff=w.cutoff, envelope_p=w.envelope_p, box=w.box, out=y, workspace=attn_ws,
        )
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
        "sources_sha256": "84afa7d832182174e207bd85e5d226f8156f28722616c3d8f53e7018826b4a74",
        "fetch_bytes": 640132977,
        "write_bytes": 640000000,
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
    (bf16, L = 4, C = 128) with seeded weights: nodes/s, and the vector-unit
    roofline of the grid kernel (the largest of the step's kernels), timed by
    the library's HIP events on its stream; the whole call by torch events."""
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
    timer = sea.KernelTimer(steps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        timer.arm()
        a.record()
        sea.swiglu_s2(x, A, B, G, O, out=y, workspace=ws)
        b.record()
    torch.cuda.synchronize()
    timer.disarm()
    grid_ms = timer.elapsed_ms()
    timer.close()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    mean = sum(ms) / len(ms)
    gmean = sum(grid_ms) / len(grid_ms)
    f_mfma, f_grid = swiglu_flops(L, C)
    achieved = n * f_grid / (gmean * 1e-3) / 1e12
    print(json.dumps({
        "metric": "SwiGLU-S2 activation nodes/s", "value": n / (mean * 1e-3), "unit": "nodes/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": mean, "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "water_100k node features", "n_atoms": n, "l_max": L, "channels": C},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_VALU_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP32_VALU_TFLOPS, "traffic": None},
        "detail": {"grid_kernel_ms_mean": gmean, "grid_flop_per_node": f_grid, "mfma_flop_per_node": f_mfma,
                   "maps_ms": mean - gmean,
                   "maps_tflops": n * f_mfma / ((mean - gmean) * 1e-3) / 1e12 if mean > gmean else None,
                   "ms_min": ms[0], "ms_median": ms[len(ms) // 2],
                   "outputs_finite": bool(torch.isfinite(y).all())},
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
    ap.add_argument("--workload", default="small_molecules")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, metavar="MIB", default=0,
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--swiglu", action="store_true",
                    help="the SwiGLU-S2 activation of the 100k-atom water box's features instead of the attention step")
    ap.add_argument("--norm", action="store_true",
                    help="only time the merged RMS layer norm on the 100k-atom water box's features")
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
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
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
