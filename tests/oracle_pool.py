"""Oracle outputs for the full-size GPU parity tests, computed in the
background while the other GPU tests run.

The fp64 oracle needs about a minute of 16 cores for every atom of the
small-molecule batch and the L = 6 water box plus 1,024 targets of the
solvated protein and of the 100k-atom water box.  conftest starts these jobs
when the session collects a test marked ``oracle_full``: one pool of
single-threaded worker processes (spawned, so they share nothing with the
process that drives the GPU) per workload, each worker building the seeded
workload once.  A test asks for its job's result and gets every sampled
target's oracle output (float32) and brute-force neighbour row.

The oracle runs on the sub-system of each batch of targets: the targets
first, then their neighbours, with the targets' rows renumbered.  A target's
output depends only on its neighbours, so this gives the same numbers as a
call on the whole system."""

import os
import time

import numpy as np

# job name -> (workload, geometry, overrides, targets: "all" or a count,
# workers); the workers split the 16 cores of the host's share about in
# proportion to each job's oracle time
JOBS = {
    "small_molecules/all": ("small_molecules", None, {}, "all", 3),
    "water_l6/all": ("water_l6", None, {}, "all", 6),
    "solvated_protein/1024": ("solvated_protein", None, {}, 1024, 2),
    "water_100k/1024": ("water_100k", None, {}, 1024, 2),
    "water_l6_13k/256": ("water_100k", {"n_atoms": 13_000}, {"l_max": 6}, 256, 2),
}
# atom count of every job's workload (the tests check it), so that the
# targets are known without building the positions in the test process
N_ATOMS = {
    "small_molecules/all": 10_384,
    "water_l6/all": 3_000,
    "solvated_protein/1024": 30_000,
    "water_100k/1024": 100_000,
    "water_l6_13k/256": 13_000,
}
TARGET_SEED = 2024
BATCH = 16

_pools = {}
_results = {}
_started = {}


def workload(job):
    from synth import make_workload

    name, geometry, overrides, _, _ = JOBS[job] if isinstance(job, str) else job
    return make_workload(name, geometry=geometry, **overrides)


def job_targets(job, n_atoms):
    count = JOBS[job][3]
    if count == "all":
        return np.arange(n_atoms)
    rng = np.random.default_rng(TARGET_SEED)
    t = np.sort(rng.choice(n_atoms, size=min(count, n_atoms), replace=False))
    return np.unique(np.concatenate([t, [0, n_atoms - 1]]))


def subsystem(targets, rows):
    """(atoms, row_ptr, col): the targets first, then their other
    neighbours; CSR rows for the targets only, in the new numbering."""
    targets = np.asarray(targets, dtype=np.int64)
    allnb = np.concatenate([np.asarray(r, dtype=np.int64) for r in rows] + [np.zeros(0, np.int64)])
    extra = np.setdiff1d(allnb, targets)
    atoms = np.concatenate([targets, extra])
    index = np.full(int(atoms.max()) + 1, -1, dtype=np.int64)
    index[atoms] = np.arange(atoms.size)
    row_ptr = np.zeros(atoms.size + 1, dtype=np.int64)
    row_ptr[1 : targets.size + 1] = np.cumsum([len(r) for r in rows])
    row_ptr[targets.size + 1 :] = row_ptr[targets.size]
    col = index[allnb]
    return atoms, row_ptr, col


_W = None
_INIT_ERROR = None


def _init(spec):
    """Worker set-up: one thread, the job's workload built once.  A failure
    is kept and raised by every task (a pool whose initializer raised would
    start new workers without end)."""
    global _W, _INIT_ERROR
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(limits=1)
        _W = workload(spec)
    except BaseException as exc:  # noqa: BLE001 - reported through the tasks
        _INIT_ERROR = repr(exc)


def _batch(targets):
    from oracle import neighbors_bruteforce, so2_attention_ref

    if _INIT_ERROR is not None:
        raise RuntimeError(f"oracle worker set-up failed: {_INIT_ERROR}")
    w = _W
    rows = neighbors_bruteforce(w.pos, w.cutoff, w.box, w.mol_id, rows=list(targets))
    atoms, row_ptr, col = subsystem(targets, rows)
    y = so2_attention_ref(
        w.pos[atoms], row_ptr, col, w.x[atoms], w.w_q, w.w_k, w.w_rad, w.w_so2, l_max=w.l_max,
        heads=w.heads, cutoff=w.cutoff, envelope_p=w.envelope_p, box=w.box, targets=range(len(targets)),
    )
    return np.asarray(targets), y.astype(np.float32), [np.asarray(r, dtype=np.int32) for r in rows]


def start(jobs):
    """Start the background oracle runs for `jobs` (idempotent)."""
    import multiprocessing as mp

    ctx = mp.get_context("spawn")
    budget = int(os.environ.get("SO2_ORACLE_WORKERS", "16"))
    for job in jobs:
        if job in _pools:
            continue
        n_workers = max(1, min(JOBS[job][4], budget))
        targets = job_targets(job, N_ATOMS[job])
        batches = [targets[i : i + BATCH] for i in range(0, targets.size, BATCH)]
        pool = ctx.Pool(n_workers, initializer=_init, initargs=(JOBS[job],))
        _pools[job] = pool
        _results[job] = pool.map_async(_batch, batches, chunksize=1)
        _started[job] = time.time()


def result(job, timeout=600.0):
    """(targets, y_ref [T, (L+1)^2, C] float32, rows) of a started job."""
    if job not in _pools:
        start([job])
    parts = _results[job].get(timeout=timeout)
    _pools.pop(job).close()
    targets = np.concatenate([p[0] for p in parts])
    y = np.concatenate([p[1] for p in parts])
    rows = [r for p in parts for r in p[2]]
    return targets, y, rows


def shutdown():
    for pool in _pools.values():
        pool.terminate()
    _pools.clear()
