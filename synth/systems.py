"""Seeded synthetic atomistic systems and random-init weights.

Five workloads, shaped after the systems the E2Former-V2 summary measures
on (small drug-like molecules, a periodic liquid-water box, a solvated
protein of about 30k atoms, a 100k-atom system; technical summary,
sections 3 and 4).  None of those datasets is used or reproduced: every
input is drawn here from a seeded NumPy PCG64 generator, in the order
positions, x, W_q, W_k, W_rad, W_so2 (m ascending, W1 before W2).

    tiny_fp32            64 atoms uniform in an 8 A cube (0.9 A rejection),
                         open boundaries, rc 5, L 2, C 16, H 2, K 8, fp32
    small_molecules      256 self-avoiding-walk molecules of 20..60 atoms
                         (steps 1.1..1.5 A, 0.9 A rejection), one molecule
                         per lattice site, mol_id given, rc 6, L 4, C 128,
                         H 8, K 16, bf16
    water_l6             1000 rigid waters (O-H 0.96 A, 104.5 deg) on a
                         jittered 10^3 lattice in a 31 A periodic cube,
                         rc 6, L 6, C 128, H 8, K 16, bf16
    solvated_protein     3000-atom walk (1.5 A steps) inside a sphere of
                         radius 19.3 A, 9000 waters around it, 67 A periodic
                         cube, 30000 atoms, rc 6, L 4, C 128, H 8, K 16, bf16
    water_100k           water at 0.1 atoms/A^3, 100 A periodic cube,
                         100000 atoms, rc 5, L 4, C 128, H 8, K 16, bf16

bf16 inputs are rounded to nearest-even here and handed to both sides as
the same values (the oracle widens them to fp64)."""

from dataclasses import dataclass, field
from math import ceil, sqrt

import numpy as np

WATER_OH = 0.96
WATER_ANGLE_DEG = 104.5
MIN_SEP = 0.9


@dataclass
class Workload:
    name: str
    pos: np.ndarray  # [N,3] float32
    box: object  # float32[3] or None
    mol_id: object  # int32[N] or None
    cutoff: float
    l_max: int
    channels: int
    heads: int
    n_rbf: int
    envelope_p: int
    dtype: str  # "fp32" or "bf16"
    x: np.ndarray  # [N,(L+1)^2,C] float32 (bf16-exact values for bf16)
    w_q: np.ndarray  # [C,C] float32 (in, out)
    w_k: np.ndarray  # [C,C]
    w_rad: np.ndarray  # [K,C]
    w_so2: np.ndarray  # packed, float32
    meta: dict = field(default_factory=dict)

    @property
    def n_atoms(self) -> int:
        return int(self.pos.shape[0])


def to_bf16_exact(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even) and return
    them as float32 (exactly representable in bf16)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty_like(a)
    flat_in = a.reshape(-1)
    flat_out = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        u = flat_in[s : s + step].view(np.uint32).astype(np.uint64)
        r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
        flat_out[s : s + step] = r.astype(np.uint32).view(np.float32)
    return out


def _unit_vectors(rng, n):
    v = rng.standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1)[:, None]


def _quat_to_matrix(q):
    w, x, y, z = q
    return np.array(
        [
            [1 - 2 * (y * y + z * z), 2 * (x * y - z * w), 2 * (x * z + y * w)],
            [2 * (x * y + z * w), 1 - 2 * (x * x + z * z), 2 * (y * z - x * w)],
            [2 * (x * z - y * w), 2 * (y * z + x * w), 1 - 2 * (x * x + y * y)],
        ]
    )


def _random_rotations(rng, n):
    q = rng.standard_normal((n, 4))
    q /= np.linalg.norm(q, axis=1)[:, None]
    return np.stack([_quat_to_matrix(qq) for qq in q])


def _water_template():
    half = np.deg2rad(WATER_ANGLE_DEG) / 2.0
    return np.array(
        [
            [0.0, 0.0, 0.0],
            [WATER_OH * np.sin(half), 0.0, WATER_OH * np.cos(half)],
            [-WATER_OH * np.sin(half), 0.0, WATER_OH * np.cos(half)],
        ]
    )


def _uniform_cube(rng, n, side, min_sep):
    pts = np.zeros((0, 3))
    while pts.shape[0] < n:
        c = rng.uniform(0.0, side, size=3)
        if pts.shape[0] and np.min(np.sum((pts - c) ** 2, axis=1)) < min_sep**2:
            continue
        pts = np.vstack([pts, c])
    return pts


def _self_avoiding_walk(rng, n, step_lo, step_hi, min_sep, max_fail=1000):
    """One molecule; restart after max_fail consecutive rejected steps."""
    while True:
        pts = np.zeros((n, 3))
        k = 1
        fails = 0
        while k < n:
            d = _unit_vectors(rng, 1)[0]
            step = rng.uniform(step_lo, step_hi)
            cand = pts[k - 1] + step * d
            if np.min(np.sum((pts[:k] - cand) ** 2, axis=1)) < min_sep**2:
                fails += 1
                if fails >= max_fail:
                    break
                continue
            pts[k] = cand
            k += 1
            fails = 0
        if k == n:
            return pts


def _confined_walk(rng, n, step, min_sep, center, radius, max_fail=1000, backtrack=10):
    """Self-avoiding walk of fixed step length kept inside a sphere; after
    max_fail consecutive rejections the last `backtrack` atoms are removed."""
    pts = np.zeros((n, 3))
    pts[0] = center
    k = 1
    fails = 0
    while k < n:
        d = _unit_vectors(rng, 1)[0]
        cand = pts[k - 1] + step * d
        bad = np.sum((cand - center) ** 2) >= radius * radius or (
            np.min(np.sum((pts[:k] - cand) ** 2, axis=1)) < min_sep**2
        )
        if bad:
            fails += 1
            if fails >= max_fail:
                k = max(1, k - backtrack)
                fails = 0
            continue
        pts[k] = cand
        k += 1
        fails = 0
    return pts


def _place_waters(rng, sites, spacing_jitter, box, fixed=None, max_rounds=2000):
    """Rigid waters at jittered sites with random orientations.  Any water
    with an atom closer than MIN_SEP to an atom of another molecule (minimum
    image) gets a new orientation and jitter, until no such pair is left.
    `fixed` are atoms of other molecules that never move (e.g. a protein)."""
    from scipy.spatial import cKDTree

    n_w = sites.shape[0]
    tmpl = _water_template()
    jit = rng.uniform(-spacing_jitter, spacing_jitter, size=(n_w, 3))
    rots = _random_rotations(rng, n_w)
    n_fixed = 0 if fixed is None else fixed.shape[0]

    def build(jit, rots):
        o = sites + jit
        w = o[:, None, :] + np.einsum("nij,aj->nai", rots, tmpl)
        return w.reshape(-1, 3)

    atoms = build(jit, rots)
    for _ in range(max_rounds):
        allp = atoms if fixed is None else np.vstack([fixed, atoms])
        mol = np.concatenate([np.full(n_fixed, -1), np.repeat(np.arange(n_w), 3)])
        wrapped = np.mod(allp, box) if box is not None else allp
        if box is not None:
            wrapped = np.where(wrapped >= box, 0.0, wrapped)
        tree = cKDTree(wrapped, boxsize=box)
        pairs = tree.query_pairs(MIN_SEP, output_type="ndarray")
        if pairs.size:
            ma, mb = mol[pairs[:, 0]], mol[pairs[:, 1]]
            inter = ma != mb
            redo = np.unique(np.maximum(ma[inter], mb[inter]))
            redo = redo[redo >= 0]
        else:
            redo = np.zeros(0, dtype=np.int64)
        if redo.size == 0:
            return atoms
        jit[redo] = rng.uniform(-spacing_jitter, spacing_jitter, size=(redo.size, 3))
        rots[redo] = _random_rotations(rng, redo.size)
        atoms = build(jit, rots)
    raise RuntimeError("water placement did not converge")


def water_box_positions(rng, n_atoms, density=0.1, jitter=0.25):
    """Water box at `density` atoms/A^3: O sites on a jittered n^3 lattice,
    a seeded subset of ceil(N/3) of them (kept in lattice order), truncated
    to N atoms.  Returns (pos [N,3] float64, box side)."""
    side = (n_atoms / density) ** (1.0 / 3.0)
    n_mol = ceil(n_atoms / 3)
    n = ceil(n_mol ** (1.0 / 3.0) - 1e-9)
    while n**3 < n_mol:
        n += 1
    spacing = side / n
    g = (np.arange(n) + 0.5) * spacing
    grid = np.stack(np.meshgrid(g, g, g, indexing="ij"), axis=-1).reshape(-1, 3)
    pick = np.sort(rng.choice(grid.shape[0], size=n_mol, replace=False))
    box = np.array([side, side, side])
    atoms = _place_waters(rng, grid[pick], jitter, box)
    return atoms[:n_atoms], side


def _draw_features_and_weights(rng, n_atoms, l_max, C, K, dtype):
    nc = (l_max + 1) ** 2
    x = rng.standard_normal((n_atoms, nc, C), dtype=np.float32)
    w_q = (rng.standard_normal((C, C)) / sqrt(C)).astype(np.float32)
    w_k = (rng.standard_normal((C, C)) / sqrt(C)).astype(np.float32)
    w_rad = (rng.standard_normal((K, C)) / sqrt(K)).astype(np.float32)
    std = 1.0 / sqrt(C * (l_max + 1))
    blocks = []
    k0 = (l_max + 1) * C
    blocks.append(rng.standard_normal(k0 * k0) * std)
    for m in range(1, l_max + 1):
        km = (l_max + 1 - m) * C
        blocks.append(rng.standard_normal(km * km) * std)  # W1_m
        blocks.append(rng.standard_normal(km * km) * std)  # W2_m
    w_so2 = np.concatenate(blocks).astype(np.float32)
    if dtype == "bf16":
        x = to_bf16_exact(x)
        w_q, w_k, w_rad, w_so2 = (to_bf16_exact(a) for a in (w_q, w_k, w_rad, w_so2))
    return x, w_q, w_k, w_rad, w_so2


def _tiny(seed, n_atoms=64, side=8.0):
    rng = np.random.default_rng(seed)
    pos = _uniform_cube(rng, n_atoms, side, MIN_SEP)
    return rng, pos, None, None


def _small_molecules(seed, n_molecules=256, n_lo=20, n_hi=60, cutoff=6.0):
    rng = np.random.default_rng(seed)
    mols = []
    for _ in range(n_molecules):
        n = int(rng.integers(n_lo, n_hi + 1))
        p = _self_avoiding_walk(rng, n, 1.1, 1.5, MIN_SEP)
        mols.append(p - p.mean(axis=0))
    r_max = max(float(np.sqrt(np.sum(p * p, axis=1)).max()) for p in mols)
    spacing = 2.0 * r_max + cutoff + 1.0
    side = ceil(n_molecules ** (1.0 / 3.0) - 1e-9)
    while side**3 < n_molecules:
        side += 1
    pos, mol = [], []
    for k, p in enumerate(mols):
        site = np.array([k % side, (k // side) % side, k // (side * side)], dtype=np.float64)
        pos.append(p + spacing * site)
        mol.append(np.full(p.shape[0], k, dtype=np.int32))
    return rng, np.vstack(pos), None, np.concatenate(mol)


def _water_l6(seed, n_side=10, spacing=3.1):
    rng = np.random.default_rng(seed)
    side = n_side * spacing
    g = (np.arange(n_side) + 0.5) * spacing
    sites = np.stack(np.meshgrid(g, g, g, indexing="ij"), axis=-1).reshape(-1, 3)
    box = np.array([side, side, side])
    pos = _place_waters(rng, sites, 0.25, box)
    return rng, pos, box, None


def _solvated_protein(seed, n_protein=3000, n_water=9000, side=67.0, n_lattice=22, density=0.1):
    rng = np.random.default_rng(seed)
    center = np.full(3, side / 2.0)
    radius = (3.0 * n_protein / (4.0 * np.pi * density)) ** (1.0 / 3.0)
    prot = _confined_walk(rng, n_protein, 1.5, MIN_SEP, center, radius)
    spacing = side / n_lattice
    g = (np.arange(n_lattice) + 0.5) * spacing
    grid = np.stack(np.meshgrid(g, g, g, indexing="ij"), axis=-1).reshape(-1, 3)
    keep = np.sum((grid - center) ** 2, axis=1) >= (radius + 1.0) ** 2
    grid = grid[keep]
    if grid.shape[0] < n_water:
        raise ValueError("not enough water sites")
    pick = np.sort(rng.choice(grid.shape[0], size=n_water, replace=False))
    box = np.array([side, side, side])
    waters = _place_waters(rng, grid[pick], 0.25, box, fixed=prot)
    return rng, np.vstack([prot, waters]), box, None


def _water_100k(seed, n_atoms=100_000):
    rng = np.random.default_rng(seed)
    pos, side = water_box_positions(rng, n_atoms)
    return rng, pos, np.array([side, side, side]), None


CONFIGS = {
    "tiny_fp32": dict(seed=0, gen=_tiny, cutoff=5.0, l_max=2, channels=16, heads=2, n_rbf=8, dtype="fp32"),
    "small_molecules": dict(seed=1, gen=_small_molecules, cutoff=6.0, l_max=4, channels=128, heads=8, n_rbf=16, dtype="bf16"),
    "water_l6": dict(seed=2, gen=_water_l6, cutoff=6.0, l_max=6, channels=128, heads=8, n_rbf=16, dtype="bf16"),
    "solvated_protein": dict(seed=3, gen=_solvated_protein, cutoff=6.0, l_max=4, channels=128, heads=8, n_rbf=16, dtype="bf16"),
    "water_100k": dict(seed=4, gen=_water_100k, cutoff=5.0, l_max=4, channels=128, heads=8, n_rbf=16, dtype="bf16"),
}


def make_workload(name: str, *, geometry=None, with_features=True, **overrides) -> Workload:
    """Build a named workload.  `geometry` passes keyword arguments to the
    position generator (e.g. n_molecules=8 for a smaller batch of the same
    kind); other keyword arguments override l_max, channels, heads, n_rbf,
    dtype, cutoff, envelope_p or seed."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    gen = cfg.pop("gen")
    geo = dict(geometry or {})
    if gen is _small_molecules:
        geo.setdefault("cutoff", cfg["cutoff"])
    rng, pos, box, mol = gen(cfg["seed"], **geo)
    pos32 = pos.astype(np.float32)
    n = pos32.shape[0]
    L, C, K = cfg["l_max"], cfg["channels"], cfg["n_rbf"]
    if with_features:
        x, w_q, w_k, w_rad, w_so2 = _draw_features_and_weights(rng, n, L, C, K, cfg["dtype"])
    else:
        x = w_q = w_k = w_rad = w_so2 = None
    return Workload(
        name=name,
        pos=pos32,
        box=None if box is None else np.asarray(box, dtype=np.float32),
        mol_id=mol,
        cutoff=float(np.float32(cfg["cutoff"])),
        l_max=L,
        channels=C,
        heads=cfg["heads"],
        n_rbf=K,
        envelope_p=cfg.get("envelope_p", 5),
        dtype=cfg["dtype"],
        x=x,
        w_q=w_q,
        w_k=w_k,
        w_rad=w_rad,
        w_so2=w_so2,
        meta=dict(seed=cfg["seed"], geometry=geo),
    )
