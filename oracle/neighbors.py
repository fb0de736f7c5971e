"""Brute-force radius graph, fp64, O(N^2).  Test infrastructure (see
oracle/__init__).

E2Former-V2 summary, technical section 2.2: attention runs over the
neighbours j in N(i) within a cutoff radius (and section 1: |E| ~ kN).  The
pages do not fix the boundary or the arithmetic, so this is the reading the
GPU builder must reproduce bit for bit:

* j is a neighbour of i iff j != i, mol_id[j] == mol_id[i] (when given),
  and s < rc*rc, with rc the fp32 cutoff widened to fp64 and squared in
  fp64;
* dx = float64(p_j.x) - float64(p_i.x); with a box side b (fp32 widened),
  dx = dx - b * rint(dx / b) (rint rounds half to even); same for y, z;
* s = (dx*dx + dy*dy) + dz*dz in that order, every operation rounded
  separately (numpy ufuncs never fuse a multiply into an add);
* CSR output with j ascending inside each row.
"""

import numpy as np


def neighbors_bruteforce(pos, cutoff, box=None, mol_id=None, rows=None):
    """Return (row_ptr int32 [N+1], col int32 [E]); with `rows`, return the
    sorted neighbour arrays of just those atoms (for sampled checks)."""
    p = np.asarray(pos, dtype=np.float32).astype(np.float64)
    n = p.shape[0]
    rc = np.float64(np.float32(cutoff))
    rc2 = rc * rc
    b = None if box is None else np.asarray(box, dtype=np.float32).astype(np.float64)
    mol = None if mol_id is None else np.asarray(mol_id)
    idx = np.arange(n)
    if rows is not None:
        return [_row(p, i, idx, rc2, b, mol) for i in rows]
    counts = np.zeros(n, dtype=np.int64)
    cols = []
    for i in range(n):
        js = _row(p, i, idx, rc2, b, mol)
        counts[i] = js.size
        cols.append(js)
    row_ptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col = np.concatenate(cols) if cols else np.zeros(0, dtype=np.int64)
    return row_ptr.astype(np.int32), col.astype(np.int32)


def _row(p, i, idx, rc2, b, mol):
    """Sorted neighbours of atom i (the test of the module docstring)."""
    d = [p[:, a] - p[i, a] for a in range(3)]
    if b is not None:
        d = [d[a] - b[a] * np.rint(d[a] / b[a]) for a in range(3)]
    s = (d[0] * d[0] + d[1] * d[1]) + d[2] * d[2]
    keep = (s < rc2) & (idx != i)
    if mol is not None:
        keep &= mol == mol[i]
    return idx[keep].astype(np.int32)  # ascending by construction
