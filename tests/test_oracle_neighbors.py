"""Pins for the brute-force radius graph: an independent KD-tree search
(scipy) on random systems, the cutoff boundary, periodic wrap, molecule
separation, symmetry and ordering.  The neighbour set N(i) within the cutoff
is what the E2Former-V2 summary's node-centric attention streams over
(technical section 2.2)."""

import numpy as np
import pytest
from scipy.spatial import cKDTree

from oracle import neighbors_bruteforce
from synth import make_workload


def _kdtree_csr(pos, cutoff, box=None, mol=None):
    p = pos.astype(np.float64)
    if box is not None:
        b = box.astype(np.float64)
        p = np.mod(p, b)
        p = np.where(p >= b, 0.0, p)
        tree = cKDTree(p, boxsize=b)
    else:
        tree = cKDTree(p)
    rows = tree.query_ball_point(p, float(cutoff))
    out = []
    for i, r in enumerate(rows):
        r = sorted(j for j in r if j != i and (mol is None or mol[j] == mol[i]))
        out.append(r)
    return out


def _rows(row_ptr, col):
    return [list(col[row_ptr[i] : row_ptr[i + 1]]) for i in range(len(row_ptr) - 1)]


@pytest.mark.parametrize("periodic", [False, True])
def test_matches_independent_kdtree_search(periodic):
    rng = np.random.default_rng(5)
    n, side, rc = 400, 14.0, 3.3
    pos = rng.uniform(-1.0, side + 1.0, size=(n, 3)).astype(np.float32)
    box = np.array([side, side * 1.1, side * 0.9], dtype=np.float32) if periodic else None
    rp, col = neighbors_bruteforce(pos, rc, box)
    assert _rows(rp, col) == _kdtree_csr(pos, rc, box)


def test_workload_small_molecules_subset_matches_kdtree():
    w = make_workload("small_molecules", geometry=dict(n_molecules=12), with_features=False)
    rp, col = neighbors_bruteforce(w.pos, w.cutoff, w.box, w.mol_id)
    assert _rows(rp, col) == _kdtree_csr(w.pos, w.cutoff, None, w.mol_id)


def test_cutoff_is_strict_and_self_excluded():
    rc = np.float32(5.0)
    inside = np.nextafter(np.float32(5.0), np.float32(0.0))
    pos = np.array(
        [[0, 0, 0], [5.0, 0, 0], [0, inside, 0], [0, 0, 0]], dtype=np.float32
    )  # atom 3 sits on atom 0
    rp, col = neighbors_bruteforce(pos, rc)
    rows = _rows(rp, col)
    assert rows[0] == [2, 3]  # exactly rc (atom 1) is excluded
    assert rows[1] == [] or 0 not in rows[1]
    assert rows[3] == [0, 2]


def test_periodic_wrap_and_minimum_image():
    box = np.array([10.0, 10.0, 10.0], dtype=np.float32)
    pos = np.array([[0.5, 5, 5], [9.7, 5, 5], [5, 5, 5], [0.5, 5, 25.0]], dtype=np.float32)
    rp, col = neighbors_bruteforce(pos, 1.0, box)
    rows = _rows(rp, col)
    assert rows[0] == [1, 3]  # across the x face; atom 3 is an image two boxes up
    assert rows[1] == [0, 3]
    assert rows[2] == []


def test_molecules_never_mix():
    pos = np.array([[0, 0, 0], [1, 0, 0], [2, 0, 0]], dtype=np.float32)
    rp, col = neighbors_bruteforce(pos, 1.5, None, np.array([0, 0, 1]))
    assert _rows(rp, col) == [[1], [0], []]


def test_symmetric_sorted_and_counts_consistent():
    w = make_workload("water_l6", with_features=False)
    rp, col = neighbors_bruteforce(w.pos, w.cutoff, w.box)
    assert rp[0] == 0 and rp[-1] == col.size
    pairs = set()
    for i in range(w.n_atoms):
        row = col[rp[i] : rp[i + 1]]
        assert np.all(np.diff(row) > 0)
        assert i not in row
        pairs.update((i, int(j)) for j in row)
    assert all((j, i) in pairs for (i, j) in pairs)
