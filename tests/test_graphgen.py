"""The seeded input generators: determinism, shape and structure."""
import hashlib

import numpy as np
import pytest

import graphgen as gg
import oracle


def _sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def _is_clean_symmetric(g):
    from scipy.sparse import csr_matrix
    A = csr_matrix((np.ones(g.m), g.col_idx, g.row_ptr), shape=(g.n, g.n))
    if (A != A.T).nnz:
        return False
    rows = np.repeat(np.arange(g.n), np.diff(g.row_ptr))
    if (rows == g.col_idx).any():
        return False
    # strictly increasing inside each row: no duplicates, sorted
    same_row = rows[1:] == rows[:-1]
    return bool((g.col_idx[1:][same_row] > g.col_idx[:-1][same_row]).all())


def test_rmat_deterministic_and_clean():
    a = gg.rmat(12, 16, seed=7, nsrc=8)
    b = gg.rmat(12, 16, seed=7, nsrc=8)
    assert _sha(a.row_ptr) == _sha(b.row_ptr) and _sha(a.col_idx) == _sha(b.col_idx)
    assert (a.sources == b.sources).all()
    assert _is_clean_symmetric(a)
    assert a.n == 4096 and 0 < a.m <= 2 * 16 * 4096
    deg = a.degrees()
    assert (deg[a.sources] >= 1).all()
    # skewed: the largest degree is far above the mean
    assert deg.max() > 20 * deg.mean()
    c = gg.rmat(12, 16, seed=8, nsrc=8)
    assert _sha(c.col_idx) != _sha(a.col_idx)


def test_er_shape():
    g = gg.erdos_renyi(1 << 14, 8, seed=3, nsrc=8)
    assert _is_clean_symmetric(g)
    deg = g.degrees()
    assert abs(deg.mean() - 16) < 0.5 and deg.max() < 45


def test_grid_damaged_shape():
    g = gg.grid_damaged(64, 48, 0.05, seed=4)
    E = 2 * 64 * 48 - 64 - 48
    assert g.meta["deleted"] == round(0.05 * E)
    assert _is_clean_symmetric(g)
    assert g.n <= 64 * 48 and g.n > 0.9 * 64 * 48
    assert g.m <= 2 * (E - g.meta["deleted"])
    dist, _, _, L = oracle.bfs(g.row_ptr, g.col_idx, g.sources[0])
    assert (dist >= 0).all()          # largest component only
    assert L >= 64 + 48 - 1           # at least the Manhattan distance to the far corner


def test_c1_shape_and_source():
    g = gg.c1_chung_lu()
    deg = g.degrees()
    # the configuration: about 3,485 vertices (largest component), about 31k
    # entries, median degree 3, mean about 9, max about 1,255, about 10 levels
    assert 3400 <= g.n <= 3485
    assert 29000 <= g.m <= 33000
    assert np.median(deg) == 3
    assert 8 <= deg.mean() <= 10
    assert 1100 <= deg.max() <= 1400
    assert _is_clean_symmetric(g)
    assert 8 <= oracle.bfs(g.row_ptr, g.col_idx, int(g.sources[0]))[3] <= 12
    # the chosen source has the largest eccentricity, by the oracle over all vertices
    levels, reached = oracle.bfs_many(g.row_ptr, g.col_idx, np.arange(g.n, dtype=np.int32))
    assert (reached == g.n).all()
    s = int(g.sources[0])
    assert levels[s] == levels.max()


def test_tiny_random_variety():
    kinds = set()
    for seed in range(200):
        g = gg.tiny_random(seed)
        assert g.row_ptr[0] == 0 and (np.diff(g.row_ptr) >= 0).all()
        assert g.col_idx.shape[0] == g.m
        if g.m:
            assert g.col_idx.min() >= 0 and g.col_idx.max() < g.n
        rows = np.repeat(np.arange(g.n), np.diff(g.row_ptr))
        kinds.add(("directed" if g.meta["directed"] else "sym",
                   bool((rows == g.col_idx).any())))
    assert len(kinds) == 4


def test_rmat_directed_clean():
    """Directed R-MAT: deterministic, no self-loops, no duplicate entries,
    sorted rows, not symmetric; sources have out-degree >= 1."""
    g1 = gg.rmat_directed(10, 16, seed=9, nsrc=4)
    g2 = gg.rmat_directed(10, 16, seed=9, nsrc=4)
    assert (g1.row_ptr == g2.row_ptr).all() and (g1.col_idx == g2.col_idx).all()
    assert not g1.symmetric
    rows = np.repeat(np.arange(g1.n), np.diff(g1.row_ptr))
    assert (rows != g1.col_idx).all()
    for u in range(g1.n):
        r = g1.col_idx[g1.row_ptr[u]:g1.row_ptr[u + 1]]
        assert (np.diff(r) > 0).all()
    fwd = set(zip(rows.tolist(), g1.col_idx.tolist()))
    assert any((v, u) not in fwd for u, v in fwd)
    assert (np.diff(g1.row_ptr)[g1.sources] >= 1).all()

