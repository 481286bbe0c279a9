"""Seeded synthetic graphs in int32 CSR form (row_ptr, col_idx).

Input preparation shared by the oracle tests, the HIP parity tests and the
benchmark.  It holds no BFS arithmetic: it builds graphs and picks sources.

Workload shapes follow the pages' workloads, as stand-ins (no dataset is read):

* ``c1_chung_lu``  -- small undirected power-law graph shaped like the word
  graph of "Day 38 - Graph traversal on a GPU" (Results: 3,485 vertices,
  median degree 3, max degree 1,255): Chung-Lu with power-law expected degrees
  (exponent 2.1), truncated; largest connected component kept.
* ``rmat``         -- R-MAT (Chakrabarti, Zhan, Faloutsos, SDM 2004) with
  (a,b,c,d) = (0.57,0.19,0.19,0.05), edge factor 16, seeded relabelling
  permutation, self-loops and duplicates removed, symmetrised.  Scale 20 and 24
  are the two R-MAT workloads; smaller scales serve the tests.
* ``erdos_renyi``  -- 8n uniform endpoint pairs, symmetrised (mean degree 16).
* ``grid_damaged`` -- w x h 4-neighbour grid with a fixed share of its edges
  deleted by a seeded shuffle, largest component kept, row-major labels.

Random numbers: numpy's PCG64 for the numpy generators; SplitMix64 in the C
helper (``csrgen.c``) for R-MAT.  Small closed-form graphs (paths, stars,
complete graphs, full grids) and tiny random graphs (directed or not, with
self-loops and duplicates) serve the parity tests.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csrgen.c")
_LIB = os.path.join(_HERE, "libcsrgen.so")
_lib = None

RMAT_ABCD = (0.57, 0.19, 0.19, 0.05)


def build(force: bool = True) -> str:
    """Compile csrgen.c into libcsrgen.so beside it (gcc -O3 -fopenmp)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-std=gnu11", "-fopenmp", "-shared", "-fPIC",
                               "-Wall", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.gen_permutation.argtypes = [ctypes.c_int32, ctypes.c_uint64, P]
        lib.gen_permutation.restype = None
        lib.gen_rmat_edges.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_double,
                                       ctypes.c_double, ctypes.c_double, ctypes.c_uint64,
                                       P, P, P]
        lib.gen_rmat_edges.restype = None
        lib.csr_build.argtypes = [ctypes.c_int32, ctypes.c_int64, P, P, P,
                                  ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)]
        lib.csr_build.restype = ctypes.c_void_p
        lib.csr_finish.argtypes = [ctypes.c_void_p, P]
        lib.csr_finish.restype = None
        _lib = lib
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


@dataclasses.dataclass
class Graph:
    """An int32 CSR graph plus the sources its workload runs BFS from."""
    name: str
    row_ptr: np.ndarray
    col_idx: np.ndarray
    symmetric: bool
    sources: np.ndarray
    meta: dict = dataclasses.field(default_factory=dict)

    @property
    def n(self) -> int:
        return int(self.row_ptr.shape[0] - 1)

    @property
    def m(self) -> int:
        return int(self.row_ptr[-1])

    def degrees(self) -> np.ndarray:
        return np.diff(self.row_ptr).astype(np.int64)


# --------------------------------------------------------------- builders --

def csr_from_lists(n, adj):
    """CSR from a list of neighbour lists, kept as given (order, duplicates,
    self-loops all preserved)."""
    deg = np.array([len(a) for a in adj], dtype=np.int64)
    row_ptr = np.zeros(n + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum(deg)
    col = np.array([v for a in adj for v in a], dtype=np.int32)
    return row_ptr, col


def csr_from_directed_edges(n, src, dst):
    """CSR of a directed edge list, rows in stable input order (no dedup)."""
    src = np.asarray(src, dtype=np.int64)
    dst = np.asarray(dst, dtype=np.int32)
    order = np.argsort(src, kind="stable")
    deg = np.bincount(src, minlength=n)
    row_ptr = np.zeros(n + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum(deg)
    return row_ptr, dst[order].astype(np.int32)


def symmetric_csr(n, src, dst):
    """Symmetric closure of an edge list as sorted, deduplicated CSR without
    self-loops (C helper, OpenMP)."""
    lib = _load()
    src = np.ascontiguousarray(src, dtype=np.int32)
    dst = np.ascontiguousarray(dst, dtype=np.int32)
    E = src.shape[0]
    row_ptr = np.empty(n + 1, dtype=np.int32)
    m = ctypes.c_int64(0)
    err = ctypes.c_int32(0)
    h = lib.csr_build(n, E, _p(src), _p(dst), _p(row_ptr), ctypes.byref(m), ctypes.byref(err))
    if not h:
        raise ValueError(f"csr_build failed ({err.value})")
    col = np.empty(int(m.value), dtype=np.int32)
    lib.csr_finish(h, _p(col))
    return row_ptr, col


def largest_component(row_ptr, col_idx):
    """Keep the largest connected component, relabelled in original order.
    Returns (row_ptr, col_idx, old_ids)."""
    from scipy.sparse import csr_matrix
    from scipy.sparse.csgraph import connected_components
    n = row_ptr.shape[0] - 1
    data = np.ones(col_idx.shape[0], dtype=np.int8)
    A = csr_matrix((data, col_idx, row_ptr), shape=(n, n))
    ncomp, labels = connected_components(A, directed=False)
    del A, data
    counts = np.bincount(labels, minlength=ncomp)
    keep = labels == int(np.argmax(counts))
    old_ids = np.flatnonzero(keep).astype(np.int32)
    new_id = np.full(n, -1, dtype=np.int32)
    new_id[old_ids] = np.arange(old_ids.shape[0], dtype=np.int32)
    deg = np.diff(row_ptr)
    kdeg = deg[old_ids]
    new_row = np.zeros(old_ids.shape[0] + 1, dtype=np.int32)
    new_row[1:] = np.cumsum(kdeg)
    row_of_entry = np.repeat(keep, deg)
    new_col = new_id[col_idx[row_of_entry]]
    assert (new_col >= 0).all()
    return new_row, new_col.astype(np.int32), old_ids


def pick_sources(row_ptr, count, seed):
    """`count` distinct sources, uniform over vertices of degree >= 1."""
    deg = np.diff(row_ptr)
    cand = np.flatnonzero(deg > 0)
    rng = np.random.Generator(np.random.PCG64(seed))
    k = min(count, cand.shape[0])
    return np.sort(rng.choice(cand, size=k, replace=False)).astype(np.int32)


# ------------------------------------------------------ pinned page graphs --

def chapter22_graph():
    """The 6-vertex directed CSR graph of Chapter 22 (section 22.1)."""
    row_ptr = np.array([0, 2, 4, 6, 8, 9, 9], dtype=np.int32)
    col_idx = np.array([1, 2, 2, 3, 3, 4, 4, 5, 5], dtype=np.int32)
    return Graph("chapter22_6v", row_ptr, col_idx, False, np.array([0], np.int32))


def pmpp_graph():
    """The 4-vertex undirected CSR graph (edges 0-1, 0-2, 1-2, 2-3) of the
    PMPP ch.15 notes, section 15.1."""
    row_ptr = np.array([0, 2, 4, 7, 8], dtype=np.int32)
    col_idx = np.array([1, 2, 0, 2, 0, 1, 3, 2], dtype=np.int32)
    return Graph("pmpp_4v", row_ptr, col_idx, True, np.array([0, 3], np.int32))


# ------------------------------------------------------------ closed forms --

def path_graph(n):
    src = np.arange(n - 1)
    r, c = symmetric_csr(n, src, src + 1) if n > 1 else (np.zeros(2, np.int32),
                                                         np.zeros(0, np.int32))
    return Graph(f"path_{n}", r, c, True, np.array([0], np.int32))


def star_graph(n):
    """Vertex 0 joined to 1..n-1."""
    leaves = np.arange(1, n)
    r, c = symmetric_csr(n, np.zeros(n - 1, np.int64), leaves)
    return Graph(f"star_{n}", r, c, True, np.array([0, n - 1], np.int32))


def complete_graph(n):
    i, j = np.triu_indices(n, 1)
    r, c = symmetric_csr(n, i, j)
    return Graph(f"complete_{n}", r, c, True, np.array([0], np.int32))


def grid_full(w, h):
    """Full w x h 4-neighbour grid, id = r*w + c."""
    ids = np.arange(w * h).reshape(h, w)
    src = np.concatenate([ids[:, :-1].ravel(), ids[:-1, :].ravel()])
    dst = np.concatenate([ids[:, 1:].ravel(), ids[1:, :].ravel()])
    r, c = symmetric_csr(w * h, src, dst)
    return Graph(f"grid_{w}x{h}", r, c, True, np.array([0], np.int32))


def disjoint_union(g1: Graph, g2: Graph):
    n1 = g1.n
    row = np.concatenate([g1.row_ptr[:-1], g2.row_ptr + g1.m]).astype(np.int32)
    col = np.concatenate([g1.col_idx, g2.col_idx + n1]).astype(np.int32)
    return Graph(f"{g1.name}+{g2.name}", row, col, g1.symmetric and g2.symmetric,
                 np.array([0, n1], np.int32))


# ------------------------------------------------------ tiny random graphs --

def tiny_random(seed, n=None, directed=None, p=None, self_loops=True, duplicates=True):
    """A tiny random graph (n <= 64) kept raw: rows unsorted, optional
    self-loops and duplicate entries, directed or symmetric, possibly
    disconnected."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if n is None:
        n = int(rng.integers(1, 65))
    if directed is None:
        directed = bool(rng.integers(0, 2))
    if p is None:
        p = float(rng.choice([0.02, 0.05, 0.1, 0.2, 0.5]))
    A = rng.random((n, n)) < p
    if not self_loops:
        np.fill_diagonal(A, False)
    if not directed:
        A = np.triu(A) | np.triu(A).T
    src, dst = np.nonzero(A)
    if duplicates and src.shape[0] > 0:
        k = int(rng.integers(0, src.shape[0] + 1))
        pick = rng.integers(0, src.shape[0], size=k)
        extra_s, extra_d = src[pick], dst[pick]
        if not directed:
            extra_s, extra_d = np.concatenate([extra_s, extra_d]), np.concatenate([extra_d, extra_s])
        src = np.concatenate([src, extra_s])
        dst = np.concatenate([dst, extra_d])
    perm = rng.permutation(src.shape[0])
    src, dst = src[perm], dst[perm]
    row_ptr, col = csr_from_directed_edges(n, src, dst)
    srcs = np.unique(rng.integers(0, n, size=min(n, 4))).astype(np.int32)
    return Graph(f"tiny_{seed}", row_ptr, col, not directed, srcs,
                 {"directed": directed, "p": p})


def edge_weights(m, seed, wmax=255, wmin=1):
    """One non-negative integer weight per CSR entry, uniform in [wmin, wmax]
    (numpy PCG64, seeded); the pages supply no weights."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(wmin, wmax + 1, size=int(m), dtype=np.uint64).astype(np.uint32)


def random_directed(n, avg_deg, seed):
    """Directed graph with n*avg_deg uniform edges (duplicates and self-loops
    kept), rows in random order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    E = int(n * avg_deg)
    src = rng.integers(0, n, size=E)
    dst = rng.integers(0, n, size=E)
    row_ptr, col = csr_from_directed_edges(n, src, dst)
    return Graph(f"dir_{n}_{avg_deg}", row_ptr, col, False, pick_sources(row_ptr, 4, seed + 1))


# -------------------------------------------------------------- workloads --

def rmat(scale, edge_factor=16, seed=5, perm_seed=None, nsrc=64, src_seed=None):
    """Undirected R-MAT graph at `scale` (see module docstring)."""
    lib = _load()
    n = 1 << scale
    E = edge_factor * n
    perm = np.empty(n, dtype=np.int32)
    lib.gen_permutation(n, ctypes.c_uint64(perm_seed if perm_seed is not None else seed + 1000),
                        _p(perm))
    src = np.empty(E, dtype=np.int32)
    dst = np.empty(E, dtype=np.int32)
    a, b, c, _ = RMAT_ABCD
    lib.gen_rmat_edges(scale, E, a, b, c, ctypes.c_uint64(seed), _p(perm), _p(src), _p(dst))
    del perm
    row_ptr, col = symmetric_csr(n, src, dst)
    del src, dst
    srcs = pick_sources(row_ptr, nsrc, src_seed if src_seed is not None else seed + 100)
    return Graph(f"rmat{scale}_ef{edge_factor}", row_ptr, col, True, srcs,
                 {"scale": scale, "edge_factor": edge_factor, "seed": seed})


def rmat_directed(scale, edge_factor=16, seed=6, nsrc=64, src_seed=None):
    """Directed R-MAT graph at `scale`: the same edge generator and relabelling
    as ``rmat`` without the symmetric closure; self-loops and duplicate edges
    removed, rows sorted.  Sources have out-degree >= 1."""
    lib = _load()
    n = 1 << scale
    E = edge_factor * n
    perm = np.empty(n, dtype=np.int32)
    lib.gen_permutation(n, ctypes.c_uint64(seed + 1000), _p(perm))
    src = np.empty(E, dtype=np.int32)
    dst = np.empty(E, dtype=np.int32)
    a, b, c, _ = RMAT_ABCD
    lib.gen_rmat_edges(scale, E, a, b, c, ctypes.c_uint64(seed), _p(perm), _p(src), _p(dst))
    del perm
    keep = src != dst
    key = np.unique(src[keep].astype(np.int64) * n + dst[keep])
    del src, dst, keep
    row_ptr, col = csr_from_directed_edges(n, key // n, key % n)
    srcs = pick_sources(row_ptr, nsrc, src_seed if src_seed is not None else seed + 100)
    return Graph(f"rmat{scale}_ef{edge_factor}_directed", row_ptr, col, False, srcs,
                 {"scale": scale, "edge_factor": edge_factor, "seed": seed})


def erdos_renyi(n=4_194_304, pairs_per_vertex=8, seed=3, nsrc=64):
    """Undirected uniform random graph: n*pairs_per_vertex uniform pairs,
    symmetrised and deduplicated (mean degree ~ 2*pairs_per_vertex)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    E = n * pairs_per_vertex
    src = rng.integers(0, n, size=E, dtype=np.int32)
    dst = rng.integers(0, n, size=E, dtype=np.int32)
    row_ptr, col = symmetric_csr(n, src, dst)
    return Graph(f"er_{n}", row_ptr, col, True, pick_sources(row_ptr, nsrc, seed + 100),
                 {"seed": seed})


def grid_damaged(w=4096, h=4096, delete_frac=0.05, seed=4):
    """w x h 4-neighbour grid, floor(delete_frac * edges) edges deleted by a
    seeded shuffle, largest component kept (row-major order).  Source: corner
    (0,0), else the first of the other three corners inside the component."""
    ids = np.arange(w * h, dtype=np.int64).reshape(h, w)
    src = np.concatenate([ids[:, :-1].ravel(), ids[:-1, :].ravel()])
    dst = np.concatenate([ids[:, 1:].ravel(), ids[1:, :].ravel()])
    E = src.shape[0]
    ndel = int(round(delete_frac * E))
    rng = np.random.Generator(np.random.PCG64(seed))
    keep = np.ones(E, dtype=bool)
    keep[rng.permutation(E)[:ndel]] = False
    row_ptr, col = symmetric_csr(w * h, src[keep], dst[keep])
    del src, dst, keep
    row_ptr, col, old = largest_component(row_ptr, col)
    corners = [0, w - 1, (h - 1) * w, h * w - 1]
    pos = np.searchsorted(old, corners)
    source = None
    for cidx, p in zip(corners, pos):
        if p < old.shape[0] and old[p] == cidx:
            source = int(p)
            break
    return Graph(f"grid{w}x{h}_del{delete_frac}", row_ptr, col, True,
                 np.array([source], np.int32),
                 {"w": w, "h": h, "deleted": ndel, "edges_before": E, "seed": seed})


# Truncated power-law expected degrees for the small Chung-Lu workload,
# calibrated once by a deterministic grid search on seed 1 over (n0, w_hi,
# i_scale) so that the kept component has about the word graph's 3,485
# vertices and ~31k CSR entries, median degree ~3, mean ~9 and max ~1,255:
# n0 = 3,740 generated vertices leave a component of 3,482 vertices and
# 30,418 entries (median 3, mean 8.74, max 1,275).  The word graph is itself
# one large component with a few strays (its search reaches 3,434 of 3,485).
CHUNG_LU_PARAMS = {"n0": 3740, "gamma": 2.1, "w_hi": 2550.0, "i_scale": 1.1, "w_lo": 1.0}


def chung_lu_weights(n0, gamma, w_hi, i_scale, w_lo):
    i = np.arange(n0, dtype=np.float64)
    w = w_hi * (i / i_scale + 1.0) ** (-1.0 / (gamma - 1.0))
    return np.maximum(w, w_lo)


def chung_lu(n0, gamma, w_hi, i_scale, w_lo, seed=1):
    """Chung-Lu graph: edge {i,j} (i<j) with probability min(1, w_i w_j / sum w);
    largest component kept.  Returns (row_ptr, col_idx)."""
    w = chung_lu_weights(n0, gamma, w_hi, i_scale, w_lo)
    S = w.sum()
    rng = np.random.Generator(np.random.PCG64(seed))
    iu, ju = np.triu_indices(n0, 1)
    p = np.minimum(1.0, w[iu] * w[ju] / S)
    take = rng.random(iu.shape[0]) < p
    row_ptr, col = symmetric_csr(n0, iu[take], ju[take])
    row_ptr, col, _ = largest_component(row_ptr, col)
    return row_ptr, col


def max_eccentricity_source(row_ptr, col_idx, seed=101):
    """Vertex of largest eccentricity (scipy's unweighted shortest paths, a
    library routine independent of the oracle and of the HIP path); ties are
    broken by a seeded pick."""
    from scipy.sparse import csr_matrix
    from scipy.sparse.csgraph import shortest_path
    n = row_ptr.shape[0] - 1
    A = csr_matrix((np.ones(col_idx.shape[0]), col_idx, row_ptr), shape=(n, n))
    D = shortest_path(A, method="D", unweighted=True)
    D[np.isinf(D)] = -1
    ecc = D.max(axis=1)
    best = np.flatnonzero(ecc == ecc.max())
    rng = np.random.Generator(np.random.PCG64(seed))
    return int(rng.choice(best)), int(ecc.max())


def c1_chung_lu():
    row_ptr, col = chung_lu(**CHUNG_LU_PARAMS, seed=1)
    s, ecc = max_eccentricity_source(row_ptr, col, seed=101)
    return Graph("c1_chung_lu_3485", row_ptr, col, True, np.array([s], np.int32),
                 {"eccentricity": ecc, **CHUNG_LU_PARAMS})


def c2_rmat20(nsrc=64):
    return rmat(20, 16, seed=2, nsrc=nsrc, src_seed=102)


def c3_er(nsrc=64):
    return erdos_renyi(4_194_304, 8, seed=3, nsrc=nsrc)


def c4_grid():
    return grid_damaged(4096, 4096, 0.05, seed=4)


def c5_rmat24(nsrc=64):
    return rmat(24, 16, seed=5, nsrc=nsrc, src_seed=105)


WORKLOADS = {
    "c1": c1_chung_lu,
    "c2": c2_rmat20,
    "c3": c3_er,
    "c4": c4_grid,
    "c5": c5_rmat24,
}
