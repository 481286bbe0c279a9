"""Reference oracle for level-synchronous BFS over an int32 CSR graph.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may use this package; the product path never does.  It
shares no code with the HIP library (``frontier_bfs_csr_amd``) and imports
nothing from it.

The BFS itself is plain C (``bfs_oracle.c``, built with gcc, no HIP headers):
a serial FIFO-queue BFS as in the sequential baseline of "Chapter 22: The
Frontier Model for Parallel Breadth-First Search" (section 22.1) and
``bfsCpu`` of the Day 38 program (bfs.cu), plus a checker that applies the
gates of that program's ``main`` (exact dist, level count, frontier sizes
summing to the reached count) and the BFS-parent and edge invariants, and
the neighbour-walk checksum that the Day 38 page's isolated level walk checks
its kernels against, and single-source shortest paths (Dijkstra, with the
smallest tight in-neighbour as predecessor) for the atomic-min relaxation
the Gunrock reading guide extends the same lambda to.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bfs_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CHECK_CODES = {
    0: "ok",
    1: "dist differs from the oracle",
    2: "level count differs",
    3: "level size differs",
    4: "level sizes do not sum to the reached count",
    5: "parent[source] != source",
    6: "dist[parent[v]] != dist[v] - 1",
    7: "v is not a neighbour of parent[v]",
    8: "unreached vertex has a parent",
    9: "symmetric edge invariant violated",
    10: "directed edge invariant violated",
    11: "bad arguments",
    12: "out of memory",
}

_lib = None
_lib_path = _LIB


def build(force: bool = True, mutant: int = 0, out: str | None = None) -> str:
    """Compile bfs_oracle.c into liboracle.so beside it (gcc -O2).

    ``mutant`` > 0 builds a deliberately broken variant (see ORACLE_MUTANT in
    the C source) into ``out``; only the mutation tests do that.
    """
    target = out or _LIB
    if force or not os.path.exists(target):
        tmp = target + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp]
        if mutant:
            cmd.insert(1, f"-DORACLE_MUTANT={int(mutant)}")
        subprocess.check_call(cmd)
        os.replace(tmp, target)
    return target


@contextlib.contextmanager
def use_library(path: str):
    """Temporarily route every oracle call through another build (mutants)."""
    global _lib, _lib_path
    saved = (_lib, _lib_path)
    _lib, _lib_path = None, path
    try:
        yield
    finally:
        _lib, _lib_path = saved


def _load():
    global _lib
    if _lib is None:
        if _lib_path == _LIB and not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_lib_path)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.oracle_bfs.argtypes = [i32, P, P, i32, P, P, P, P]
        lib.oracle_bfs.restype = i32
        lib.oracle_bfs_many.argtypes = [i32, P, P, i32, P, P, P, P]
        lib.oracle_bfs_many.restype = i32
        lib.oracle_check.argtypes = [i32, P, P, i32, P, i32, P, P, P, i32, P, i32,
                                     ctypes.POINTER(i64)]
        lib.oracle_check.restype = i32
        lib.oracle_walk_checksum.argtypes = [i32, P, P, i32, P, i32, P]
        lib.oracle_walk_checksum.restype = i32
        lib.oracle_sssp.argtypes = [i32, P, P, P, i32, P, P]
        lib.oracle_sssp.restype = i32
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def bfs(row_ptr, col_idx, source, *, want_order=False):
    """Serial FIFO BFS.  Returns (dist, parent, level_sizes[:L], L[, order]).

    dist/parent are int32 with -1 for unreached vertices; parent[source] is
    source.  ``order`` is the FIFO dequeue order of the reached vertices.
    """
    lib = _load()
    row_ptr, col_idx = _i32(row_ptr), _i32(col_idx)
    n = row_ptr.shape[0] - 1
    dist = np.empty(n, np.int32)
    parent = np.empty(n, np.int32)
    sizes = np.empty(n, np.int32)
    order = np.empty(n, np.int32)
    L = lib.oracle_bfs(n, _ptr(row_ptr), _ptr(col_idx), int(source), _ptr(dist),
                       _ptr(parent), _ptr(sizes), _ptr(order))
    if L < 0:
        raise ValueError(f"oracle_bfs failed with {L}")
    if want_order:
        reached = int(sizes[:L].sum())
        return dist, parent, sizes[:L].copy(), L, order[:reached].copy()
    return dist, parent, sizes[:L].copy(), L


def bfs_many(row_ptr, col_idx, sources):
    """BFS from each source in turn; returns (levels[nsrc], reached[nsrc])."""
    lib = _load()
    row_ptr, col_idx = _i32(row_ptr), _i32(col_idx)
    n = row_ptr.shape[0] - 1
    src = _i32(sources)
    dist = np.empty(n, np.int32)
    levels = np.empty(src.shape[0], np.int32)
    reached = np.empty(src.shape[0], np.int64)
    rc = lib.oracle_bfs_many(n, _ptr(row_ptr), _ptr(col_idx), src.shape[0], _ptr(src),
                             _ptr(dist), _ptr(levels), _ptr(reached))
    if rc != 0:
        raise ValueError(f"oracle_bfs_many failed with {rc}")
    return levels, reached


def walk_checksum(row_ptr, col_idx, vertices, repeats=64):
    """Per-vertex neighbour-walk checksums (uint32) of the listed vertices:
    the wrapping sum over repeats r and CSR entries of (neighbour XOR r), as
    the Day 38 page's isolated level walk defines it."""
    lib = _load()
    row_ptr, col_idx = _i32(row_ptr), _i32(col_idx)
    n = row_ptr.shape[0] - 1
    v = _i32(vertices)
    out = np.empty(v.shape[0], np.uint32)
    rc = lib.oracle_walk_checksum(n, _ptr(row_ptr), _ptr(col_idx), v.shape[0], _ptr(v), int(repeats),
                                  _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_walk_checksum failed with {rc}")
    return out


def sssp(row_ptr, col_idx, weights, source):
    """Shortest-path distances (int64, -1 unreachable) and predecessors (int32:
    the smallest tight in-neighbour, the source's own id for the source, -1
    unreachable) from ``source``, with weights[e] >= 0 on CSR entry e."""
    lib = _load()
    row_ptr, col_idx = _i32(row_ptr), _i32(col_idx)
    w = np.ascontiguousarray(weights, dtype=np.uint32)
    n = row_ptr.shape[0] - 1
    if w.shape[0] != col_idx.shape[0]:
        raise ValueError("one weight per CSR entry")
    dist = np.empty(n, np.int64)
    pred = np.empty(n, np.int32)
    rc = lib.oracle_sssp(n, _ptr(row_ptr), _ptr(col_idx), _ptr(w), int(source), _ptr(dist), _ptr(pred))
    if rc != 0:
        raise ValueError(f"oracle_sssp failed with {rc}")
    return dist, pred


def check(row_ptr, col_idx, source, ref, dist, parent=None, L=None, sizes=None,
          symmetric=True):
    """Check a BFS result against the oracle's ``ref = (dist, parent, sizes, L)``.

    Returns (code, bad_index); code 0 means every gate passed.
    """
    lib = _load()
    row_ptr, col_idx = _i32(row_ptr), _i32(col_idx)
    n = row_ptr.shape[0] - 1
    ref_dist, _, ref_sizes, ref_L = ref
    ref_dist, ref_sizes = _i32(ref_dist), _i32(ref_sizes)
    dist = _i32(dist)
    parent = None if parent is None else _i32(parent)
    if L is None:
        L = ref_L
    sizes = None if sizes is None else _i32(sizes)
    if sizes is not None and sizes.shape[0] < L:
        return 3, sizes.shape[0]
    bad = ctypes.c_int64(-1)
    code = lib.oracle_check(n, _ptr(row_ptr), _ptr(col_idx), int(source), _ptr(ref_dist),
                            int(ref_L), _ptr(ref_sizes), _ptr(dist), _ptr(parent), int(L),
                            _ptr(sizes), 1 if symmetric else 0, ctypes.byref(bad))
    return int(code), int(bad.value)


def assert_bfs_ok(row_ptr, col_idx, source, ref, dist, parent=None, L=None, sizes=None,
                  symmetric=True, label=""):
    code, bad = check(row_ptr, col_idx, source, ref, dist, parent, L, sizes, symmetric)
    if code != 0:
        extra = ""
        if code == 1:
            extra = f" (got {int(np.asarray(dist)[bad])}, oracle {int(ref[0][bad])})"
        raise AssertionError(f"{label}: {CHECK_CODES.get(code, code)} at index {bad}{extra}")
