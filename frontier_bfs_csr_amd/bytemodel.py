"""Algorithmic bytes of one BFS (see csrc/bytemodel.c for the model).

Host-side measurement helper: the numbers feed the roofline fraction the
benchmark reports; nothing on the search path uses it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_PKG, "csrc", "bytemodel.c")
_LIB = os.path.join(_PKG, "libbfs_bytemodel.so")
_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-Wall",
                               _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.bfs_alg_bytes.argtypes = [ctypes.c_int32, P, P, P, P, P, ctypes.c_int32, P, P, ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int64), P, ctypes.POINTER(ctypes.c_int64)]
        lib.bfs_alg_bytes.restype = ctypes.c_int32
        _lib = lib
    return _lib


def transpose(row_ptr, col_idx):
    """In-edge CSR (in_row_ptr, in_col_idx) with every in-list ascending."""
    n = row_ptr.shape[0] - 1
    src = np.repeat(np.arange(n, dtype=np.int64), np.diff(row_ptr))
    key = np.asarray(col_idx, np.int64) * n + src
    key.sort()
    in_rp = np.zeros(n + 1, np.int32)
    in_rp[1:] = np.cumsum(np.bincount(key // n, minlength=n))
    return in_rp, (key % n).astype(np.int32)


def alg_bytes(row_ptr, col_idx, dist, dirs, with_parent=True, in_csr=None, flags=None):
    """Returns (init_bytes, level_bytes[L], finish_bytes) for one search.
    in_csr = (in_row_ptr, in_col_idx) of a directed graph (see transpose);
    None: the graph is symmetric and serves as its own.  flags: the search's
    per-level flags (BfsGraph.level_flags(), plus 16 on level 0 when the
    finishing pass ran); None: every level stores its own dist."""
    lib = _load()
    rp = np.ascontiguousarray(row_ptr, np.int32)
    ci = np.ascontiguousarray(col_idx, np.int32)
    irp, ici = (rp, ci) if in_csr is None else (np.ascontiguousarray(in_csr[0], np.int32),
                                                np.ascontiguousarray(in_csr[1], np.int32))
    d = np.ascontiguousarray(dist, np.int32)
    dr = np.ascontiguousarray(dirs, np.int8)
    L = dr.shape[0]
    out = np.zeros(L, np.int64)
    init = ctypes.c_int64(0)
    fin = ctypes.c_int64(0)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    fl = None if flags is None else np.ascontiguousarray(flags, np.uint8)
    if fl is not None and fl.shape[0] != L:
        raise ValueError("flags must hold one entry per level")
    rc = lib.bfs_alg_bytes(rp.shape[0] - 1, p(rp), p(ci), p(irp), p(ici), p(d), L, p(dr),
                           None if fl is None else p(fl), 1 if with_parent else 0,
                           ctypes.byref(init), p(out), ctypes.byref(fin))
    if rc != 0:
        raise ValueError(f"bfs_alg_bytes failed ({rc})")
    return int(init.value), out, int(fin.value)
