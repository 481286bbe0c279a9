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
        lib.bfs_alg_bytes.argtypes = [ctypes.c_int32, P, P, P, P, P, ctypes.c_int32, P, ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int64), P]
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


def alg_bytes(row_ptr, col_idx, dist, dirs, with_parent=True, in_csr=None):
    """Returns (init_bytes, level_bytes[L]) for one search.  in_csr = (in_row_ptr,
    in_col_idx) of a directed graph (see transpose); None: the graph is
    symmetric and serves as its own."""
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
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    rc = lib.bfs_alg_bytes(rp.shape[0] - 1, p(rp), p(ci), p(irp), p(ici), p(d), L, p(dr),
                           1 if with_parent else 0,
                           ctypes.byref(init), p(out))
    if rc != 0:
        raise ValueError(f"bfs_alg_bytes failed ({rc})")
    return int(init.value), out
