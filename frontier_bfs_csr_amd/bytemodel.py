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
        lib.bfs_alg_bytes.argtypes = [ctypes.c_int32, P, P, P, ctypes.c_int32, P, ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int64), P]
        lib.bfs_alg_bytes.restype = ctypes.c_int32
        _lib = lib
    return _lib


def alg_bytes(row_ptr, col_idx, dist, dirs, with_parent=True):
    """Returns (init_bytes, level_bytes[L]) for one search."""
    lib = _load()
    rp = np.ascontiguousarray(row_ptr, np.int32)
    ci = np.ascontiguousarray(col_idx, np.int32)
    d = np.ascontiguousarray(dist, np.int32)
    dr = np.ascontiguousarray(dirs, np.int8)
    L = dr.shape[0]
    out = np.zeros(L, np.int64)
    init = ctypes.c_int64(0)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    rc = lib.bfs_alg_bytes(rp.shape[0] - 1, p(rp), p(ci), p(d), L, p(dr), 1 if with_parent else 0,
                           ctypes.byref(init), p(out))
    if rc != 0:
        raise ValueError(f"bfs_alg_bytes failed ({rc})")
    return int(init.value), out
