"""Python binding of libfrontier_bfs.so: level-synchronous, frontier-based BFS
over an int32 CSR graph on one MI355X (gfx950).

Argument marshalling only: every step of the search runs in the library's HIP
kernels.  The functions mirror the C ABI in ``include/frontier_bfs.h``; PyTorch
supplies device memory (int32 CUDA tensors) and streams.  There is no CPU
fallback: if the library is not built, or no GPU is present, calls raise.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# FBFS_LIBRARY names another build of the same library (e.g. a variant built
# with different compile-time constants); default: the in-tree build.
LIB_PATH = os.environ.get("FBFS_LIBRARY") or os.path.join(_PKG, "libfrontier_bfs.so")

BFS_EINVAL, BFS_EHIP, BFS_ENOMEM, BFS_EDEVICE = -1, -2, -3, -4
DIR_AUTO, DIR_PUSH, DIR_PULL = 0, 1, 2
ADV_AUTO, ADV_BINNED, ADV_EDGE = 0, 1, 2
LOOP_DEVICE, LOOP_HOST, LOOP_CHAIN = 0, 1, 2
WALK_LANE, WALK_WAVE, WALK_BINNED, WALK_MERGE = 0, 1, 2, 3
CLAIM_BITMAP, CLAIM_MIN = 0, 1
COMPACT_DEFAULT, COMPACT_ATOMIC, COMPACT_PADDED, COMPACT_FILTER, COMPACT_FLAGS = 0, 1, 2, 3, 4
# graphs of at most this many vertices are searched by one workgroup under the
# default policy (the library's ONE_N; bfs_small.hip)
SMALL_GRAPH_N = 3584

EXPORTS = ("bfs_graph_create", "bfs_run", "bfs_graph_destroy", "bfs_last_error",
           "bfs_set_policy", "bfs_last_run_stats", "bfs_last_run_level_flags", "bfs_set_timing", "bfs_last_run_timing",
           "bfs_graph_info", "bfs_set_switch", "bfs_last_run_kernel_timing", "bfs_walk_level", "bfs_set_primitives",
           "bfs_sssp", "bfs_last_run_launch_timing", "bfs_run_noalloc", "bfs_debug_enqueue_counts",
           "bfs_last_error_code")

_lib = None


class BfsError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


# the enqueue-counting debug build (validator V5 of the tests)
LIB_V5_PATH = os.path.join(_PKG, "libfrontier_bfs_v5.so")
_lib_v5 = None


def load():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


def load_v5():
    """Load the enqueue-counting debug build (tests only)."""
    global _lib_v5
    if _lib_v5 is None:
        _lib_v5 = _open(LIB_V5_PATH)
    return _lib_v5


def _open(path):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.bfs_graph_create.argtypes = [i32, P, P]
    lib.bfs_graph_create.restype = P
    lib.bfs_run.argtypes = [P, i32, P, P, P, P]
    lib.bfs_run.restype = i32
    lib.bfs_graph_destroy.argtypes = [P]
    lib.bfs_graph_destroy.restype = None
    lib.bfs_last_error.argtypes = []
    lib.bfs_last_error.restype = ctypes.c_char_p
    lib.bfs_last_error_code.argtypes = []
    lib.bfs_last_error_code.restype = i32
    lib.bfs_set_policy.argtypes = [P, i32, i32, i32]
    lib.bfs_set_policy.restype = i32
    lib.bfs_set_switch.argtypes = [P, i32, i32]
    lib.bfs_set_switch.restype = i32
    lib.bfs_last_run_stats.argtypes = [P, i32, P, P]
    lib.bfs_last_run_stats.restype = i32
    lib.bfs_last_run_level_flags.argtypes = [P, i32, P]
    lib.bfs_last_run_level_flags.restype = i32
    lib.bfs_graph_info.argtypes = [P, ctypes.POINTER(i64), ctypes.POINTER(i32),
                                   ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.bfs_graph_info.restype = i32
    lib.bfs_set_timing.argtypes = [P, i32]
    lib.bfs_set_timing.restype = i32
    lib.bfs_last_run_timing.argtypes = [P, ctypes.POINTER(ctypes.c_float),
                                        ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
    lib.bfs_last_run_timing.restype = i32
    lib.bfs_last_run_kernel_timing.argtypes = [P, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32),
                                               ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
    lib.bfs_last_run_kernel_timing.restype = i32
    lib.bfs_debug_enqueue_counts.argtypes = [P, P]
    lib.bfs_debug_enqueue_counts.restype = i32
    lib.bfs_run_noalloc.argtypes = [i32, P, P, i32, P, P, P, P]
    lib.bfs_run_noalloc.restype = i32
    lib.bfs_last_run_launch_timing.argtypes = [P, i32, P, P]
    lib.bfs_last_run_launch_timing.restype = i32
    lib.bfs_walk_level.argtypes = [P, P, i32, i32, i32, P, P]
    lib.bfs_walk_level.restype = i32
    lib.bfs_set_primitives.argtypes = [P, i32, i32]
    lib.bfs_set_primitives.restype = i32
    lib.bfs_sssp.argtypes = [P, i32, P, ctypes.c_uint32, P, P, P]
    lib.bfs_sssp.restype = i32
    return lib


def bfs_last_error() -> str:
    return load().bfs_last_error().decode()


_torch = None
# raw handle -> (n, m) of its graph, for the size checks of the calls on it
_handle_sizes = {}


def _t():
    global _torch
    if _torch is None:
        import torch
        _torch = torch
    return _torch


def _dev_i32(t, name, numel=None):
    """Device address of a contiguous int32 CUDA tensor with at least `numel`
    elements (the kernels write every one of those), or None."""
    if t is None:
        return None
    torch = _t()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dtype is not torch.int32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 tensor")
    k = t.numel()
    if numel is not None and k < numel:
        raise ValueError(f"{name} needs at least {numel} elements, has {k}")
    return t.data_ptr() if k else None


def _dev_tensor(t, name, dtypes, numel=None):
    if t is None:
        return None
    torch = _t()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dtype not in dtypes or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous tensor of {', '.join(map(str, dtypes))}")
    k = t.numel()
    if numel is not None and k < numel:
        raise ValueError(f"{name} needs at least {numel} elements, has {k}")
    return t.data_ptr() if k else None


def _stream_handle(stream):
    if stream is None:
        stream = _t().cuda.current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def bfs_graph_create(n, row_ptr, col_idx):
    """Wrap an int32 CSR graph held in CUDA tensors; returns a raw handle.
    The tensors are borrowed and must outlive the handle."""
    rp = _dev_i32(row_ptr, "row_ptr", n + 1)
    ci = _dev_i32(col_idx, "col_idx")
    h = load().bfs_graph_create(int(n), rp, ci)
    if not h:
        raise BfsError(load().bfs_last_error_code() or BFS_EINVAL, bfs_last_error())
    _handle_sizes[h] = (int(n), bfs_graph_info(h)["m"])
    return h


def bfs_run(g, source, dist, parent=None, level_sizes=None, stream=None):
    """One BFS from `source` into the int32 CUDA tensors (each of at least n
    elements); returns L."""
    n = _handle_sizes.get(g, (None,))[0]
    L = load().bfs_run(g, int(source), _dev_i32(dist, "dist", n), _dev_i32(parent, "parent", n),
                       _dev_i32(level_sizes, "level_sizes", n), _stream_handle(stream))
    if L < 0:
        raise BfsError(L, bfs_last_error())
    return L


# bounds of bfs_run_noalloc (its fixed scratch is sized for them)
NOALLOC_MAX_N = 1 << 16
NOALLOC_MAX_M = 1 << 21


def bfs_run_noalloc(row_ptr, col_idx, source, dist, parent=None, level_sizes=None, stream=None):
    """One BFS without a handle or any device allocation (graphs of at most
    NOALLOC_MAX_N vertices and NOALLOC_MAX_M entries); returns L."""
    n = int(row_ptr.numel()) - 1
    L = load().bfs_run_noalloc(n, _dev_i32(row_ptr, "row_ptr", n + 1), _dev_i32(col_idx, "col_idx"),
                               int(source), _dev_i32(dist, "dist", n), _dev_i32(parent, "parent", n),
                               _dev_i32(level_sizes, "level_sizes", n), _stream_handle(stream))
    if L < 0:
        raise BfsError(L, bfs_last_error())
    return L


def bfs_graph_destroy(g):
    if g:
        _handle_sizes.pop(g, None)
        load().bfs_graph_destroy(g)


def bfs_set_policy(g, direction=DIR_AUTO, advance=ADV_AUTO, loop=LOOP_DEVICE):
    rc = load().bfs_set_policy(g, int(direction), int(advance), int(loop))
    if rc < 0:
        raise BfsError(rc, bfs_last_error())


def bfs_sssp(g, source, weights, max_weight, dist, pred=None, stream=None):
    """Shortest paths from source: weights (device uint32/int32 tensor, one per
    CSR entry), dist (device int64, n), pred (device int32, n, or None).
    Returns the number of relaxation rounds."""
    torch = _t()
    n, m = _handle_sizes.get(g, (None, None))
    w = _dev_tensor(weights, "weights", (torch.int32, torch.uint32), m)
    d = _dev_tensor(dist, "dist", (torch.int64,), n)
    p = _dev_i32(pred, "pred", n)
    rc = load().bfs_sssp(g, int(source), w, int(max_weight), d, p, _stream_handle(stream))
    if rc < 0:
        raise BfsError(rc, bfs_last_error())
    return rc


def bfs_set_primitives(g, claim=CLAIM_BITMAP, compaction=COMPACT_DEFAULT):
    rc = load().bfs_set_primitives(g, int(claim), int(compaction))
    if rc < 0:
        raise BfsError(rc, bfs_last_error())


def bfs_set_switch(g, alpha=40, beta=96):
    rc = load().bfs_set_switch(g, int(alpha), int(beta))
    if rc < 0:
        raise BfsError(rc, bfs_last_error())


def bfs_walk_level(g, vertices, out, mapping=WALK_WAVE, repeats=64, stream=None):
    """Isolated neighbour walk of the listed vertices (int32 CUDA tensor) into
    out (int32 CUDA tensor of the same length; its bits are the uint32 sums)."""
    count = vertices.numel() if vertices is not None else 0
    v = _dev_i32(vertices, "vertices")
    o = _dev_i32(out, "out", count)
    rc = load().bfs_walk_level(g, v, count, int(mapping), int(repeats), o, _stream_handle(stream))
    if rc < 0:
        raise BfsError(rc, bfs_last_error())


def bfs_last_run_stats(g, cap=1 << 22):
    """(L, dir[int8, per level: 0 top-down, 1 bottom-up], frontier_edges[int64])."""
    L0 = load().bfs_last_run_stats(g, 0, None, None)
    if L0 < 0:
        raise BfsError(L0, bfs_last_error())
    cnt = min(L0, cap)
    d = np.zeros(cnt, np.int8)
    fe = np.zeros(cnt, np.int64)
    L = load().bfs_last_run_stats(g, cnt, d.ctypes.data_as(ctypes.c_void_p),
                                  fe.ctypes.data_as(ctypes.c_void_p))
    if L < 0:
        raise BfsError(L, bfs_last_error())
    return L, d, fe


LF_QUEUE_FREE, LF_FINDS_KEPT, LF_FRONTIER_KEPT, LF_FRONTIER_DIST, LF_FINISHING = 1, 2, 4, 8, 16


def bfs_last_run_level_flags(g, cap=1 << 22):
    """uint8 per level of the last run: LF_* bits, where the level's dist stores went."""
    L0 = load().bfs_last_run_level_flags(g, 0, None)
    if L0 < 0:
        raise BfsError(L0, bfs_last_error())
    f = np.zeros(min(L0, cap), np.uint8)
    L = load().bfs_last_run_level_flags(g, f.shape[0], f.ctypes.data_as(ctypes.c_void_p))
    if L < 0:
        raise BfsError(L, bfs_last_error())
    return f


def bfs_set_timing(g, on=True):
    rc = load().bfs_set_timing(g, 1 if on else 0)
    if rc < 0:
        raise BfsError(rc, bfs_last_error())


def bfs_last_run_timing(g):
    """(init_ms, level_ms, level_launches) of the last timed run."""
    a, b, c = ctypes.c_float(), ctypes.c_float(), ctypes.c_int32()
    rc = load().bfs_last_run_timing(g, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    if rc < 0:
        raise BfsError(rc, bfs_last_error())
    return a.value, b.value, c.value


def bfs_last_run_kernel_timing(g):
    """{"td": (ms, launches), "bu": (ms, launches)} of the last timed run."""
    a, b = ctypes.c_float(), ctypes.c_float()
    c, d = ctypes.c_int32(), ctypes.c_int32()
    rc = load().bfs_last_run_kernel_timing(g, ctypes.byref(a), ctypes.byref(c), ctypes.byref(b),
                                           ctypes.byref(d))
    if rc < 0:
        raise BfsError(rc, bfs_last_error())
    return {"td": (a.value, c.value), "bu": (b.value, d.value)}


def bfs_last_run_launch_timing(g):
    """(ms[float32], ran[uint8]) per level launch of the last timed run."""
    cnt = load().bfs_last_run_launch_timing(g, 0, None, None)
    if cnt < 0:
        raise BfsError(cnt, bfs_last_error())
    ms = np.zeros(cnt, np.float32)
    ran = np.zeros(cnt, np.uint8)
    rc = load().bfs_last_run_launch_timing(g, cnt, ms.ctypes.data_as(ctypes.c_void_p),
                                           ran.ctypes.data_as(ctypes.c_void_p))
    if rc < 0:
        raise BfsError(rc, bfs_last_error())
    return ms, ran


def bfs_graph_info(g):
    m, srt, sym, mx, pr = (ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(),
                           ctypes.c_int32())
    rc = load().bfs_graph_info(g, ctypes.byref(m), ctypes.byref(srt), ctypes.byref(sym),
                               ctypes.byref(mx), ctypes.byref(pr))
    if rc < 0:
        raise BfsError(rc, bfs_last_error())
    return {"m": m.value, "sorted_rows": bool(srt.value), "symmetric": bool(sym.value),
            "max_degree": mx.value, "pull_ready": bool(pr.value)}


class BfsGraph:
    """Owns a handle and keeps the borrowed CSR tensors alive with it."""

    def __init__(self, row_ptr, col_idx):
        self.row_ptr = row_ptr
        self.col_idx = col_idx
        self.n = int(row_ptr.numel() - 1)
        self.handle = bfs_graph_create(self.n, row_ptr, col_idx)

    def run(self, source, dist, parent=None, level_sizes=None, stream=None):
        return bfs_run(self.handle, source, dist, parent, level_sizes, stream)

    def set_policy(self, direction=DIR_AUTO, advance=ADV_AUTO, loop=LOOP_DEVICE):
        bfs_set_policy(self.handle, direction, advance, loop)

    def walk(self, vertices, out, mapping=WALK_WAVE, repeats=64, stream=None):
        bfs_walk_level(self.handle, vertices, out, mapping, repeats, stream)

    def set_switch(self, alpha=40, beta=96):
        bfs_set_switch(self.handle, alpha, beta)

    def set_primitives(self, claim=CLAIM_BITMAP, compaction=COMPACT_DEFAULT):
        bfs_set_primitives(self.handle, claim, compaction)

    def sssp(self, source, weights, max_weight, dist, pred=None, stream=None):
        return bfs_sssp(self.handle, source, weights, max_weight, dist, pred, stream)

    def stats(self):
        return bfs_last_run_stats(self.handle)

    def level_flags(self):
        return bfs_last_run_level_flags(self.handle)

    def info(self):
        return bfs_graph_info(self.handle)

    def set_timing(self, on=True):
        bfs_set_timing(self.handle, on)

    def timing(self):
        return bfs_last_run_timing(self.handle)

    def kernel_timing(self):
        return bfs_last_run_kernel_timing(self.handle)

    def launch_timing(self):
        return bfs_last_run_launch_timing(self.handle)

    def close(self):
        if self.handle:
            bfs_graph_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
