"""The C-ABI library: it loads, exports every declared entry point, and
rejects bad arguments on the host side without touching a GPU."""
import ctypes
import os
import re

import frontier_bfs_csr_amd as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if fn.endswith(".h"):
            src = open(os.path.join(inc, fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(bfs_[a-z_]+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    lib = fb.load()
    declared = _declared()
    assert declared, "no declarations found"
    assert declared == set(fb.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_host_side_argument_errors():
    lib = fb.load()
    assert lib.bfs_graph_create(0, ctypes.c_void_p(1), ctypes.c_void_p(1)) is None
    assert "at least one vertex" in fb.bfs_last_error()
    assert lib.bfs_graph_create(5, None, ctypes.c_void_p(1)) is None
    assert "row_ptr must be a device pointer" in fb.bfs_last_error()
    assert lib.bfs_run(None, 0, None, None, None, None) == fb.BFS_EINVAL
    assert "NULL graph" in fb.bfs_last_error()
    assert lib.bfs_set_policy(None, 0, 0, 0) == fb.BFS_EINVAL
    assert lib.bfs_set_switch(None, 14, 24) == fb.BFS_EINVAL
    assert lib.bfs_last_run_kernel_timing(None, None, None, None, None) == fb.BFS_EINVAL
    assert lib.bfs_walk_level(None, None, 0, 0, 64, None, None) == fb.BFS_EINVAL
    assert lib.bfs_set_primitives(None, 0, 1) == fb.BFS_EINVAL
    assert lib.bfs_sssp(None, 0, None, 1, None, None, None) == fb.BFS_EINVAL
    assert lib.bfs_last_run_stats(None, 0, None, None) == fb.BFS_EINVAL
    assert lib.bfs_last_run_level_flags(None, 0, None) == fb.BFS_EINVAL
    assert lib.bfs_graph_info(None, None, None, None, None, None) == fb.BFS_EINVAL
    assert lib.bfs_last_run_launch_timing(None, 0, None, None) == fb.BFS_EINVAL
    # the allocation-free search refuses sizes beyond its fixed scratch, and
    # missing pointers, before any device work
    assert lib.bfs_run_noalloc(fb.NOALLOC_MAX_N + 1, ctypes.c_void_p(1), ctypes.c_void_p(1), 0,
                               ctypes.c_void_p(1), None, None, None) == fb.BFS_EINVAL
    assert "limit" in fb.bfs_last_error()
    assert lib.bfs_run_noalloc(0, ctypes.c_void_p(1), ctypes.c_void_p(1), 0,
                               ctypes.c_void_p(1), None, None, None) == fb.BFS_EINVAL
    assert lib.bfs_run_noalloc(10, None, ctypes.c_void_p(1), 0, ctypes.c_void_p(1), None, None,
                               None) == fb.BFS_EINVAL
    assert lib.bfs_run_noalloc(10, ctypes.c_void_p(1), ctypes.c_void_p(1), 0, None, None, None,
                               None) == fb.BFS_EINVAL
    assert lib.bfs_run_noalloc(10, ctypes.c_void_p(1), ctypes.c_void_p(1), 10, ctypes.c_void_p(1), None,
                               None, None) == fb.BFS_EINVAL
    assert "source 10" in fb.bfs_last_error()
    lib.bfs_graph_destroy(None)   # no-op


def test_binding_rejects_host_tensors():
    import pytest
    import torch
    with pytest.raises(TypeError):
        fb.bfs_graph_create(3, torch.zeros(4, dtype=torch.int32), torch.zeros(0, dtype=torch.int32))
