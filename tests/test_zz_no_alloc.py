"""The allocation-free entry point (bfs_run_noalloc) against bfs_run on a
handle, through the C ABI: dist, L and level sizes equal to bfs_run's and the
oracle's, parents valid BFS parents, entries past L untouched; calls in a row
on the shared fixed scratch, each on a smaller graph than the one before,
across the one-workgroup, multi-workgroup and push-only (directed) paths; and
the size bounds refused with the outputs untouched."""
import numpy as np
import pytest

import graphgen as gg
import oracle
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _run_handle(g, s):
    import torch
    import frontier_bfs_csr_amd as fb
    rp, ci = to_dev(g)
    dist = torch.full((g.n,), -7, dtype=torch.int32, device="cuda")
    parent = torch.full((g.n,), -7, dtype=torch.int32, device="cuda")
    sizes = torch.full((g.n,), -7, dtype=torch.int32, device="cuda")
    with fb.BfsGraph(rp, ci) as bg:
        L = bg.run(int(s), dist, parent, sizes)
    torch.cuda.synchronize()
    return L, dist.cpu().numpy(), parent.cpu().numpy(), sizes.cpu().numpy()


def _run_noalloc(g, s, with_parent=True, with_sizes=True):
    import torch
    import frontier_bfs_csr_amd as fb
    rp, ci = to_dev(g)
    dist = torch.full((g.n,), -7, dtype=torch.int32, device="cuda")
    parent = torch.full((g.n,), -7, dtype=torch.int32, device="cuda") if with_parent else None
    sizes = torch.full((g.n,), -7, dtype=torch.int32, device="cuda") if with_sizes else None
    L = fb.bfs_run_noalloc(rp, ci, int(s), dist, parent, sizes)
    torch.cuda.synchronize()
    return (L, dist.cpu().numpy(), None if parent is None else parent.cpu().numpy(),
            None if sizes is None else sizes.cpu().numpy())


def _compare(g, s, label):
    print(f"[gpu] noalloc {label} n={g.n} m={g.m} source={s}", flush=True)
    La, da, pa, za = _run_noalloc(g, s)
    Lb, db, pb, zb = _run_handle(g, s)
    assert La == Lb, (label, La, Lb)
    assert (da == db).all(), f"{label}: dist differs from bfs_run"
    assert (za[:La] == zb[:Lb]).all(), f"{label}: level sizes differ from bfs_run"
    assert (za[La:] == -7).all(), f"{label}: level sizes written past L"
    ref = oracle.bfs(g.row_ptr, g.col_idx, int(s))
    oracle.assert_bfs_ok(g.row_ptr, g.col_idx, int(s), ref, da, pa, La, za[:La],
                         symmetric=g.symmetric, label=f"noalloc {label} s={s}")


def test_noalloc_matches_bfs_run_on_shrinking_inputs():
    """Calls in a row, each on a smaller graph, so that what a larger call
    left in the scratch would show in a smaller one."""
    big = gg.rmat(16, 16, seed=66, nsrc=2)          # 65,536 vertices: the vertex bound
    assert big.m <= 1 << 21
    mid = gg.rmat(15, 16, seed=65, nsrc=2)
    small = gg.rmat(12, 16, seed=62, nsrc=2)        # 4,096 vertices: multi-workgroup path
    directed = gg.random_directed(20000, 8, 2)      # push-only here
    tiny = gg.chapter22_graph()                     # one-workgroup path
    for g, label in ((big, "rmat16"), (mid, "rmat15"), (directed, "directed 20000"), (small, "rmat12"),
                     (tiny, "chapter22")):
        for s in list(g.sources[:2]):
            _compare(g, int(s), label)
    # the same graph twice in a row, then the larger one again
    _compare(small, int(small.sources[0]), "rmat12 again")
    _compare(big, int(big.sources[1]), "rmat16 again")


def test_noalloc_optional_outputs_and_path():
    g = gg.disjoint_union(gg.path_graph(5000), gg.star_graph(100))
    for wp, ws in ((False, False), (True, False), (False, True)):
        L, dist, parent, sizes = _run_noalloc(g, 0, wp, ws)
        assert L == 5000
        assert (dist[:5000] == np.arange(5000)).all() and (dist[5000:] == -1).all()
        if sizes is not None:
            assert (sizes[:L] == 1).all() and (sizes[L:] == -7).all()


def test_noalloc_bounds_refused_outputs_untouched():
    import torch
    import frontier_bfs_csr_amd as fb
    # one vertex over the bound
    n = fb.NOALLOC_MAX_N + 1
    rp = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    ci = torch.zeros(1, dtype=torch.int32, device="cuda")
    d = torch.full((n,), 9, dtype=torch.int32, device="cuda")
    with pytest.raises(fb.BfsError) as ei:
        fb.bfs_run_noalloc(rp, ci, 0, d)
    assert ei.value.code == fb.BFS_EINVAL and "limit" in str(ei.value)
    # entries over the bound: a star whose row_ptr[n] is above it
    n = 1000
    m = fb.NOALLOC_MAX_M + 2
    rpn = np.zeros(n + 1, np.int32)
    rpn[1:] = m
    rp = torch.from_numpy(rpn).cuda()
    ci = torch.ones(m, dtype=torch.int32, device="cuda")
    d = torch.full((n,), 9, dtype=torch.int32, device="cuda")
    with pytest.raises(fb.BfsError) as ei:
        fb.bfs_run_noalloc(rp, ci, 0, d)
    assert ei.value.code == fb.BFS_EINVAL and "CSR entries" in str(ei.value)
    # an invalid graph: the first bad entry is named
    rp = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    ci = torch.tensor([1, 5], dtype=torch.int32, device="cuda")
    d = torch.full((2,), 9, dtype=torch.int32, device="cuda")
    with pytest.raises(fb.BfsError) as ei:
        fb.bfs_run_noalloc(rp, ci, 0, d)
    assert "col_idx[1]" in str(ei.value)
    assert (d.cpu().numpy() == 9).all()
    # and a good call right after the refused ones
    g = gg.rmat(13, 16, seed=63, nsrc=1)
    _compare(g, int(g.sources[0]), "rmat13 after refusals")
