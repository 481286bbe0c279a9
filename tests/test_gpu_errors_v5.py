"""Error paths and validator V5 through the C ABI.

- BFS_ENOMEM: a graph whose workspace does not fit in the device memory left
  free; the handle is not created and what it had allocated is released.
- BFS_EINVAL: a valid handle with a NULL dist_out; outputs untouched.
- BFS_EDEVICE: the small-frontier barrier's bounded wait given a limit of
  zero at creation, so it gives up at once; every kernel exits normally, and
  the next search on the same handle (without that mode) and on a fresh handle
  match the oracle.
- V5 (debug build with per-vertex enqueue counts): every reached vertex but
  the source is written into a next frontier exactly once, unreached vertices
  never, under every policy.
"""
import ctypes
import os

import numpy as np
import pytest

import graphgen as gg
import oracle
from gpu_util import POLICIES, run_hip, to_dev

pytestmark = pytest.mark.gpu


def test_workspace_out_of_memory():
    import torch
    import frontier_bfs_csr_amd as fb
    # the library's kernels loaded first (a first launch needs device memory
    # of its own), on a small graph
    h = gg.path_graph(5000)
    hr, hc = to_dev(h)
    with fb.BfsGraph(hr, hc) as bg:
        run_hip(bg, h.n, 0)
    g = gg.star_graph(1 << 24)   # a workspace of about 0.8 GB, two levels
    rp, ci = to_dev(g)
    torch.cuda.synchronize()
    # hold device memory in 64 MB pieces until the next piece does not fit,
    # then give one back: under 128 MB are left
    pieces = []
    try:
        while True:
            try:
                pieces.append(torch.empty(64 << 20, dtype=torch.uint8, device="cuda"))
            except torch.OutOfMemoryError:
                break
        del pieces[-1:]
        torch.cuda.synchronize()
        print(f"[gpu] out-of-memory create: {len(pieces) * 64} MB held, n={g.n}", flush=True)
        with pytest.raises(fb.BfsError) as ei:
            fb.bfs_graph_create(g.n, rp, ci)
        assert ei.value.code == fb.BFS_ENOMEM, str(ei.value)
        assert "failed" in str(ei.value)
    finally:
        pieces.clear()
        torch.cuda.empty_cache()
    # the partial workspace was released: the same graph now fits
    with fb.BfsGraph(rp, ci) as bg:
        L, dist, _, _ = run_hip(bg, g.n, 0, False, False)
        assert L == 2 and dist[0] == 0 and (dist[1:] == 1).all()


def test_null_dist_on_valid_handle():
    import torch
    import frontier_bfs_csr_amd as fb
    g = gg.rmat(10, 16, seed=9, nsrc=1)
    rp, ci = to_dev(g)
    with fb.BfsGraph(rp, ci) as bg:
        parent = torch.full((g.n,), 9, dtype=torch.int32, device="cuda")
        rc = fb.load().bfs_run(bg.handle, int(g.sources[0]), None, parent.data_ptr(), None, None)
        assert rc == fb.BFS_EINVAL
        assert "dist_out is required" in fb.bfs_last_error()
        assert (parent.cpu().numpy() == 9).all()
        # the normal build has no enqueue counts
        assert fb.load().bfs_debug_enqueue_counts(bg.handle, parent.data_ptr()) == fb.BFS_EINVAL
        assert "does not count enqueues" in fb.bfs_last_error()


def test_barrier_timeout_reports_edevice():
    """A path of 5,000 vertices runs level after level in the 32-workgroup
    small-frontier mode, behind its barrier; with a wait limit of zero the
    first barrier gives up."""
    import frontier_bfs_csr_amd as fb
    g = gg.path_graph(5000)
    rp, ci = to_dev(g)
    os.environ["FBFS_BARRIER_TIMEOUT_US"] = "0"
    try:
        bg = fb.BfsGraph(rp, ci)
    finally:
        del os.environ["FBFS_BARRIER_TIMEOUT_US"]
    try:
        print("[gpu] barrier timeout: default policy, wait limit 0", flush=True)
        with pytest.raises(fb.BfsError) as ei:
            run_hip(bg, g.n, 0)
        assert ei.value.code == fb.BFS_EDEVICE
        assert "barrier" in str(ei.value)
        # one level per launch needs no barrier: the same handle, reset by the
        # next search's start, gives the oracle's result
        bg.set_policy(*POLICIES["auto_chain"])
        for s in (0, 2500):
            L, dist, parent, sizes = run_hip(bg, g.n, s)
            ref = oracle.bfs(g.row_ptr, g.col_idx, s)
            oracle.assert_bfs_ok(g.row_ptr, g.col_idx, s, ref, dist, parent, L, sizes[:L],
                                 label=f"after timeout s={s}")
    finally:
        bg.close()
    with fb.BfsGraph(rp, ci) as bg2:
        L, dist, parent, sizes = run_hip(bg2, g.n, 0)
        assert L == g.n and (dist == np.arange(g.n)).all()


class _V5:
    """The enqueue-counting debug build, driven through its C ABI."""

    def __init__(self):
        import frontier_bfs_csr_amd as fb
        self.fb = fb
        self.lib = fb.load_v5()

    def counts(self, g, policy, sources):
        import torch
        lib = self.lib
        rp, ci = to_dev(g)
        h = lib.bfs_graph_create(g.n, rp.data_ptr(), ci.data_ptr() if g.m else None)
        assert h, lib.bfs_last_error().decode()
        try:
            assert lib.bfs_set_policy(h, *POLICIES[policy]) == 0
            for s in sources:
                s = int(s)
                print(f"[gpu] V5 {g.name} n={g.n} source={s} policy={policy}", flush=True)
                dist = torch.full((g.n,), -7, dtype=torch.int32, device="cuda")
                parent = torch.full((g.n,), -7, dtype=torch.int32, device="cuda")
                cnt = torch.full((g.n,), -7, dtype=torch.int32, device="cuda")
                L = lib.bfs_run(h, s, dist.data_ptr(), parent.data_ptr(), None, None)
                assert L > 0, lib.bfs_last_error().decode()
                assert lib.bfs_debug_enqueue_counts(h, cnt.data_ptr()) == 0
                torch.cuda.synchronize()
                d, c = dist.cpu().numpy(), cnt.cpu().numpy()
                ref = oracle.bfs(g.row_ptr, g.col_idx, s)
                assert (d == ref[0]).all(), f"V5 build {g.name} s={s} {policy}: dist"
                reached = d >= 0
                assert c[s] == 0, (g.name, s, policy, int(c[s]))
                others = reached.copy()
                others[s] = False
                bad = np.nonzero(others & (c != 1))[0]
                assert bad.size == 0, f"{g.name} s={s} {policy}: vertex {bad[0]} enqueued {c[bad[0]]} times"
                assert (c[~reached] == 0).all(), f"{g.name} s={s} {policy}: unreached vertex enqueued"
        finally:
            lib.bfs_graph_destroy(h)


@pytest.mark.parametrize("policy", ["auto", "push_binned", "push_edge", "pull", "auto_chain",
                                    "auto_binned_hostloop"])
def test_v5_each_vertex_enqueued_once(policy):
    v5 = _V5()
    graphs = [gg.chapter22_graph(), gg.pmpp_graph(), gg.path_graph(5000), gg.grid_full(90, 70),
              gg.rmat(16, 16, seed=17, nsrc=3), gg.rmat_directed(12, 16, seed=52, nsrc=2),
              gg.c1_chung_lu()]
    if policy == "auto":
        # a wide top-down level that writes only the next bitmap (queue-free)
        graphs.append(gg.disjoint_union(gg.star_graph(200_001), gg.rmat(14, 16, seed=23, nsrc=1)))
    for g in graphs:
        srcs = list(g.sources[:3]) if len(g.sources) else [0]
        v5.counts(g, policy, srcs)
    for seed in range(20):
        g = gg.tiny_random(seed)
        v5.counts(g, policy, g.sources[:2])
