"""The kept-bitmap path: levels run from or into a bitmap (bottom-up levels,
and the level after a wide top-down level) record their found sets as
bitmaps, and a finishing launch writes dist in vertex order once the search
is done.  The library takes it on graphs of at least 2^23 vertices (the C5
tests run it at full size); FBFS_FINISH_MIN_N, read at bfs_graph_create,
lowers that size so that small graphs of every shape run it here.  dist, L
and the level sizes bit-exact against the oracle, parents valid, under every
policy (the one-workgroup path of graphs under 3,585 vertices takes only the
default policy, so the others cover those graphs)."""
import contextlib
import os

import numpy as np
import pytest

import graphgen as gg
import oracle
from gpu_util import check_graph, run_hip, sorted_rows_copy, to_dev

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def finish_from(n):
    os.environ["FBFS_FINISH_MIN_N"] = str(n)
    try:
        yield
    finally:
        del os.environ["FBFS_FINISH_MIN_N"]


def test_finish_tiny_random():
    with finish_from(0):
        for seed in range(120):
            g = gg.tiny_random(seed)
            check_graph(g, label=f"finish tiny seed {seed}")
            if g.symmetric:
                check_graph(sorted_rows_copy(g), label=f"finish tiny seed {seed} sorted")


def test_finish_closed_forms():
    """A 3,000-level path pulled level by level passes the 16 kept levels (the
    later ones store dist directly); stars, grids and a complete graph."""
    with finish_from(0):
        for g in (gg.path_graph(3000), gg.star_graph(5000), gg.complete_graph(300), gg.grid_full(97, 61),
                  gg.disjoint_union(gg.path_graph(50), gg.complete_graph(40))):
            check_graph(g, label=f"finish {g.name}")


@pytest.mark.parametrize("scale", [14, 17])
def test_finish_rmat(scale):
    with finish_from(0):
        check_graph(gg.rmat(scale, 16, seed=300 + scale, nsrc=3), label=f"finish rmat {scale}")


def test_finish_directed():
    """Vertices without in-edges start out visited and are never reached: the
    finishing pass writes -1 for them (and leaves a source without in-edges
    at 0)."""
    with finish_from(0):
        check_graph(gg.rmat_directed(14, 16, seed=77, nsrc=3), label="finish directed rmat")
        g = gg.random_directed(20000, 4, 9)
        deg_in = np.bincount(g.col_idx, minlength=g.n)
        s = int(np.nonzero((deg_in == 0) & (np.diff(g.row_ptr) > 0))[0][0])
        check_graph(g, sources=[s] + [int(x) for x in g.sources], label="finish directed random")


@pytest.mark.parametrize("finish", [True, False])
def test_finish_queue_free_wide_levels(finish):
    """A wide top-down level stores no dist; the next level keeps its frontier
    as a bitmap (kept-bitmap path) or writes its dist (default path at this
    size), whether it pulls (alpha = 40) or expands from the bitmap (alpha = 1
    or 4).  The level flags record which, and the kept path's bottom-up levels
    keep their finds."""
    import frontier_bfs_csr_amd as fb
    g = gg.disjoint_union(gg.star_graph(200_001), gg.rmat(16, 16, seed=23, nsrc=1))
    rp, ci = to_dev(g)
    seen = 0
    ctx = finish_from(0) if finish else contextlib.nullcontext()
    with ctx, fb.BfsGraph(rp, ci) as bg:
        for alpha in (1, 4, 40):
            bg.set_switch(alpha, 48)
            for s in (0, 1, 200_001 + 7):
                print(f"[gpu] finish={finish} queue-free alpha={alpha} source={s}", flush=True)
                L, dist, parent, sizes = run_hip(bg, g.n, s)
                ref = oracle.bfs(g.row_ptr, g.col_idx, s)
                oracle.assert_bfs_ok(g.row_ptr, g.col_idx, s, ref, dist, parent, L, sizes[:L],
                                     symmetric=True, label=f"finish {g.name} s={s} alpha={alpha}")
                _, dirs, _ = bg.stats()
                fl = bg.level_flags()
                assert ((fl[0] & fb.LF_FINISHING) != 0) == finish, fl
                for k in range(L):
                    if dirs[k] == 1 and k + 1 < 16:
                        assert bool(fl[k] & fb.LF_FINDS_KEPT) == finish, (k, fl)
                    if dirs[k] == 0:
                        assert not fl[k] & fb.LF_FINDS_KEPT, (k, fl)
                    if k > 0 and fl[k - 1] & fb.LF_QUEUE_FREE:
                        seen += 1
                        want = fb.LF_FRONTIER_KEPT if finish else fb.LF_FRONTIER_DIST
                        assert fl[k] & (fb.LF_FRONTIER_KEPT | fb.LF_FRONTIER_DIST) == want, (k, fl)
    assert seen > 0


def test_finish_unaligned_and_optional_outputs():
    """dist 4 bytes past a 16-byte boundary (the finishing pass then stores
    entry by entry), no parent array, and sources at both ends."""
    import torch
    import frontier_bfs_csr_amd as fb
    g = gg.rmat(13, 16, seed=34, nsrc=3)
    rp, ci = to_dev(g)
    db = torch.full((g.n + 1,), 5, dtype=torch.int32, device="cuda")
    dist = db[1:]
    assert dist.data_ptr() % 16 != 0
    deg = np.diff(g.row_ptr)
    with finish_from(0), fb.BfsGraph(rp, ci) as bg:
        for s in list(g.sources) + [int(np.nonzero(deg)[0][0]), int(np.nonzero(deg)[0][-1])]:
            for with_parent in (True, False):
                parent = torch.full((g.n,), -7, dtype=torch.int32, device="cuda") if with_parent else None
                L = bg.run(int(s), dist, parent, None)
                ref = oracle.bfs(g.row_ptr, g.col_idx, int(s))
                oracle.assert_bfs_ok(g.row_ptr, g.col_idx, int(s), ref, dist.cpu().numpy(),
                                     None if parent is None else parent.cpu().numpy(), L, None,
                                     label=f"finish unaligned s={s} parent={with_parent}")
                assert int(db[0]) == 5
