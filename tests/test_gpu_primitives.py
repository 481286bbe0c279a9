"""The claim and compaction primitives (bfs_set_primitives) through the C ABI:
every claim x compaction pair gives the oracle's dist, L and level sizes
bit for bit and valid parents, on the pages' worked graphs, tiny random
graphs, closed forms, directed graphs and R-MAT; the per-level frontier edge
sums (which are also the padded frontiers' lengths) match the oracle's."""
import numpy as np
import pytest

import graphgen as gg
import oracle
from gpu_util import run_hip, to_dev

pytestmark = pytest.mark.gpu

PAIRS = [(c, k) for c in (0, 1) for k in (1, 2, 3, 4)]   # (claim, compaction)


def _check(g, sources, label, pairs=PAIRS):
    import frontier_bfs_csr_amd as fb
    rp, ci = to_dev(g)
    deg = np.diff(g.row_ptr).astype(np.int64)
    with fb.BfsGraph(rp, ci) as bg:
        for s in sources:
            s = int(s)
            ref = oracle.bfs(g.row_ptr, g.col_idx, s)
            d_ref = ref[0]
            want_fe = np.bincount(d_ref[d_ref >= 0], weights=deg[d_ref >= 0]).astype(np.int64)
            for claim, comp in pairs:
                bg.set_primitives(claim, comp)
                print(f"[gpu] primitives {label} n={g.n} m={g.m} source={s} claim={claim} compaction={comp}",
                      flush=True)
                L, dist, parent, sizes = run_hip(bg, g.n, s)
                oracle.assert_bfs_ok(g.row_ptr, g.col_idx, s, ref, dist, parent, L, sizes[:L],
                                     symmetric=g.symmetric, label=f"{label} s={s} {claim}/{comp}")
                assert (sizes[L:] == -7).all(), f"{label}: level_sizes written beyond L"
                Ls, dirs, fe = bg.stats()
                assert Ls == L and (dirs == 0).all()
                assert (fe == want_fe[:L]).all(), (label, claim, comp, fe, want_fe)
        bg.set_primitives(0, 0)   # back to the direction-optimising path
        L, dist, _, _ = run_hip(bg, g.n, int(sources[0]))
        assert (dist == oracle.bfs(g.row_ptr, g.col_idx, int(sources[0]))[0]).all()


def test_primitives_worked_graphs():
    for g in (gg.chapter22_graph(), gg.pmpp_graph()):
        _check(g, range(g.n), g.name)


def test_primitives_tiny_random():
    for seed in range(40):
        g = gg.tiny_random(seed)
        _check(g, [0, g.n - 1] if g.n > 1 else [0], f"tiny{seed}")


def test_primitives_closed_forms():
    _check(gg.path_graph(1500), [0, 749], "path")          # 1,500 levels of one vertex
    _check(gg.star_graph(5000), [0, 17], "star")            # one hub
    _check(gg.disjoint_union(gg.complete_graph(40), gg.path_graph(30)), [0, 45], "union")


def test_primitives_directed_and_rmat():
    g = gg.random_directed(5000, 12, 9)
    _check(g, g.sources[:2], "directed")
    g = gg.rmat_directed(12, nsrc=2)
    _check(g, g.sources, "rmat12_directed")
    g = gg.rmat(16, 16, seed=41, nsrc=2)
    _check(g, g.sources, "rmat16")


def test_primitives_arguments():
    import frontier_bfs_csr_amd as fb
    g = gg.path_graph(10)
    rp, ci = to_dev(g)
    with fb.BfsGraph(rp, ci) as bg:
        for claim, comp in ((1, 0), (2, 1), (0, 5), (-1, 1), (0, -1)):
            with pytest.raises(fb.BfsError) as ei:
                bg.set_primitives(claim, comp)
            assert ei.value.code == fb.BFS_EINVAL
        bg.set_primitives(1, 3)
        bg.set_timing(True)
        L, dist, _, _ = run_hip(bg, g.n, 0)
        init_ms, level_ms, launches = bg.timing()
        assert L == 10 and launches == L and level_ms > 0.0
