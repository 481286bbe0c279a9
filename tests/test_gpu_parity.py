"""HIP path vs the oracle, through the C ABI: dist, L and level sizes
bit-exact; parents valid BFS parents; every policy (direction x advance x
loop).  Graphs: the pages' worked graphs, tiny random graphs, closed forms,
scaled-down and full-size workloads."""
import numpy as np
import pytest

import graphgen as gg
import oracle
from gpu_util import check_graph, check_sources_parallel, run_hip, sorted_rows_copy, to_dev

pytestmark = pytest.mark.gpu


def test_chapter22_graph():
    g = gg.chapter22_graph()
    check_graph(g, sources=range(g.n))


def test_pmpp_graph():
    g = gg.pmpp_graph()
    check_graph(g, sources=range(g.n))


@pytest.mark.parametrize("block", range(6))
def test_tiny_random(block):
    for seed in range(block * 50, block * 50 + 50):
        g = gg.tiny_random(seed)
        check_graph(g, label=f"tiny seed {seed}")
        if g.symmetric:
            check_graph(sorted_rows_copy(g), label=f"tiny seed {seed} sorted")


def test_closed_forms():
    for g in (gg.path_graph(1), gg.path_graph(2), gg.path_graph(3000), gg.star_graph(5000),
              gg.complete_graph(300), gg.grid_full(97, 61),
              gg.disjoint_union(gg.path_graph(50), gg.complete_graph(40))):
        check_graph(g)


def test_directed_random():
    for n, deg, seed in ((1000, 3, 1), (20000, 8, 2), (5000, 40, 3)):
        check_graph(gg.random_directed(n, deg, seed))


@pytest.mark.parametrize("scale", [12, 16])
def test_directed_rmat(scale):
    """Directed R-MAT (no symmetrisation): pull and direction switching run on
    in-edges from the transpose built at graph creation."""
    g = gg.rmat_directed(scale, 16, seed=40 + scale, nsrc=3)
    check_graph(g)


@pytest.mark.parametrize("scale", [10, 14, 17])
def test_rmat_scaled(scale):
    g = gg.rmat(scale, 16, seed=100 + scale, nsrc=3)
    check_graph(g)


def test_hub_source():
    """Source of maximum degree on an R-MAT graph: tiles split over workgroups."""
    g = gg.rmat(16, 16, seed=7, nsrc=1)
    s = int(np.argmax(np.diff(g.row_ptr)))
    check_graph(g, sources=[s])


def test_c1_workload():
    g = gg.c1_chung_lu()
    check_graph(g, sources=list(g.sources) + [0, g.n - 1])


def test_c2_workload_all_sources():
    """R-MAT scale 20: all 64 sources under the default policy, every policy
    on the first four."""
    g = gg.c2_rmat20(nsrc=64)
    assert check_sources_parallel(g, g.sources) == 64
    check_graph(g, sources=g.sources[:4])


def test_c3_workload_all_sources():
    """Erdos-Renyi, 4M vertices: all 64 sources under the default policy; the
    binned and edge-balanced push advances and pull on two."""
    g = gg.c3_er(nsrc=64)
    assert check_sources_parallel(g, g.sources) == 64
    check_graph(g, sources=g.sources[:2], policies=["push_binned", "push_edge", "pull"])


def test_c4_workload():
    """The damaged 4096 x 4096 grid from a corner: thousands of levels."""
    g = gg.c4_grid()
    check_graph(g, policies=["auto", "push_edge"])


def test_c5_workload_all_sources():
    """R-MAT scale 24 at full size, in the benchmark's configuration (auto
    policy, parents and level sizes written), on all 64 of its sources (the
    oracle on 16 host threads); the other policies on two of them."""
    g = gg.c5_rmat24(nsrc=64)
    assert check_sources_parallel(g, g.sources, chunk=16, workers=16) == 64
    check_graph(g, sources=g.sources[16:18], policies=["push_binned", "push_edge", "pull", "auto_chain"])


@pytest.mark.parametrize("alpha,beta", [(1, 1), (1, 10**6), (10**6, 1), (10**6, 10**6), (4, 64)])
def test_switch_parameters(alpha, beta):
    """The automatic policy under extreme direction-switch parameters: results
    never change; a huge alpha pulls from the second level on.  (The
    edge-balanced advance is named explicitly: it keeps the small C1 graph on
    the multi-workgroup path, whose direction switch this checks.)"""
    import frontier_bfs_csr_amd as fb
    for g in (gg.rmat(14, 16, seed=21, nsrc=3), gg.c1_chung_lu()):
        rp, ci = to_dev(g)
        with fb.BfsGraph(rp, ci) as bg:
            bg.set_policy(fb.DIR_AUTO, fb.ADV_EDGE, fb.LOOP_DEVICE)
            bg.set_switch(alpha, beta)
            for s in g.sources[:3]:
                s = int(s)
                print(f"[gpu] switch {alpha},{beta} {g.name} source={s}", flush=True)
                L, dist, parent, sizes = run_hip(bg, g.n, s)
                ref = oracle.bfs(g.row_ptr, g.col_idx, s)
                oracle.assert_bfs_ok(g.row_ptr, g.col_idx, s, ref, dist, parent, L, sizes[:L],
                                     symmetric=True, label=f"{g.name} s={s} switch {alpha},{beta}")
                _, dirs, _ = bg.stats()
                if alpha == 10**6 and L > 2:
                    assert dirs[1] == 1, dirs


def test_queue_free_wide_levels():
    """A wide top-down level whose next level may pull writes its new vertices
    to the next bitmap only.  From the centre of a star of 200,000 leaves
    beside an R-MAT component (so that the remaining edges outweigh the
    leaves), alpha = 1 or 4 keeps the leaf level top-down, and it expands from
    that bitmap; the path is taken (a top-down level of at least 2^17 frontier
    edges followed by a top-down level) and results never change."""
    import frontier_bfs_csr_amd as fb
    g = gg.disjoint_union(gg.star_graph(200_001), gg.rmat(16, 16, seed=23, nsrc=1))
    rp, ci = to_dev(g)
    seen = 0
    with fb.BfsGraph(rp, ci) as bg:
        for alpha in (1, 4, 40):
            bg.set_switch(alpha, 48)
            for s in (0, 1, 5, 200_001 + 7):
                print(f"[gpu] queue-free levels alpha={alpha} source={s}", flush=True)
                L, dist, parent, sizes = run_hip(bg, g.n, s)
                ref = oracle.bfs(g.row_ptr, g.col_idx, s)
                oracle.assert_bfs_ok(g.row_ptr, g.col_idx, s, ref, dist, parent, L, sizes[:L],
                                     symmetric=True, label=f"{g.name} s={s} alpha={alpha}")
                _, dirs, fdeg = bg.stats()
                seen += sum(1 for k in range(L - 1)
                            if dirs[k] == 0 and dirs[k + 1] == 0 and fdeg[k] >= 1 << 17)
    assert seen > 0


def test_timing_hooks():
    """Per-launch timing splits the level launches between the two kernels."""
    import frontier_bfs_csr_amd as fb
    g = gg.rmat(14, 16, seed=5, nsrc=2)
    rp, ci = to_dev(g)
    with fb.BfsGraph(rp, ci) as bg:
        for pol in ((0, 0, 0), (0, 0, 1), (0, 0, 2)):
            bg.set_policy(*pol)
            bg.set_timing(True)
            L, dist, parent, sizes = run_hip(bg, g.n, g.sources[0])
            init_ms, level_ms, launches = bg.timing()
            kt = bg.kernel_timing()
            assert kt["td"][1] + kt["bu"][1] == launches, (pol, kt, launches)
            assert kt["td"][1] - kt["bu"][1] in (0, 1), kt   # they alternate, top-down first
            assert abs(kt["td"][0] + kt["bu"][0] - level_ms) <= 1e-3 * max(1.0, level_ms)
            _, dirs, _ = bg.stats()
            ms, ran = bg.launch_timing()
            assert ms.shape[0] == launches
            assert abs(float(ms.sum()) - level_ms) <= 1e-3 * max(1.0, level_ms)
            # every bottom-up level ran in a bottom-up launch of its own, which
            # recorded it; one more bottom-up record when such a launch found
            # the empty frontier
            nbu = int((dirs == 1).sum())
            assert int((ran == 2).sum()) in (nbu, nbu + 1), (pol, dirs, ran)
            assert kt["bu"][1] >= nbu
            if pol[2] == 2:   # one level per launch: a top-down record per top-down level
                ntd = int((dirs == 0).sum())
                assert int((ran == 1).sum()) in (ntd, ntd + 1), (pol, dirs, ran)
            assert init_ms > 0 and level_ms > 0
            bg.set_timing(False)


def test_launch_plan_follows_last_search():
    """A search enqueues the recent searches' working launches (those that ran
    a level or found the end) first: the repeated search uses no more
    launches, and searches whose direction pattern differs from the last one,
    or that run longer than the recorded launches, still give the oracle's
    result."""
    import frontier_bfs_csr_amd as fb
    g = gg.rmat(15, 16, seed=7, nsrc=4)
    rp, ci = to_dev(g)
    with fb.BfsGraph(rp, ci) as bg:
        bg.set_timing(True)
        s0 = int(g.sources[0])
        run_hip(bg, g.n, s0)
        first = bg.timing()[2]
        run_hip(bg, g.n, s0)
        again = bg.timing()[2]
        assert again <= first, (first, again)
        leaves = np.nonzero(np.diff(g.row_ptr) == 1)[0][:3]
        for s in list(g.sources) + [int(x) for x in leaves] + [s0]:
            L, dist, parent, sizes = run_hip(bg, g.n, int(s))
            ref = oracle.bfs(g.row_ptr, g.col_idx, int(s))
            oracle.assert_bfs_ok(g.row_ptr, g.col_idx, int(s), ref, dist, parent, L, sizes[:L],
                                 label=f"plan rmat15 s={s}")
            kt = bg.kernel_timing()
            assert kt["td"][1] + kt["bu"][1] == bg.timing()[2]
    for h in (gg.grid_full(50, 40), gg.disjoint_union(gg.star_graph(3000), gg.path_graph(200))):
        rp, ci = to_dev(h)
        with fb.BfsGraph(rp, ci) as bg:
            for s in (0, h.n - 1, 0, h.n // 2, h.n - 1):
                L, dist, parent, sizes = run_hip(bg, h.n, s)
                ref = oracle.bfs(h.row_ptr, h.col_idx, s)
                oracle.assert_bfs_ok(h.row_ptr, h.col_idx, s, ref, dist, parent, L, sizes[:L],
                                     label=f"plan {h.name} s={s}")


def test_optional_outputs():
    import torch
    import frontier_bfs_csr_amd as fb
    g = gg.rmat(12, 16, seed=3, nsrc=2)
    rp, ci = to_dev(g)
    with fb.BfsGraph(rp, ci) as bg:
        for wp, ws in ((False, False), (True, False), (False, True)):
            L, dist, parent, sizes = run_hip(bg, g.n, g.sources[0], wp, ws)
            ref = oracle.bfs(g.row_ptr, g.col_idx, int(g.sources[0]))
            assert L == ref[3] and (dist == ref[0]).all()


def test_repeated_runs_and_two_handles():
    import torch
    import frontier_bfs_csr_amd as fb
    g1 = gg.rmat(13, 16, seed=21, nsrc=3)
    g2 = gg.grid_full(50, 40)
    r1, c1 = to_dev(g1)
    r2, c2 = to_dev(g2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with fb.BfsGraph(r1, c1) as b1, fb.BfsGraph(r2, c2) as b2:
        for rep in range(3):
            for s in g1.sources:
                d1 = torch.empty(g1.n, dtype=torch.int32, device="cuda")
                d2 = torch.empty(g2.n, dtype=torch.int32, device="cuda")
                with torch.cuda.stream(s1):
                    L1 = b1.run(int(s), d1, stream=s1)
                with torch.cuda.stream(s2):
                    L2 = b2.run(0, d2, stream=s2)
                torch.cuda.synchronize()
                ref1 = oracle.bfs(g1.row_ptr, g1.col_idx, int(s))
                assert L1 == ref1[3] and (d1.cpu().numpy() == ref1[0]).all()
                assert L2 == 50 + 40 - 1
                rr, cc = np.divmod(np.arange(g2.n), 50)
                assert (d2.cpu().numpy() == rr + cc).all()


def test_invalid_graphs_rejected():
    import torch
    import frontier_bfs_csr_amd as fb
    cases = [
        (np.array([1, 2, 3], np.int32), np.array([0, 1, 0], np.int32), "row_ptr[0]"),
        (np.array([0, 2, 1, 3], np.int32), np.array([1, 2, 0], np.int32), "decreasing at index 1"),
        (np.array([0, 1, 2], np.int32), np.array([1, 5], np.int32), "col_idx[1]"),
        (np.array([0, 1, 2], np.int32), np.array([-1, 0], np.int32), "col_idx[0]"),
    ]
    for rp, ci, msg in cases:
        with pytest.raises(fb.BfsError) as ei:
            fb.bfs_graph_create(rp.shape[0] - 1, torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda())
        assert msg in str(ei.value), (msg, str(ei.value))


def test_run_argument_errors():
    import torch
    import frontier_bfs_csr_amd as fb
    g = gg.chapter22_graph()
    rp, ci = to_dev(g)
    with fb.BfsGraph(rp, ci) as bg:
        d = torch.full((g.n,), 9, dtype=torch.int32, device="cuda")
        for bad in (-1, g.n):
            with pytest.raises(fb.BfsError) as ei:
                bg.run(bad, d)
            assert ei.value.code == fb.BFS_EINVAL
        assert (d.cpu().numpy() == 9).all()   # untouched on EINVAL
        # the binding refuses output tensors shorter than n before any launch
        short = torch.full((g.n - 1,), 9, dtype=torch.int32, device="cuda")
        for kw in ({"dist": short}, {"dist": d, "parent": short}, {"dist": d, "level_sizes": short}):
            with pytest.raises(ValueError):
                bg.run(0, **kw)
        assert (short.cpu().numpy() == 9).all() and (d.cpu().numpy() == 9).all()
        with pytest.raises(fb.BfsError):
            bg.set_policy(7)                   # unknown direction
        with pytest.raises(fb.BfsError):
            bg.set_switch(0, 24)               # alpha outside [1, 1e6]
        info = bg.info()
        assert not info["symmetric"] and info["pull_ready"]   # directed: pull via the transpose
        bg.set_policy(fb.DIR_PULL)


def test_unaligned_col_idx():
    """col_idx starting 4 bytes past a 16-byte boundary (the bottom-up scan
    then takes its scalar-load path)."""
    import torch
    import frontier_bfs_csr_amd as fb
    g = gg.rmat(13, 16, seed=31, nsrc=3)
    rp = torch.from_numpy(g.row_ptr).cuda()
    buf = torch.zeros(g.m + 1, dtype=torch.int32, device="cuda")
    buf[1:] = torch.from_numpy(g.col_idx).cuda()
    ci = buf[1:]
    assert ci.data_ptr() % 16 != 0
    with fb.BfsGraph(rp, ci) as bg:
        for pol in ((2, 0, 0), (0, 0, 0)):
            bg.set_policy(*pol)
            for s in g.sources:
                L, dist, parent, sizes = run_hip(bg, g.n, s)
                ref = oracle.bfs(g.row_ptr, g.col_idx, int(s))
                oracle.assert_bfs_ok(g.row_ptr, g.col_idx, int(s), ref, dist, parent, L, sizes[:L],
                                     label=f"unaligned s={s} {pol}")


def test_unaligned_outputs():
    """dist and parent starting 4 bytes past a 16-byte boundary: the start of
    a search then initialises them entry by entry; the sources include the
    first and last vertices (an aligned group's first lane and the tail)."""
    import torch
    import frontier_bfs_csr_amd as fb
    g = gg.rmat(13, 16, seed=33, nsrc=3)
    rp, ci = to_dev(g)
    db = torch.full((g.n + 1,), 5, dtype=torch.int32, device="cuda")
    pb = torch.full((g.n + 1,), 5, dtype=torch.int32, device="cuda")
    dist, parent = db[1:], pb[1:]
    assert dist.data_ptr() % 16 != 0 and parent.data_ptr() % 16 != 0
    sizes = torch.zeros(g.n, dtype=torch.int32, device="cuda")
    deg = np.diff(g.row_ptr)
    last = int(np.nonzero(deg)[0][-1])
    with fb.BfsGraph(rp, ci) as bg:
        for s in list(g.sources) + [int(np.nonzero(deg)[0][0]), last]:
            L = bg.run(int(s), dist, parent, sizes)
            ref = oracle.bfs(g.row_ptr, g.col_idx, int(s))
            oracle.assert_bfs_ok(g.row_ptr, g.col_idx, int(s), ref, dist.cpu().numpy(), parent.cpu().numpy(),
                                 L, sizes[:L].cpu().numpy(), label=f"unaligned outputs s={s}")
            assert int(db[0]) == 5 and int(pb[0]) == 5   # nothing written before the arrays


def test_single_workgroup_small_graphs():
    """Graphs of at most 3,584 vertices under the default policy are searched
    by one workgroup in one launch (visited bits and frontiers in LDS): the
    oracle's results on both sides of that bound, on directed graphs, from a
    source of degree 0, and on a dense graph whose levels take many edge
    passes; the run is one top-down launch and the statistics are top-down."""
    import frontier_bfs_csr_amd as fb
    cases = [
        (gg.random_directed(3584, 12, 41), True),    # exactly at the bound
        (gg.random_directed(3585, 12, 42), False),   # one vertex above it
        (gg.rmat(11, 16, seed=43, nsrc=4), True),
        (gg.complete_graph(600), True),              # 359,400 entries: 44 passes on level 1
        (gg.disjoint_union(gg.star_graph(2000), gg.path_graph(300)), True),
        (gg.c1_chung_lu(), True),
    ]
    for g, one in cases:
        rp, ci = to_dev(g)
        with fb.BfsGraph(rp, ci) as bg:
            bg.set_timing(True)
            deg = np.diff(g.row_ptr)
            srcs = [int(x) for x in g.sources[:3]]
            if (deg == 0).any():
                srcs.append(int(np.nonzero(deg == 0)[0][0]))   # a source of degree 0
            for s in srcs:
                print(f"[gpu] single workgroup {g.name} n={g.n} source={s}", flush=True)
                L, dist, parent, sizes = run_hip(bg, g.n, s)
                ref = oracle.bfs(g.row_ptr, g.col_idx, s)
                oracle.assert_bfs_ok(g.row_ptr, g.col_idx, s, ref, dist, parent, L, sizes[:L],
                                     symmetric=g.symmetric, label=f"single workgroup {g.name} s={s}")
                kt = bg.kernel_timing()
                Ls, dirs, fdeg = bg.stats()
                assert Ls == L
                if one:
                    assert kt["td"][1] == 1 and kt["bu"][1] == 0, kt
                    assert (dirs == 0).all()
                    assert int(fdeg[0]) == int(deg[s])


def test_sources_across_components():
    """One handle, its launch plan learnt from the searches before, with
    sources in turn in an R-MAT component (which pulls), on a path, and of
    degree 0, under several policies; outputs start out holding garbage, so
    an entry a search leaves unwritten shows."""
    big = gg.rmat(14, 16, seed=21, nsrc=3)
    assert (np.diff(big.row_ptr) == 0).any()   # isolated vertices in the pulled part
    g = gg.disjoint_union(gg.disjoint_union(big, gg.path_graph(40)), gg.path_graph(1))
    b = [int(s) for s in big.sources]
    srcs = b + [big.n + 5, g.n - 1, b[0], big.n + 39, g.n - 1, b[1], b[2]]
    check_graph(g, sources=srcs, policies=["auto"])
    check_graph(g, sources=[b[0], big.n + 20, b[1]], policies=["pull", "auto", "push_edge", "auto"])
