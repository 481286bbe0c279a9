"""Single-source shortest paths (bfs_sssp) through the C ABI: distances and
predecessors equal the oracle's (Dijkstra; predecessor = smallest tight
in-neighbour) exactly, on tiny random weighted graphs, closed forms,
directed graphs and R-MAT; plus the argument and weight-bound checks."""
import numpy as np
import pytest

import graphgen as gg
import oracle
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _run(bg, g, w_dev, maxw, s):
    import torch
    dist = torch.full((g.n,), -7, dtype=torch.int64, device="cuda")
    pred = torch.full((g.n,), -7, dtype=torch.int32, device="cuda")
    rounds = bg.sssp(int(s), w_dev, maxw, dist, pred)
    torch.cuda.synchronize()
    return rounds, dist.cpu().numpy(), pred.cpu().numpy()


def _check(g, w, maxw, sources, label):
    import torch
    import frontier_bfs_csr_amd as fb
    rp, ci = to_dev(g)
    w_dev = torch.from_numpy(w.view(np.int32)).cuda()
    with fb.BfsGraph(rp, ci) as bg:
        for s in sources:
            print(f"[gpu] sssp {label} n={g.n} m={g.m} source={s} maxw={maxw}", flush=True)
            rounds, d, p = _run(bg, g, w_dev, maxw, s)
            wd, wp = oracle.sssp(g.row_ptr, g.col_idx, w, int(s))
            assert rounds >= 1
            Ls, dirs, fe = bg.stats()        # per round: the frontier edges relaxed
            assert Ls == rounds and fe.shape[0] == rounds and (fe >= 0).all()
            deg = np.diff(g.row_ptr)
            assert fe[0] == deg[int(s)]
            bad = np.nonzero(d != wd)[0]
            assert bad.size == 0, (label, s, bad[:5], d[bad[:5]], wd[bad[:5]])
            bad = np.nonzero(p != wp)[0]
            assert bad.size == 0, (label, s, bad[:5], p[bad[:5]], wp[bad[:5]])


def test_sssp_tiny_random():
    for seed in range(60):
        g = gg.tiny_random(seed)
        w = gg.edge_weights(g.m, seed + 500, wmax=9, wmin=0)
        _check(g, w, 9, g.sources, f"tiny{seed}")


def test_sssp_closed_forms_and_edges():
    g = gg.path_graph(2000)                       # 1,999 rounds at least
    _check(g, gg.edge_weights(g.m, 1, wmax=100), 100, [0, 999], "path")
    g = gg.star_graph(3000)
    _check(g, gg.edge_weights(g.m, 2, wmax=50), 50, [0, 5], "star")
    g = gg.tiny_random(5, directed=True)
    _check(g, np.zeros(g.m, np.uint32), 0, g.sources, "zero_weights")
    g = gg.path_graph(1)
    _check(g, np.zeros(0, np.uint32), 1, [0], "single_vertex")


def test_sssp_directed_and_rmat():
    g = gg.random_directed(5000, 12, 9)
    _check(g, gg.edge_weights(g.m, 3), 255, g.sources[:2], "directed")
    g = gg.rmat(14, 16, seed=31, nsrc=2)
    _check(g, gg.edge_weights(g.m, 4), 255, g.sources, "rmat14")
    g = gg.rmat_directed(14, nsrc=2)
    _check(g, gg.edge_weights(g.m, 5, wmax=1000), 1000, g.sources, "rmat14_directed")
    g = gg.rmat(17, 16, seed=36, nsrc=1)
    _check(g, gg.edge_weights(g.m, 6), 255, g.sources, "rmat17")


def test_sssp_arguments():
    import torch
    import frontier_bfs_csr_amd as fb
    g = gg.path_graph(100)
    rp, ci = to_dev(g)
    w = torch.from_numpy(gg.edge_weights(g.m, 7, wmax=10).view(np.int32)).cuda()
    dist = torch.zeros(g.n, dtype=torch.int64, device="cuda")
    with fb.BfsGraph(rp, ci) as bg:
        for src in (-1, g.n):
            with pytest.raises(fb.BfsError) as ei:
                bg.sssp(src, w, 10, dist)
            assert ei.value.code == fb.BFS_EINVAL
        with pytest.raises(fb.BfsError) as ei:          # n * max_weight reaches 2^32 - 1
            bg.sssp(0, w, -(-((1 << 32) - 1) // g.n), dist)
        assert ei.value.code == fb.BFS_EINVAL
        with pytest.raises(fb.BfsError) as ei:          # a weight above the declared maximum
            bg.sssp(0, w, 5, dist)
        assert ei.value.code == fb.BFS_EINVAL and "above max_weight" in str(ei.value)
        rounds = bg.sssp(0, w, 10, dist)                 # the handle still works
        assert rounds >= 99
        assert (dist.cpu().numpy() == oracle.sssp(g.row_ptr, g.col_idx, w.cpu().numpy().view(np.uint32), 0)[0]).all()
        with pytest.raises(TypeError):
            bg.sssp(0, w, 10, torch.zeros(g.n, dtype=torch.int32, device="cuda"))
        # weights shorter than m, or outputs shorter than n, are refused
        with pytest.raises(ValueError):
            bg.sssp(0, w[:-1], 10, dist)
        with pytest.raises(ValueError):
            bg.sssp(0, w, 10, dist[:-1])
        with pytest.raises(ValueError):
            bg.sssp(0, w, 10, dist, torch.zeros(g.n - 1, dtype=torch.int32, device="cuda"))
