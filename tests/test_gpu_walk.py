"""The isolated neighbour walk (the Day 38 page's per-level mapping
measurement) through the C ABI: every mapping returns, for every listed
vertex, the oracle's wrapping checksum bit for bit."""
import numpy as np
import pytest

import graphgen as gg
import oracle
from gpu_util import to_dev

pytestmark = pytest.mark.gpu

MAPPINGS = (0, 1, 2, 3)   # lane, wavefront, binned, edge-balanced


def _levels(g, source):
    dist, _, sizes, L, order = oracle.bfs(g.row_ptr, g.col_idx, int(source), want_order=True)
    starts = np.concatenate([[0], np.cumsum(sizes)])
    return [order[starts[k]:starts[k + 1]] for k in range(L)]


def _walk_all(bg, g, vertices, repeats):
    import torch
    v = torch.from_numpy(np.ascontiguousarray(vertices, np.int32)).cuda()
    want = oracle.walk_checksum(g.row_ptr, g.col_idx, vertices, repeats)
    for mapping in MAPPINGS:
        out = torch.full((max(len(vertices), 1),), 7, dtype=torch.int32, device="cuda")
        print(f"[gpu] walk {g.name} count={len(vertices)} mapping={mapping} repeats={repeats}", flush=True)
        bg.walk(v, out, mapping, repeats)
        got = out[:len(vertices)].cpu().numpy().view(np.uint32)
        assert (got == want).all(), (g.name, mapping, repeats, np.nonzero(got != want)[0][:5])


@pytest.mark.parametrize("name", ["c1", "rmat14", "directed", "hubs"])
def test_walk_levels(name):
    import frontier_bfs_csr_amd as fb
    if name == "c1":
        g = gg.c1_chung_lu()
    elif name == "rmat14":
        g = gg.rmat(14, 16, seed=31, nsrc=1)
    elif name == "directed":
        g = gg.random_directed(5000, 12, 9)
    else:   # lists around every bin threshold: stars of 1 .. 3000 leaves
        g = gg.disjoint_union(gg.star_graph(3001), gg.disjoint_union(gg.star_graph(600), gg.star_graph(40)))
    rp, ci = to_dev(g)
    with fb.BfsGraph(rp, ci) as bg:
        for vertices in _levels(g, g.sources[0]) if name != "hubs" else [np.arange(g.n, dtype=np.int32)]:
            for repeats in (64,) if len(vertices) > 3 else (0, 1, 64):
                _walk_all(bg, g, vertices, repeats)


def test_walk_edge_cases():
    import torch
    import frontier_bfs_csr_amd as fb
    g = gg.rmat(12, 16, seed=32, nsrc=1)
    rp, ci = to_dev(g)
    with fb.BfsGraph(rp, ci) as bg:
        _walk_all(bg, g, np.zeros(0, np.int32), 64)                      # empty list
        _walk_all(bg, g, np.array([5, 5, 5, 0], np.int32), 3)            # repeats of one vertex
        _walk_all(bg, g, np.arange(g.n)[::-1].astype(np.int32), 2)       # every vertex, reversed
        # the list-length limit (8n): at it every mapping runs, above it the call is refused
        rng = np.random.default_rng(33)
        _walk_all(bg, g, rng.integers(0, g.n, 8 * g.n).astype(np.int32), 1)
        big = torch.zeros(8 * g.n + 1, dtype=torch.int32, device="cuda")
        with pytest.raises(fb.BfsError) as ei:
            bg.walk(big, big, fb.WALK_MERGE, 1)
        assert ei.value.code == fb.BFS_EINVAL
        out = torch.zeros(4, dtype=torch.int32, device="cuda")
        for mapping in MAPPINGS:
            for bad in ([0, g.n, 1], [-1]):
                v = torch.tensor(bad, dtype=torch.int32, device="cuda")
                with pytest.raises(fb.BfsError) as ei:
                    bg.walk(v, out, mapping, 4)
                assert ei.value.code == fb.BFS_EINVAL
        with pytest.raises(fb.BfsError):
            bg.walk(torch.zeros(1, dtype=torch.int32, device="cuda"), out, 9, 4)   # unknown mapping


def test_walk_heavy_level():
    # two million entries: the edge-balanced walk takes its longest runs and
    # several grid-stride passes; the bins hold lists of every class
    import frontier_bfs_csr_amd as fb
    g = gg.rmat(16, 16, seed=34, nsrc=1)
    rp, ci = to_dev(g)
    with fb.BfsGraph(rp, ci) as bg:
        _walk_all(bg, g, np.arange(g.n, dtype=np.int32), 8)
