"""Pins for the oracle: checks against things other than the oracle itself.

Each pin returns None when it holds, or a short description of the failure.
They are collected here (not in a test file) so that the mutation tests can run
the same pins against deliberately broken oracle builds.
"""
import json
import os

import numpy as np

import graphgen as gg
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def floyd_warshall(n, row_ptr, col_idx):
    """All-pairs hop distances by Floyd-Warshall on the 0/1 adjacency matrix;
    unreachable = -1."""
    INF = np.iinfo(np.int64).max // 4
    D = np.full((n, n), INF, dtype=np.int64)
    for u in range(n):
        for e in range(row_ptr[u], row_ptr[u + 1]):
            D[u, col_idx[e]] = 1
    np.fill_diagonal(D, 0)
    for k in range(n):
        D = np.minimum(D, D[:, k:k + 1] + D[k:k + 1, :])
    D[D >= INF] = -1
    return D


def _cmp(name, got, want):
    got = np.asarray(got).tolist()
    want = np.asarray(want).tolist()
    if got != want:
        return f"{name}: got {got}, expected {want}"
    return None


def pin_chapter22_bfs():
    """Printed dist, dequeue order, level groups and termination level."""
    G = load_golden("chapter22_6v.json")
    rp, ci, s = G["graph"]["row_offsets"], G["graph"]["col_idx"], G["graph"]["source"]
    dist, parent, sizes, L, order = oracle.bfs(rp, ci, s, want_order=True)
    want = G["bfs_from_0"]
    for r in (_cmp("dist", dist, want["dist"]), _cmp("order", order, want["dequeue_order"])):
        if r:
            return r
    groups = [sorted(np.flatnonzero(dist == k).tolist()) for k in range(L)]
    if groups != want["levels"]:
        return f"levels {groups}"
    if L != G["termination"]["level_after_last_nonempty"]:
        return f"L={L}"
    return _cmp("sizes", sizes, [len(g) for g in want["levels"]])


def pin_chapter22_partial_states():
    """State after level 1 (dist masked to <= 2, exactly 2 discoveries), the
    next frontier {3,4}, the level-2 degree scan, edge map and next frontier."""
    G = load_golden("chapter22_6v.json")
    rp = np.array(G["graph"]["row_offsets"])
    ci = np.array(G["graph"]["col_idx"])
    dist, parent, sizes, L = oracle.bfs(rp, ci, 0)
    a1 = G["after_level_1"]
    masked = np.where(dist <= 2, dist, -1)
    r = _cmp("dist after level 1", masked, a1["dist"])
    if r:
        return r
    if L <= 2 or sizes[2] != a1["discoveries_cas"]:
        return f"level-2 size {sizes[2] if L > 2 else None}"
    if sorted(np.flatnonzero(dist == 1).tolist()) != a1["frontier"]:
        return "level-1 frontier"
    if sorted(np.flatnonzero(dist == 2).tolist()) != G["next_frontier_level_1"]["set"]:
        return "level-2 set"
    ep = G["edge_parallel_level_2"]
    f2 = np.flatnonzero(dist == 2)
    if f2.tolist() != ep["frontier"]:
        return "frontier {3,4}"
    deg = rp[f2 + 1] - rp[f2]
    offs = np.concatenate([[0], np.cumsum(deg)])
    for r in (_cmp("degree", deg, ep["frontier_degree"]), _cmp("offsets", offs, ep["frontier_offsets"])):
        if r:
            return r
    edges = [[int(u), int(ci[e])] for u in f2 for e in range(rp[u], rp[u + 1])]
    if edges != ep["edges"]:
        return f"edges {edges}"
    return _cmp("next frontier", np.flatnonzero(dist == 3), ep["next_frontier"])


def pin_pmpp_graph():
    """Printed neighbour list of vertex 2; distances from 0 and 3 equal the
    Floyd-Warshall rows (derived, not printed)."""
    G = load_golden("pmpp_4v.json")
    rp, ci = np.array(G["graph"]["row_ptr"]), np.array(G["graph"]["col"])
    r = _cmp("adj(2)", sorted(ci[rp[2]:rp[3]].tolist()), G["neighbours_of_2"]["value"])
    if r:
        return r
    D = floyd_warshall(4, rp, ci)
    for s, key in ((0, "dist_from_0"), (3, "dist_from_3")):
        dist, _, _, _ = oracle.bfs(rp, ci, s)
        for r in (_cmp(f"fw row {s}", D[s], G["derived_not_printed"][key]),
                  _cmp(f"dist from {s}", dist, G["derived_not_printed"][key])):
            if r:
                return r
    return None


def pin_tiny_random(count=300, start=0):
    """Brute force: oracle dist == Floyd-Warshall row; level sizes and L
    follow from it; parents pass the checker."""
    for seed in range(start, start + count):
        g = gg.tiny_random(seed)
        D = floyd_warshall(g.n, g.row_ptr, g.col_idx)
        for s in g.sources:
            dist, parent, sizes, L = oracle.bfs(g.row_ptr, g.col_idx, s)
            want = D[s]
            if dist.tolist() != want.tolist():
                return f"seed {seed} source {s}: dist {dist.tolist()} vs FW {want.tolist()}"
            if L != want.max() + 1:
                return f"seed {seed} source {s}: L={L}"
            bc = np.bincount(want[want >= 0], minlength=L)
            if sizes.tolist() != bc.tolist():
                return f"seed {seed} source {s}: sizes"
            code, bad = oracle.check(g.row_ptr, g.col_idx, s, (want, None, bc, int(want.max()) + 1),
                                     dist, parent, L, sizes, symmetric=g.symmetric)
            if code:
                return f"seed {seed} source {s}: checker code {code} at {bad}"
    return None


def pin_closed_forms():
    """Paths, stars, complete graphs, full grids from a corner (dist = r + c,
    sizes = anti-diagonal lengths), disjoint unions (-1 off the component)."""
    for n in (1, 2, 7, 100):
        g = gg.path_graph(n)
        dist, _, sizes, L = oracle.bfs(g.row_ptr, g.col_idx, 0)
        if dist.tolist() != list(range(n)) or L != n or sizes.tolist() != [1] * n:
            return f"path {n}"
    g = gg.star_graph(9)
    d0, _, s0, L0 = oracle.bfs(g.row_ptr, g.col_idx, 0)
    d8, _, s8, L8 = oracle.bfs(g.row_ptr, g.col_idx, 8)
    if L0 != 2 or s0.tolist() != [1, 8] or L8 != 3 or s8.tolist() != [1, 1, 7]:
        return "star"
    g = gg.complete_graph(12)
    d, _, s, L = oracle.bfs(g.row_ptr, g.col_idx, 5)
    if L != 2 or s.tolist() != [1, 11]:
        return "complete"
    w, h = 13, 7
    g = gg.grid_full(w, h)
    d, _, s, L = oracle.bfs(g.row_ptr, g.col_idx, 0)
    rr, cc = np.divmod(np.arange(w * h), w)
    if d.tolist() != (rr + cc).tolist() or L != w + h - 1:
        return "grid dist"
    anti = [sum(1 for r in range(h) for c in range(w) if r + c == k) for k in range(w + h - 1)]
    if s.tolist() != anti:
        return "grid sizes"
    u = gg.disjoint_union(gg.path_graph(5), gg.complete_graph(4))
    d, _, s, L = oracle.bfs(u.row_ptr, u.col_idx, 0)
    if d.tolist() != [0, 1, 2, 3, 4, -1, -1, -1, -1]:
        return "union from 0"
    d, _, s, L = oracle.bfs(u.row_ptr, u.col_idx, 5)
    if d.tolist() != [-1] * 5 + [0, 1, 1, 1]:
        return "union from 5"
    return None


def pin_checker_rejects():
    """The checker rejects each kind of corrupted result (its own negative
    cases), and accepts an alternative valid parent."""
    g = gg.grid_full(6, 5)
    rp, ci = g.row_ptr, g.col_idx
    ref = oracle.bfs(rp, ci, 0)
    dist, parent, sizes, L = ref
    ok, _ = oracle.check(rp, ci, 0, ref, dist, parent, L, sizes)
    if ok:
        return f"accepts nothing ({ok})"
    # an alternative valid parent: vertex 7 (r1,c1) may hang off 1 or 6
    alt = parent.copy()
    alt[7] = 1 if parent[7] == 6 else 6
    if oracle.check(rp, ci, 0, ref, dist, alt, L, sizes)[0]:
        return "rejects a valid alternative parent"
    cases = []
    d = dist.copy(); d[29] += 1; cases.append(("dist", 1, dict(dist=d)))
    d = dist.copy(); d[-1] = dist[-1] + 0; cases.append(("L", 2, dict(L=L + 1, sizes=np.append(sizes, 0))))
    sz = sizes.copy(); sz[2] += 1; sz[3] -= 1; cases.append(("sizes", 3, dict(sizes=sz)))
    p = parent.copy(); p[0] = 1; cases.append(("parent src", 5, dict(parent=p)))
    p = parent.copy(); p[13] = 0; cases.append(("parent level", 6, dict(parent=p)))
    # same level as a true parent but not adjacent: vertex 14 (r2,c2) dist 4;
    # vertex 3 (r0,c3) has dist 3 but is not its neighbour
    p = parent.copy(); p[14] = 3; cases.append(("parent edge", 7, dict(parent=p)))
    for name, code, kw in cases:
        args = dict(dist=dist, parent=parent, L=L, sizes=sizes)
        args.update(kw)
        got, _ = oracle.check(rp, ci, 0, ref, **args)
        if got != code:
            return f"{name}: code {got}, expected {code}"
    # unreached vertex with a parent
    u = gg.disjoint_union(gg.path_graph(3), gg.path_graph(2))
    uref = oracle.bfs(u.row_ptr, u.col_idx, 0)
    p = uref[1].copy(); p[4] = 3
    got, _ = oracle.check(u.row_ptr, u.col_idx, 0, uref, uref[0], p, uref[3], uref[2])
    if got != 8:
        return f"unreached parent: code {got}"
    # edge invariants with a reference that is wrong in the same way
    d = dist.copy(); d[29] = d[29] + 2
    bad_ref = (d, None, np.bincount(d, minlength=d.max() + 1), int(d.max()) + 1)
    got, _ = oracle.check(rp, ci, 0, bad_ref, d, None, bad_ref[3], bad_ref[2])
    if got != 9:
        return f"symmetric invariant: code {got}"
    g6 = gg.chapter22_graph()
    d6 = np.array([0, 1, 1, 2, 4, 5], np.int32)
    ref6 = (d6, None, np.array([1, 2, 1, 0, 1, 1]), 6)
    got, _ = oracle.check(g6.row_ptr, g6.col_idx, 0, ref6, d6, None, 6, None, symmetric=False)
    if got != 10:
        return f"directed invariant: code {got}"
    return None


def pin_walk_checksum():
    """The neighbour-walk checksum against closed forms of the XOR sum:
    sum_{r<R} (c ^ r) = R*c + R(R-1)/2 when c has no bit below R set, and
    R*c - R(R-1)/2 when c has every bit below R set (R a power of two), all
    mod 2**32; a vertex's checksum is the sum over its entries; degree 0
    gives 0; the listed order is kept."""
    R = 64
    n = 1 << 20
    c_hi = 1024                 # bits above R only
    c_lo = (1 << 20) - 1        # every bit below R set (and more)
    adj = {0: [0], 1: [c_hi], 2: [c_lo], 3: [c_hi, c_lo, 0], 4: []}
    row_ptr = np.zeros(n + 1, np.int32)
    col = []
    for u in range(n):
        col += adj.get(u, [])
        row_ptr[u + 1] = len(col)
    col = np.array(col, np.int32)
    tri = R * (R - 1) // 2
    f = {0: tri, c_hi: R * c_hi + tri, c_lo: R * c_lo - tri}
    want = {u: sum(f[c] for c in cs) % 2**32 for u, cs in adj.items()}
    order = [3, 0, 4, 2, 1]
    got = oracle.walk_checksum(row_ptr, col, order, R)
    if got.tolist() != [want[u] for u in order]:
        return f"walk checksum {got.tolist()} != {[want[u] for u in order]}"
    # wrap-around: 2**13 repeats of c_lo exceed 2**32 before the reduction
    R2 = 1 << 13
    got2 = int(oracle.walk_checksum(row_ptr, col, [2], R2)[0])
    want2 = (R2 * c_lo - R2 * (R2 - 1) // 2) % 2**32
    if got2 != want2:
        return f"walk checksum with wrap {got2} != {want2}"
    return None


def _bellman_ford(n, row_ptr, col_idx, w, source):
    """Shortest distances by repeated relaxation of every entry (a method
    unlike the oracle's Dijkstra): -1 for unreachable."""
    INF = np.int64(1) << 62
    d = np.full(n, INF, np.int64)
    d[source] = 0
    rows = np.repeat(np.arange(n), np.diff(row_ptr))
    w = w.astype(np.int64)
    for _ in range(n):
        cand = np.where(d[rows] < INF, d[rows] + w, INF)
        new = d.copy()
        np.minimum.at(new, col_idx, cand)
        if (new == d).all():
            break
        d = new
    return np.where(d < INF, d, -1)


def _pred_ok(n, row_ptr, col_idx, w, source, dist, pred):
    """pred[v] is the smallest u with an entry u -> v and dist[u] + w = dist[v]."""
    rows = np.repeat(np.arange(n), np.diff(row_ptr))
    tight = (dist[rows] >= 0) & (dist[rows] + w.astype(np.int64) == dist[col_idx]) & (col_idx != source)
    best = np.full(n, n, np.int64)
    np.minimum.at(best, col_idx[tight], rows[tight])
    want = np.where(dist >= 0, np.where(best < n, best, -1), -1)
    want[source] = source
    return (pred == want).all()


def pin_sssp():
    """SSSP distances against Bellman-Ford on 200 tiny random graphs with
    weights 0..9 (duplicates with different weights, self-loops, directed and
    symmetric); predecessors are the smallest tight in-neighbours; unit
    weights give the BFS levels; weighted paths and stars have closed forms;
    sums beyond 32 bits stay exact."""
    for seed in range(200):
        g = gg.tiny_random(seed)
        w = gg.edge_weights(g.m, seed + 1000, wmax=9, wmin=0)
        for s in g.sources:
            d, p = oracle.sssp(g.row_ptr, g.col_idx, w, int(s))
            bf = _bellman_ford(g.n, g.row_ptr, g.col_idx, w, int(s))
            if not (d == bf).all():
                return f"sssp tiny {seed} s={s}: dist differs from Bellman-Ford"
            if not _pred_ok(g.n, g.row_ptr, g.col_idx, w, int(s), d, p):
                return f"sssp tiny {seed} s={s}: predecessor is not the smallest tight in-neighbour"
        ones = np.ones(g.m, np.uint32)
        s = int(g.sources[0])
        d1, _ = oracle.sssp(g.row_ptr, g.col_idx, ones, s)
        if not (d1 == oracle.bfs(g.row_ptr, g.col_idx, s)[0]).all():
            return f"sssp tiny {seed}: unit weights do not give the BFS levels"
    # weighted path 0-1-...-9 from 0: prefix sums of the forward entries
    g = gg.path_graph(10)
    w = gg.edge_weights(g.m, 7, wmax=1000, wmin=0)
    d, p = oracle.sssp(g.row_ptr, g.col_idx, w, 0)
    rows = np.repeat(np.arange(g.n), np.diff(g.row_ptr))
    fwd = {int(r): int(w[e]) for e, r in enumerate(rows) if g.col_idx[e] == r + 1}
    want = np.concatenate([[0], np.cumsum([fwd[i] for i in range(9)])])
    if not (d == want).all() or not (p == np.concatenate([[0], np.arange(9)])).all():
        return f"sssp path: {d.tolist()} != {want.tolist()}"
    # star from the hub: each leaf at its own entry's weight; from a leaf: via the hub
    g = gg.star_graph(6)
    w = np.arange(1, g.m + 1, dtype=np.uint32) * 3
    d, _ = oracle.sssp(g.row_ptr, g.col_idx, w, 0)
    want = np.zeros(g.n, np.int64)
    for e in range(g.row_ptr[0], g.row_ptr[1]):
        want[g.col_idx[e]] = w[e]
    if not (d == want).all():
        return f"sssp star: {d.tolist()} != {want.tolist()}"
    # all-zero weights: every reachable vertex at 0
    g = gg.tiny_random(3, directed=True)
    d, _ = oracle.sssp(g.row_ptr, g.col_idx, np.zeros(g.m, np.uint32), int(g.sources[0]))
    b = oracle.bfs(g.row_ptr, g.col_idx, int(g.sources[0]))[0]
    if not ((d >= 0) == (b >= 0)).all() or (d[d >= 0] != 0).any():
        return "sssp zero weights"
    # 32-bit weights summed past 2**32
    g = gg.path_graph(4)
    d, _ = oracle.sssp(g.row_ptr, g.col_idx, np.full(g.m, 0xFFFFFFFF, np.uint32), 0)
    if d.tolist() != [0, 0xFFFFFFFF, 2 * 0xFFFFFFFF, 3 * 0xFFFFFFFF]:
        return f"sssp wide sums {d.tolist()}"
    return None


ALL_PINS = [pin_chapter22_bfs, pin_chapter22_partial_states, pin_pmpp_graph,
            pin_tiny_random, pin_closed_forms, pin_checker_rejects, pin_walk_checksum, pin_sssp]


def failing_pins(tiny_count=300):
    out = []
    for pin in ALL_PINS:
        try:
            r = pin(count=tiny_count) if pin is pin_tiny_random else pin()
        except Exception as e:  # a mutant may also crash a pin
            r = f"raised {type(e).__name__}: {e}"
        if r:
            out.append((pin.__name__, r))
    return out
