"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
check it against the oracle."""
import sys

import numpy as np

import oracle

POLICIES = {
    "auto": (0, 0, 0),
    "push_binned": (1, 1, 0),
    "push_edge": (1, 2, 0),
    "pull": (2, 0, 0),
    "auto_edge": (0, 2, 0),
    "auto_binned_hostloop": (0, 1, 1),
    "auto_chain": (0, 0, 2),
}


def policies_for(g):
    """Every policy: pull runs on symmetric graphs and, through the transpose
    the library builds, on directed ones."""
    return list(POLICIES)


def to_dev(g):
    import torch
    rp = torch.from_numpy(np.ascontiguousarray(g.row_ptr)).cuda()
    ci = torch.from_numpy(np.ascontiguousarray(g.col_idx)).cuda()
    return rp, ci


def run_hip(bg, n, source, with_parent=True, with_sizes=True):
    import torch
    dist = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    parent = torch.full((n,), -7, dtype=torch.int32, device="cuda") if with_parent else None
    sizes = torch.full((n,), -7, dtype=torch.int32, device="cuda") if with_sizes else None
    L = bg.run(int(source), dist, parent, sizes)
    torch.cuda.synchronize()
    return (L, dist.cpu().numpy(),
            None if parent is None else parent.cpu().numpy(),
            None if sizes is None else sizes.cpu().numpy())


def is_symmetric(g):
    """Every entry u->v has an entry v->u (self-loops count as symmetric)."""
    rows = np.repeat(np.arange(g.n, dtype=np.int64), np.diff(g.row_ptr))
    fwd = np.unique(rows * g.n + g.col_idx)
    bwd = np.unique(g.col_idx.astype(np.int64) * g.n + rows)
    return fwd.shape == bwd.shape and bool((fwd == bwd).all())


def sorted_rows_copy(g):
    """Same graph with every row sorted ascending (duplicates and self-loops kept)."""
    import copy
    col = g.col_idx.copy()
    for u in range(g.n):
        col[g.row_ptr[u]:g.row_ptr[u + 1]].sort()
    h = copy.copy(g)
    h.col_idx = col
    h.name = g.name + "_sorted"
    return h


def check_graph(g, sources=None, policies=None, label="", ref_cache=None):
    """Every source x policy: bit-exact dist, L and level sizes; valid parents;
    sizes beyond L untouched."""
    import frontier_bfs_csr_amd as fb
    rp, ci = to_dev(g)
    sources = g.sources if sources is None else sources
    policies = policies_for(g) if policies is None else policies
    with fb.BfsGraph(rp, ci) as bg:
        info = bg.info()
        if g.n <= 5000:
            rows_sorted = bool(all((np.diff(g.col_idx[g.row_ptr[u]:g.row_ptr[u + 1]]) >= 0).all()
                                   for u in range(g.n)))
            assert info["sorted_rows"] == rows_sorted, (label, info)
            # symmetry is detected only on sorted rows (it needs a binary search)
            assert info["symmetric"] == (is_symmetric(g) and rows_sorted), (label, info)
        else:
            # generated workloads are symmetric with sorted rows, or directed
            assert info["symmetric"] == g.symmetric, (label, info)
        assert info["pull_ready"], (label, info)
        for s in sources:
            s = int(s)
            key = (g.name, s)
            if ref_cache is not None and key in ref_cache:
                ref = ref_cache[key]
            else:
                ref = oracle.bfs(g.row_ptr, g.col_idx, s)
                if ref_cache is not None:
                    ref_cache[key] = ref
            for pol in policies:
                d, a, lp = POLICIES[pol]
                if d == 2 and not info["pull_ready"]:
                    continue
                bg.set_policy(d, a, lp)
                print(f"[gpu] {label or g.name} n={g.n} m={g.m} source={s} policy={pol}",
                      file=sys.stderr, flush=True)
                L, dist, parent, sizes = run_hip(bg, g.n, s)
                oracle.assert_bfs_ok(g.row_ptr, g.col_idx, s, ref, dist, parent, L, sizes[:L],
                                     symmetric=g.symmetric, label=f"{label or g.name} s={s} {pol}")
                assert (sizes[L:] == -7).all(), f"{label}: level_sizes written beyond L"
                Ls, dirs, fe = bg.stats()
                assert Ls == L and dirs.shape[0] == L
                if d == 1:
                    assert (dirs == 0).all()
                if d == 2:
                    assert (dirs == 1).all()
                deg = np.diff(g.row_ptr).astype(np.int64)
                want_fe = np.bincount(ref[0][ref[0] >= 0], weights=deg[ref[0] >= 0],
                                      minlength=L).astype(np.int64)
                assert (fe == want_fe).all(), f"{label}: frontier edge sums"


def check_sources_parallel(g, sources, policy="auto", chunk=8, workers=8, label=""):
    """dist, L and level sizes bit-exact, parents valid, for many sources of a
    large graph under one policy: the oracle's searches and the checks run on
    host threads (the oracle is C and releases the interpreter lock), the GPU
    searches one after another, `chunk` sources at a time."""
    from concurrent.futures import ThreadPoolExecutor
    import frontier_bfs_csr_amd as fb
    rp, ci = to_dev(g)
    d, a, lp = POLICIES[policy]
    sources = [int(s) for s in sources]
    with fb.BfsGraph(rp, ci) as bg, ThreadPoolExecutor(workers) as pool:
        bg.set_policy(d, a, lp)
        for c0 in range(0, len(sources), chunk):
            part = sources[c0:c0 + chunk]
            refs = list(pool.map(lambda s: oracle.bfs(g.row_ptr, g.col_idx, s), part))
            outs = []
            for s in part:
                print(f"[gpu] {label or g.name} n={g.n} m={g.m} source={s} policy={policy}",
                      file=sys.stderr, flush=True)
                outs.append(run_hip(bg, g.n, s))

            def chk(i):
                s, ref = part[i], refs[i]
                L, dist, parent, sizes = outs[i]
                oracle.assert_bfs_ok(g.row_ptr, g.col_idx, s, ref, dist, parent, L, sizes[:L],
                                     symmetric=g.symmetric, label=f"{label or g.name} s={s} {policy}")
                assert (sizes[L:] == -7).all(), f"{label}: level sizes written beyond L"
                return True
            assert all(pool.map(chk, range(len(part))))
    return len(sources)
