"""Shortest paths on the benchmark graphs: the atomic-min relaxation that the
Gunrock reading guide extends the BFS lambda to, on the same CSR.  The pages
give no weights, so every CSR entry gets a seeded uniform weight in [1, 255]
(numpy PCG64).  Per source: a warm-up call, then --runs timed calls (wall
time around the call, which returns after the last round); distances and
predecessors of the first --check sources are compared with the oracle's
Dijkstra, whose time is the CPU baseline.  Algorithmic bytes per call count
init, output and 16 bytes per relaxation tried (bfs_last_run_stats gives the
frontier edges of every round), against 8 TB/s.

    python tests/ssspbench.py [--workload c2] [--sources 8]

Prints a table to stderr and one JSON line to stdout.

It lives with the tests because it checks every result against the oracle
(test infrastructure); the library itself never calls the oracle.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

WMAX = 255



def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="c2", choices=["c1", "c2", "c3", "c5"])
    ap.add_argument("--sources", type=int, default=8)
    ap.add_argument("--runs", type=int, default=3)
    ap.add_argument("--check", type=int, default=2, help="sources compared with the oracle")
    ap.add_argument("--seed", type=int, default=11)
    args = ap.parse_args()

    import torch

    import frontier_bfs_csr_amd as fb
    import graphgen as gg

    g = gg.WORKLOADS[args.workload]()
    w = gg.edge_weights(g.m, args.seed, wmax=WMAX)
    dev = torch.device("cuda:0")
    rp = torch.from_numpy(g.row_ptr).to(dev)
    ci = torch.from_numpy(g.col_idx).to(dev)
    wd = torch.from_numpy(w.view(np.int32)).to(dev)
    dist = torch.empty(g.n, dtype=torch.int64, device=dev)
    pred = torch.empty(g.n, dtype=torch.int32, device=dev)
    deg = g.degrees()
    rows = []
    cpu = []
    with fb.BfsGraph(rp, ci) as bg:
        print(f"[sssp] {args.workload}: n={g.n} m={g.m} weights 1..{WMAX} (seed {args.seed})", file=sys.stderr)
        for k, s in enumerate(int(x) for x in g.sources[:args.sources]):
            bg.sssp(s, wd, WMAX, dist, pred)
            torch.cuda.synchronize()
            ts = []
            for _ in range(args.runs):
                t0 = time.perf_counter()
                rounds = bg.sssp(s, wd, WMAX, dist, pred)
                ts.append(time.perf_counter() - t0)
            _, _, fe = bg.stats()
            relax = int(fe.sum())
            # algorithmic bytes, counted low: init (8n keys), output (12n) and,
            # per frontier edge, the neighbour id, weight and target key (16);
            # the frontier vertices' own reads are left out
            alg = 8 * g.n + 12 * g.n + 16 * relax
            d = dist.cpu().numpy()
            reached = d >= 0
            # edges in the source's component (each undirected edge once on
            # symmetric graphs, every out-entry on directed ones)
            medges = int(deg[reached].sum()) // (2 if g.symmetric else 1)
            ms = float(np.mean(ts)) * 1e3
            row = {"source": s, "rounds": rounds, "ms": round(ms, 4), "reached": int(reached.sum()),
                   "gteps": round(medges / (ms * 1e-3) / 1e9, 3), "max_dist": int(d.max()),
                   "relaxations": relax, "alg_GB_per_s": round(alg / (ms * 1e-3) / 1e9, 1)}
            if k < args.check:
                import oracle   # the parity check and CPU baseline: the oracle as it stands
                t0 = time.perf_counter()
                od, op = oracle.sssp(g.row_ptr, g.col_idx, w, s)
                cpu_s = time.perf_counter() - t0
                row["oracle_equal"] = bool((od == d).all() and (op == pred.cpu().numpy()).all())
                row["oracle_ms"] = round(cpu_s * 1e3, 1)
                cpu.append((medges, cpu_s))
            rows.append(row)
            print(f"[sssp] source {s}: {rounds} rounds, {relax} relaxations, {ms:.3f} ms, {row['gteps']} GTEPS, "
                  f"{row['alg_GB_per_s']} GB/s algorithmic"
                  + (f", oracle {row['oracle_ms']} ms, equal {row['oracle_equal']}" if k < args.check else ""),
                  file=sys.stderr, flush=True)
    ms_all = [r["ms"] for r in rows]
    out = {"workload": args.workload, "n": g.n, "m": g.m, "weights": f"uniform 1..{WMAX}, seed {args.seed}",
           "ms_per_source_median": round(float(np.median(ms_all)), 4),
           "gteps_hmean": round(len(rows) / sum(1.0 / r["gteps"] for r in rows), 3),
           "rounds_median": int(np.median([r["rounds"] for r in rows])),
           "cpu_oracle_gteps": round(sum(e for e, _ in cpu) / sum(t for _, t in cpu) / 1e9, 4) if cpu else None,
           "alg_GB_per_s_median": round(float(np.median([r["alg_GB_per_s"] for r in rows])), 1),
           "roofline_frac_median": round(float(np.median([r["alg_GB_per_s"] for r in rows])) / 8000.0, 4),
           "oracle_equal_all": all(r.get("oracle_equal", True) for r in rows), "sources": rows}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
