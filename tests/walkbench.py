"""Per-level mapping benchmark: the isolated neighbour walk of every level.

The measurement of the "Day 38 - Graph traversal on a GPU" page ("Measuring
the mapping without measuring the launch"), on MI355X with 64-lane
wavefronts: for each level of one search (frontier in the serial FIFO order,
levels with at least --min-edges entries), each mapping walks the frontier's
lists --repeats times inside the kernel, is warmed up, then timed --runs times
with HIP events on the search stream (mean), and its per-vertex checksums are
compared with the oracle's.  Beside the times it prints the analytic lane-slot
model extended to 64 lanes: the share of issued lane slots that walk an entry.

    python tests/walkbench.py [--workload c1] [--repeats 64]

Prints the table to stderr and one JSON line to stdout.

It lives with the tests because it checks every result against the oracle
(test infrastructure); the library itself never calls the oracle.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

NAMES = {0: "lane", 1: "wave", 2: "binned", 3: "merge"}
WAVE, BLOCK, T_LANE, T_WG, MERGE_K = 64, 512, 32, 512, 4
MERGE_LANES = 256 * 2 * BLOCK   # the merge walk's grid on 256 compute units


def lane_slots(deg, mapping):
    """Lane slots one pass of a mapping issues for a frontier with these
    degrees (in frontier order): a wavefront runs until its longest list ends."""
    deg = np.asarray(deg, np.int64)
    if mapping == 0:
        pad = (-len(deg)) % WAVE
        d = np.concatenate([deg, np.zeros(pad, np.int64)]).reshape(-1, WAVE)
        return int(d.max(axis=1).sum() * WAVE)
    if mapping == 1:
        return int((np.ceil(deg / WAVE) * WAVE).sum())
    if mapping == 2:
        # global bins: the lane bin is packed 64 lists to a wavefront
        small = deg[deg < T_LANE]
        pad = (-len(small)) % WAVE
        d = np.concatenate([small, np.zeros(pad, np.int64)]).reshape(-1, WAVE)
        mid = deg[(deg >= T_LANE) & (deg < T_WG)]
        big = deg[deg >= T_WG]
        return int(d.max(axis=1).sum() * WAVE + (np.ceil(mid / WAVE) * WAVE).sum()
                   + (np.ceil(big / BLOCK) * BLOCK).sum())
    # merge: runs of equal length, one per lane, the last one short
    E = int(deg.sum())
    k = min(MERGE_K, max(1, -(-E // MERGE_LANES)))
    return -(-E // k) * k


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="c1", choices=["c1", "c2", "c3", "c5"])
    ap.add_argument("--repeats", type=int, default=64)
    ap.add_argument("--runs", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--min-edges", type=int, default=1000)
    ap.add_argument("--mappings", default="lane,wave,binned,merge",
                    help="comma-separated subset of lane, wave, binned, merge")
    args = ap.parse_args()
    maps = [m for m in NAMES if NAMES[m] in args.mappings.split(",")]

    import torch

    import frontier_bfs_csr_amd as fb
    import graphgen as gg
    import oracle

    g = gg.WORKLOADS[args.workload]()
    src = int(g.sources[0])
    _, _, sizes, L, order = oracle.bfs(g.row_ptr, g.col_idx, src, want_order=True)
    starts = np.concatenate([[0], np.cumsum(sizes)])
    deg_all = np.diff(g.row_ptr).astype(np.int64)
    dev = torch.device("cuda:0")
    rp = torch.from_numpy(g.row_ptr).to(dev)
    ci = torch.from_numpy(g.col_idx).to(dev)
    stream = torch.cuda.current_stream()
    rows = []
    with fb.BfsGraph(rp, ci) as bg:
        print(f"[walk] {args.workload}: n={g.n} m={g.m} source={src} L={L}, walk x{args.repeats}",
              file=sys.stderr)
        print(f"{'level':>5} {'frontier':>9} {'edges':>10} {'max deg':>8} " +
              " ".join(f"{NAMES[m] + ' ms':>11} {'slots%':>6}" for m in maps), file=sys.stderr)
        for k in range(L):
            vs = order[starts[k]:starts[k + 1]].astype(np.int32)
            deg = deg_all[vs]
            edges = int(deg.sum())
            if edges < args.min_edges:
                continue
            want = oracle.walk_checksum(g.row_ptr, g.col_idx, vs, args.repeats)
            v = torch.from_numpy(vs).to(dev)
            out = torch.empty(len(vs), dtype=torch.int32, device=dev)
            row = {"level": k, "frontier": int(len(vs)), "edges": edges, "max_degree": int(deg.max())}
            for m in maps:
                for _ in range(args.warmup):
                    bg.walk(v, out, m, args.repeats, stream)
                bg.set_timing(True)
                ms = 0.0
                for _ in range(args.runs):
                    bg.walk(v, out, m, args.repeats, stream)
                    ms += bg.timing()[1]
                bg.set_timing(False)
                got = out.cpu().numpy().view(np.uint32)
                if not (got == want).all():
                    raise SystemExit(f"level {k} mapping {NAMES[m]}: checksum differs from the oracle")
                slots = lane_slots(deg, m)
                row[NAMES[m]] = {"ms": round(ms / args.runs, 5),
                                 "lane_slot_use": round(edges / slots, 4) if slots else None}
            rows.append(row)
            print(f"{k:>5} {row['frontier']:>9} {edges:>10} {row['max_degree']:>8} " +
                  " ".join(f"{row[NAMES[m]]['ms']:>11.4f} {100 * (row[NAMES[m]]['lane_slot_use'] or 0):>6.1f}"
                           for m in maps), file=sys.stderr)
    print(json.dumps({"workload": args.workload, "source": src, "repeats": args.repeats, "runs": args.runs,
                      "levels": rows, "checksums": "equal to the oracle on every level and mapping"}))


if __name__ == "__main__":
    main()
