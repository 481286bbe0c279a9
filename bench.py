"""Benchmark: level-synchronous BFS over an int32 CSR graph on one MI355X.

One step = one complete search (initialisation plus every level) from the next
source of the workload's source list, with the graph already resident in HBM.
Prints ONE JSON line:

  value       GTEPS = sum over timed steps of the edges in the part of the
              graph the search reached (undirected edges; out-edges of the
              reached vertices on the directed workloads) / wall time of the
              timed steps
  roofline    for the dominant level kernel (bfs_td_kernel or bfs_bu_kernel, or
              bfs_one_kernel for a small graph under the default policy,
              whichever takes more time): algorithmic bytes of the levels it
              ran (byte model in frontier_bfs_csr_amd/csrc/bytemodel.c) / its
              summed launch time, each launch timed by HIP events on the search
              stream in a second pass over the same sources, against 8 TB/s
  cpu_baseline  the CPU oracle (serial FIFO BFS, one core) on a bounded sample
              of the same sources, same GTEPS definition

Usage: python bench.py [--gpus 1] [--steps 64] [--warmup 4] [--workload c5]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
WORKLOAD_DESC = {
    "c1": "chung_lu_3485: Chung-Lu power-law (exponent 2.1), largest component, max-eccentricity source",
    "c2": "rmat20_ef16: R-MAT scale 20, edge factor 16, (0.57,0.19,0.19,0.05), symmetrised, deduplicated",
    "c3": "er_4M_deg16: Erdos-Renyi 4,194,304 vertices, 8n uniform pairs symmetrised",
    "c4": "grid4096_del5: 4096x4096 4-neighbour grid, 5% edges deleted, largest component, corner source",
    "c5": "rmat24_ef16: R-MAT scale 24, edge factor 16, (0.57,0.19,0.19,0.05), symmetrised, deduplicated",
    "c2d": "rmat20_ef16_directed: R-MAT scale 20, edge factor 16, (0.57,0.19,0.19,0.05), directed, deduplicated",
    "c5d": "rmat24_ef16_directed: R-MAT scale 24, edge factor 16, (0.57,0.19,0.19,0.05), directed, deduplicated",
}
DIRECTED = {"c2d": (20, 6), "c5d": (24, 7)}   # scale, seed
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "level_kernels_traffic.json")
KERNEL_NAMES = {"td": "bfs_td_kernel", "bu": "bfs_bu_kernel"}


def kernel_source_hash():
    h = hashlib.sha256()
    for fn in ("bfs_device.hip", "bfs_internal.h"):
        with open(os.path.join(ROOT, "frontier_bfs_csr_amd", "csrc", fn), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed PMC summary, if it
    was taken on the current kernel source for this workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload, {}).get(kernel)
    if not e or e.get("kernel_source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def component_edges(deg, dist, symmetric=True):
    """Edges of the part of the graph the search reached: half the reached
    degrees of an undirected graph; the reached vertices' out-edges of a
    directed one."""
    total = int(deg[dist >= 0].sum())
    return total // 2 if symmetric else total


def host_cpu():
    """The host's CPU model name and core counts (for the CPU baseline)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 0
    return {"cpu_model": model, "nproc": usable, "cpu_count": os.cpu_count() or 0}


def copy_calibration(nbytes):
    """A plain device copy of known size, for scaling PMC byte counters."""
    import torch
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 5}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default="c5", choices=sorted(WORKLOAD_DESC))
    ap.add_argument("--direction", type=int, default=0, help="0 auto, 1 push, 2 pull")
    ap.add_argument("--advance", type=int, default=0, help="0 auto, 1 binned, 2 edge-balanced")
    ap.add_argument("--loop", type=int, default=0, help="0 device-resident, 1 host-driven")
    ap.add_argument("--alpha", type=int, default=40, help="direction switch: pull when alpha*deg(F) > deg(U)")
    ap.add_argument("--beta", type=int, default=96, help="direction switch: push when beta*|F| < n, shrinking")
    ap.add_argument("--claim", type=int, default=0, help="0 visited-bitmap atomicOr, 1 atomicMin on dist")
    ap.add_argument("--compaction", type=int, default=0,
                    help="0 direction-optimising path; top-down only: 1 atomic append, 2 sentinel-padded, "
                         "3 padded + flag/scan/scatter filter, 4 flag/scan/scatter over all vertices")
    ap.add_argument("--no-parent", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="budget of the CPU-oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "this BFS build has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch

    import frontier_bfs_csr_amd as fb
    import graphgen as gg
    from frontier_bfs_csr_amd import bytemodel

    t0 = time.time()
    if args.workload in DIRECTED:
        scale, seed = DIRECTED[args.workload]
        g = gg.rmat_directed(scale, 16, seed=seed, nsrc=64)
    else:
        g = gg.WORKLOADS[args.workload]()
    in_csr = None if g.symmetric else bytemodel.transpose(g.row_ptr, g.col_idx)
    print(f"[bench] {args.workload}: n={g.n} m={g.m} sources={len(g.sources)} "
          f"generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    deg = g.degrees()
    dev = torch.device("cuda:0")
    rp = torch.from_numpy(g.row_ptr).to(dev)
    ci = torch.from_numpy(g.col_idx).to(dev)
    stream = torch.cuda.current_stream()
    bg = fb.BfsGraph(rp, ci)
    bg.set_policy(args.direction, args.advance, args.loop)
    bg.set_switch(args.alpha, args.beta)
    bg.set_primitives(args.claim, args.compaction)
    dist = torch.empty(g.n, dtype=torch.int32, device=dev)
    parent = None if args.no_parent else torch.empty(g.n, dtype=torch.int32, device=dev)
    sizes = torch.empty(g.n, dtype=torch.int32, device=dev)
    sources = [int(s) for s in g.sources]

    def step(i):
        return bg.run(sources[i % len(sources)], dist, parent, sizes, stream)

    # timed pass: the timing hook off, so only the searches are in the wall time
    bg.set_timing(False)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    per_step = []
    t_start = time.perf_counter()
    for i in range(args.steps):
        ts = time.perf_counter()
        L = step(i)
        per_step.append((sources[i % len(sources)], L, time.perf_counter() - ts))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    print(f"[bench] timed {args.steps} searches in {wall * 1e3:.2f} ms", file=sys.stderr, flush=True)

    # kernel pass: the same searches again, every level launch timed by HIP
    # events on the search stream
    bg.set_timing(True)
    init_ms, level_ms, launches = 0.0, 0.0, 0
    kt = {"td": [0.0, 0], "bu": [0.0, 0]}
    for i in range(args.steps):
        step(i)
        a, b, c = bg.timing()
        init_ms, level_ms, launches = init_ms + a, level_ms + b, launches + c
        for kind, (ms, nl) in bg.kernel_timing().items():
            kt[kind][0] += ms
            kt[kind][1] += nl
    bg.set_timing(False)

    # per distinct source: result, directions, byte model, component edges
    model = {}
    gpu_dist = {}
    for s in sorted({p[0] for p in per_step}):
        L = bg.run(s, dist, parent, sizes, stream)
        Ls, dirs, _ = bg.stats()
        flags = bg.level_flags()
        d = dist.cpu().numpy()
        init_b, lvl_b, fin_b = bytemodel.alg_bytes(g.row_ptr, g.col_idx, d, dirs, with_parent=parent is not None,
                                                   flags=flags, in_csr=in_csr)
        # the init kernel and the finishing pass (dist written in vertex order
        # at the end, on large graphs) are counted together, as they are timed
        model[s] = {"L": L, "init": init_b + fin_b, "levels": int(lvl_b.sum()),
                    "medges": component_edges(deg, d, g.symmetric),
                    "td": int(lvl_b[dirs == 0].sum()), "bu": int(lvl_b[dirs == 1].sum()),
                    "dirs": "".join("TB"[x] for x in dirs)}
        gpu_dist[s] = d if len(gpu_dist) < 8 else None

    edges = sum(model[s]["medges"] for s, *_ in per_step)
    value = edges / wall / 1e9
    bytes_levels = sum(model[s]["levels"] for s, *_ in per_step)
    bytes_init = sum(model[s]["init"] for s, *_ in per_step)
    kinds = {}
    # a small graph under the default policy runs as one launch of the
    # one-workgroup kernel, timed as the top-down kind
    one = (g.n <= fb.SMALL_GRAPH_N and (args.direction, args.advance, args.loop) == (0, 0, 0)
           and not args.compaction)
    for kind in ("td", "bu"):
        ms, nl = kt[kind]
        b = sum(model[s][kind] for s, *_ in per_step)
        kinds[kind] = {"kernel": "bfs_one_kernel" if (one and kind == "td") else KERNEL_NAMES[kind],
                       "ms": ms, "launches": nl, "bytes": b,
                       "achieved": b / (ms * 1e-3) / 1e9 if ms > 0 else 0.0}
    dom = max(kinds, key=lambda k: kinds[k]["ms"])
    kd = kinds[dom]
    traffic = measured_traffic(args.workload, kd["kernel"])
    if args.compaction:
        # the alternative primitives run a host-driven loop: its time is the
        # whole loop's (every kernel and the per-level read), not one kernel's
        kd["kernel"] = "variant level loop (host-driven, all kernels)"
        traffic = None
    step_gteps = [model[s]["medges"] / t / 1e9 for s, L, t in per_step]

    cpu = None
    parity_sample = None
    if not args.no_cpu_baseline:
        import oracle   # the CPU baseline leg: the oracle, timed as it stands
        spent, cedges, cnt, ok = 0.0, 0, 0, True
        for s in sources:
            ts = time.perf_counter()
            ref = oracle.bfs(g.row_ptr, g.col_idx, s)
            spent += time.perf_counter() - ts
            cedges += component_edges(deg, ref[0], g.symmetric)
            cnt += 1
            if s in gpu_dist and gpu_dist[s] is not None:
                ok = ok and bool((gpu_dist[s] == ref[0]).all())
            if spent >= args.cpu_seconds:
                break
        host = host_cpu()
        cpu = {"value": cedges / spent / 1e9, "unit": "GTEPS", "cores": 1, "kind": "oracle",
               "sample": f"{cnt} of the {len(sources)} sources of the same graph, serial FIFO BFS "
                         f"(gcc -O2) on one core of {host['nproc']} ({host['cpu_model']}), {spent:.1f} s",
               "ms_per_bfs": spent / cnt * 1e3, "host_cpu_model": host["cpu_model"],
               "host_nproc": host["nproc"]}
        parity_sample = {"sources_compared": sum(1 for s in sources[:cnt] if gpu_dist.get(s) is not None),
                         "dist_equal": ok}

    s0 = per_step[0][0]
    out = {
        "metric": "GTEPS on one MI355X (R-MAT scale 24) + % HBM roofline; ms per BFS",
        "value": round(value, 4),
        "unit": "GTEPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_DESC[args.workload], "n": g.n, "m_csr_entries": g.m,
                   "sources": len(sources), "parent_out": parent is not None,
                   "policy": {"direction": args.direction, "advance": args.advance, "loop": args.loop,
                              "alpha": args.alpha, "beta": args.beta, "claim": args.claim,
                              "compaction": args.compaction}},
        "roofline": {"bound": "hbm", "achieved": round(kd["achieved"], 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(kd["achieved"] / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": kd["kernel"],
                     "bytes_per_launch": round(kd["bytes"] / max(kd["launches"], 1)),
                     "avg_launch_us": round(kd["ms"] / max(kd["launches"], 1) * 1e3, 3),
                     "launches": kd["launches"]},
        "cpu_baseline": cpu,
        "detail": {
            "ms_per_bfs_median": round(float(np.median([p[2] for p in per_step])) * 1e3, 4),
            "gteps_hmean": round(len(step_gteps) / sum(1.0 / x for x in step_gteps), 4),
            "init_finish_us_avg": round(init_ms / args.steps * 1e3, 2),
            "level_kernels_ms_avg": round(level_ms / args.steps, 4),
            "level_launches_avg": round(launches / args.steps, 2),
            "kernels": {v["kernel"]: {"ms_avg": round(v["ms"] / args.steps, 4),
                                      "launches": v["launches"],
                                      "alg_GB_per_s": round(v["achieved"], 1)}
                        for v in kinds.values()},
            "alg_GB_per_bfs": round((bytes_levels + bytes_init) / args.steps / 1e9, 4),
            "whole_bfs_alg_GBps": round((bytes_levels + bytes_init) / wall / 1e9, 1),
            "levels_first_source": model[s0]["L"],
            "directions_first_source": model[s0]["dirs"],
            "parity_sample": parity_sample,
        },
    }
    bg.close()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
