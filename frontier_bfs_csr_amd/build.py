"""Builds libfrontier_bfs.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfrontier_bfs.so")
# the same library built with per-vertex enqueue counting (validator V5 of the
# tests); never the one the product path loads
LIB_V5 = os.path.join(PKG, "libfrontier_bfs_v5.so")
SOURCES = ["bfs_device.hip", "bfs_small.hip", "bfs_walk.hip", "bfs_variants.hip", "bfs_sssp.hip", "bfs_api.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off (none of this code needs them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # atomics on one address with per-lane values (the small-frontier
    # staging's LDS counter, reached from divergent code) are combined per
    # wavefront by a DPP scan instead of a loop over the active lanes
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=DPP",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def _build_one(out: str, extra, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """The library, then its enqueue-counting debug build (both in-tree)."""
    _build_one(LIB, [], verbose)
    _build_one(LIB_V5, ["-DFBFS_COUNT_ENQUEUES"], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
