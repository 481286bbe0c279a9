"""bench.py's host logic, on the CPU: the one-GPU guard, the gate that reports
measured HBM traffic only for the kernel source it was taken on, and the edge
count behind GTEPS."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    for argv, env in ((["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                           capture_output=True, text=True, timeout=120,
                           env={**os.environ, **env})
        assert r.returncode == 2, (argv, env, r.returncode)
        assert "one GPU only" in r.stderr
        assert r.stdout == ""   # no JSON line


def test_traffic_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("c5", "bfs_bu_kernel") is None          # no file
    f.write_text(json.dumps({"c5": {"bfs_bu_kernel": {"bytes_per_launch": 123, "kernel_source_hash": h}}}))
    assert bench.measured_traffic("c5", "bfs_bu_kernel") == 123
    assert bench.measured_traffic("c5", "bfs_td_kernel") is None          # another kernel
    assert bench.measured_traffic("c3", "bfs_bu_kernel") is None          # another workload
    f.write_text(json.dumps({"c5": {"bfs_bu_kernel": {"bytes_per_launch": 123,
                                                      "kernel_source_hash": "0" * 16}}}))
    assert bench.measured_traffic("c5", "bfs_bu_kernel") is None          # kernel changed since
    f.write_text("not json")
    assert bench.measured_traffic("c5", "bfs_bu_kernel") is None


def test_component_edges():
    # path 0-1-2 plus an isolated vertex 3, searched from 0: two undirected edges
    deg = np.array([1, 2, 1, 0])
    dist = np.array([0, 1, 2, -1])
    assert bench.component_edges(deg, dist, symmetric=True) == 2
    # directed: the reached vertices' out-edges, each counted once
    assert bench.component_edges(np.array([2, 0, 1]), np.array([0, 1, -1]), symmetric=False) == 2
    assert bench.component_edges(deg, np.full(4, -1), symmetric=True) == 0


def test_host_cpu_fields():
    h = bench.host_cpu()
    assert isinstance(h["cpu_model"], str) and h["cpu_model"]
    assert h["nproc"] >= 1 and h["cpu_count"] >= h["nproc"]
