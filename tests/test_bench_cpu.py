"""bench.py's host side (no GPU): it refuses more than one GPU, the device-code
hash ignores comments and whitespace but not code (and covers the kernel
body include), and committed counter figures are used only while the hash
matches."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def test_source_hash_ignores_comments_but_not_code(tmp_path):
    a = tmp_path / "k.hip"
    a.write_text("int f(int x) { return x + 1; }  // add one\n")
    h0 = bench.kernel_source_hash([str(a)])
    a.write_text("/* a\\n block */ int f(int x)  {\n  return x + 1;   }\n// another\n")
    assert bench.kernel_source_hash([str(a)]) == h0
    a.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_source_hash([str(a)]) != h0


def test_device_sources_include_the_kernel_body():
    names = {os.path.basename(f) for f in bench.KERNEL_SOURCES}
    assert "gemm_w4_ring_body.inc" in names and "gemm_w4_ring_impl.h" in names
    assert "fcshard_api.hip" not in names  # the host-only C-ABI layer


def test_traffic_figures_only_for_the_current_device_code(tmp_path, monkeypatch):
    rec = {"source_hash": bench.kernel_source_hash(),
           "workloads": {"w": {"kernels": {"k": {"hbm_bytes_per_launch": 123.0}}}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("k", "w") == 123.0
    assert bench.measured_traffic("other", "w") is None
    assert bench.measured_traffic("k", "other") is None
    rec["source_hash"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert bench.measured_traffic("k", "w") is None


def test_traffic_weighs_this_runs_calls_by_launch_grid(tmp_path, monkeypatch):
    rec = {"source_hash": bench.kernel_source_hash(),
           "workloads": {"w": {"kernels": {"k": {"hbm_bytes_per_launch": 300.0,
                                                 "by_grid": {"1024": {"launches": 1, "hbm_bytes_per_launch": 100.0},
                                                             "4096": {"launches": 2,
                                                                      "hbm_bytes_per_launch": 400.0}}}}}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("k", "w", [1024, 1024, 4096]) == 200.0
    assert bench.measured_traffic("k", "w", [4096]) == 400.0
    # a grid the counter runs did not see, or no grids: the kernel's overall mean
    assert bench.measured_traffic("k", "w", [1024, 2048]) == 300.0
    assert bench.measured_traffic("k", "w", [None]) == 300.0
    assert bench.measured_traffic("k", "w") == 300.0
