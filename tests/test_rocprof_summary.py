"""The profiling harness's arithmetic on small synthetic rocprofv3 databases
(CPU): kernel-trace averages, HBM bytes from FETCH_SIZE / WRITE_SIZE scaled by
a copy of known size, and the engine clock and MFMA busy fraction."""
from __future__ import annotations

import io
import os
import sqlite3
import tempfile

import pytest

from sharded_fc_layer_amd import rocprof_summary as R

GEMM = "void fcs::(anonymous namespace)::gemm_w4k64_kernel<false, true, false>(fcs::GemmArgs)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::bfloat16_copy_kernel_cuda>(int)"


def _counter_db(path, rows):
    """rows: (kernel_name, counter_name, value, dispatch_id, duration_ns)"""
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real, "
                "dispatch_id integer, duration integer)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_kernel_trace_averages():
    with tempfile.TemporaryDirectory() as d:
        db = os.path.join(d, "t.db")
        con = sqlite3.connect(db)
        con.execute("create table kernels (id integer, name text, duration integer, grid_x integer, grid_y integer, "
                    "grid_z integer, start integer)")
        con.executemany("insert into kernels values (?, ?, ?, ?, ?, ?, ?)",
                        [(1, GEMM, 100_000, 65536, 1, 1, 0), (2, GEMM, 300_000, 65536, 1, 1, 1),
                         (3, COPY, 50_000, 1024, 1, 1, 2)])
        con.commit()
        con.close()
        out = io.StringIO()
        R.summarize(db, False, out)
    line = next(l for l in out.getvalue().splitlines() if l.startswith("gemm_w4k64_kernel"))
    f = line.split()
    # calls 2, avg 200 us, min 100, max 300, total 0.4 ms, 400 of 450 us = 88.89 %
    assert f[-6:] == ["2", "200.00", "100.00", "300.00", "0.400", "88.89"]


def test_traffic_scales_each_counter_by_the_copy():
    gib = 1 << 30
    # the copy reads and writes 1 GiB; FETCH_SIZE reads half of it (KiB), WRITE_SIZE all of it
    rows_f = [(COPY, "FETCH_SIZE", gib / 2 / 1024, 1, 1), (GEMM, "FETCH_SIZE", 100_000.0, 2, 1),
              (GEMM, "FETCH_SIZE", 300_000.0, 3, 1)]
    rows_w = [(COPY, "WRITE_SIZE", gib / 1024, 1, 1), (GEMM, "WRITE_SIZE", 50_000.0, 2, 1),
              (GEMM, "WRITE_SIZE", 50_000.0, 3, 1)]
    with tempfile.TemporaryDirectory() as d:
        f, w = os.path.join(d, "f.db"), os.path.join(d, "w.db")
        _counter_db(f, rows_f)
        _counter_db(w, rows_w)
        res = R.traffic(f, w, "elementwise", gib, io.StringIO())
    assert res["fetch_scale"] == pytest.approx(2.0) and res["write_scale"] == pytest.approx(1.0)
    k = res["kernels"]["gemm_w4k64_kernel<false, true, false>"]
    assert k["launches"] == 2
    assert k["fetch_bytes_per_launch"] == pytest.approx(200_000 * 1024 * 2.0)
    assert k["write_bytes_per_launch"] == pytest.approx(50_000 * 1024 * 1.0)
    assert k["hbm_bytes_per_launch"] == pytest.approx(k["fetch_bytes_per_launch"] + k["write_bytes_per_launch"])


def test_mfma_busy_and_clock():
    dur = 100_000  # ns
    clock = 2.0  # GHz -> 200 000 engine cycles
    cycles = dur * clock
    busy = 0.75
    rows = []
    for disp in (1, 2):
        # GRBM_GUI_ACTIVE comes summed over the 8 XCDs; the MFMA counter over 1024 SIMDs
        rows.append((GEMM, "GRBM_GUI_ACTIVE", cycles * R.XCDS, disp, dur))
        rows.append((GEMM, "SQ_VALU_MFMA_BUSY_CYCLES", busy * R.SIMDS * cycles, disp, dur))
        rows.append((GEMM, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 2 * 8192 * 2048 * 2048 / 512, disp, dur))
    rows.append((COPY, "GRBM_GUI_ACTIVE", 8 * 1000.0, 3, 500))
    rows.append((COPY, "SQ_VALU_MFMA_BUSY_CYCLES", 0.0, 3, 500))
    # the MFMA-only probe: one 2 ms launch (counted) and a 4 us clock sample (left out)
    PROBE = "void fcs::(anonymous namespace)::mfma_probe_kernel(long, unsigned long long*)"
    for disp, d, busy_p in ((4, 2_000_000, 0.96), (5, 4_000, 0.1)):
        cyc = d * 2.3
        rows.append((PROBE, "GRBM_GUI_ACTIVE", cyc * R.XCDS, disp, d))
        rows.append((PROBE, "SQ_VALU_MFMA_BUSY_CYCLES", busy_p * R.SIMDS * cyc, disp, d))
    with tempfile.TemporaryDirectory() as d:
        db = os.path.join(d, "m.db")
        _counter_db(db, rows)
        res = R.mfma_util(db, io.StringIO())
    # the copy has no MFMA work; of the probe only the long launch counts
    assert set(res) == {"gemm_w4k64_kernel<false, true, false>", "mfma_probe_kernel"}
    p = res["mfma_probe_kernel"]
    assert p["dispatches"] == 1 and p["clock_ghz"] == pytest.approx(2.3) and p["mfma_busy"] == pytest.approx(0.96)
    r = res["gemm_w4k64_kernel<false, true, false>"]
    assert r["dispatches"] == 2 and r["avg_us"] == pytest.approx(100.0)
    assert r["clock_ghz"] == pytest.approx(clock) and r["mfma_busy"] == pytest.approx(busy)
    assert r["implied_tflops"] == pytest.approx(busy * 2500.0 * clock / 2.4)
    assert r["hw_flops_per_launch"] == pytest.approx(2 * 8192 * 2048 * 2048)


def test_tail_split_plans_count_only_their_main_launch():
    # bwd_weight of M=8192 tokens, K=26624, N=4096: output K x N, reduction M;
    # a tail plan whose unsplit part is the first 24576 output rows
    rec = {"op": "bwd_weight", "M": 8192, "K": 26624, "N": 4096, "kernel": "k_main", "tail": "m24576"}
    assert R.main_launch_extent(rec) == (24576, 4096, 8192)
    whole = dict(rec, kernel="k_whole")
    del whole["tail"]
    assert R.main_launch_extent(whole) == (26624, 4096, 8192)
    fl = R.analytical_flops({"plans": [rec, whole]})
    assert fl["k_main"] == 2 * 24576 * 4096 * 8192 and fl["k_whole"] == 2 * 26624 * 4096 * 8192
    by = R.algorithmic_bytes({"plans": [rec]})
    assert by["k_main"] == 2 * (24576 * 8192 + 8192 * 4096 + 24576 * 4096)
    # column tails, and the other products' extents
    assert R.main_launch_extent({"op": "fwd", "M": 8, "K": 16, "N": 32, "tail": "n24"}) == (8, 24, 16)
    assert R.main_launch_extent({"op": "bwd_data", "M": 8, "K": 16, "N": 32}) == (8, 16, 32)
    with pytest.raises(ValueError):
        R.main_launch_extent({"op": "fwd", "M": 8, "K": 16, "N": 32, "tail": "x3"})


def test_traffic_per_launch_grid():
    # two GEMM shapes share one kernel: grids of 1024 and 4096 threads
    gib = 1 << 30

    def db(path, counter, rows):
        con = sqlite3.connect(path)
        con.execute("create table counters_collection (kernel_name text, counter_name text, value real, "
                    "dispatch_id integer, duration integer, grid_size_x integer)")
        con.executemany("insert into counters_collection values (?, ?, ?, ?, ?, ?)", rows)
        con.commit()
        con.close()

    with tempfile.TemporaryDirectory() as d:
        f, w = os.path.join(d, "f.db"), os.path.join(d, "w.db")
        db(f, "FETCH_SIZE", [(COPY, "FETCH_SIZE", gib / 1024, 1, 1, 64), (GEMM, "FETCH_SIZE", 100.0, 2, 1, 1024),
                             (GEMM, "FETCH_SIZE", 300.0, 3, 1, 4096), (GEMM, "FETCH_SIZE", 500.0, 4, 1, 4096)])
        db(w, "WRITE_SIZE", [(COPY, "WRITE_SIZE", gib / 1024, 1, 1, 64), (GEMM, "WRITE_SIZE", 10.0, 2, 1, 1024),
                             (GEMM, "WRITE_SIZE", 20.0, 3, 1, 4096), (GEMM, "WRITE_SIZE", 20.0, 4, 1, 4096)])
        res = R.traffic(f, w, "elementwise", gib, io.StringIO())
    k = res["kernels"]["gemm_w4k64_kernel<false, true, false>"]
    assert k["hbm_bytes_per_launch"] == pytest.approx((300 + 50 / 3) * 1024)
    assert k["by_grid"]["1024"] == {"launches": 1, "hbm_bytes_per_launch": pytest.approx(110 * 1024)}
    assert k["by_grid"]["4096"]["launches"] == 2
    assert k["by_grid"]["4096"]["hbm_bytes_per_launch"] == pytest.approx(420 * 1024)


def test_report_refuses_runs_of_another_workload():
    """A report names its files by workload: runs of another workload's bench
    line (a wrong --workload-number) are refused before anything is written."""
    import json
    with tempfile.TemporaryDirectory() as d:
        line = {"metric": "m", "value": 1.0, "config": {"workload": "mlp_up_shard_h12288_2x2x2"}}
        with open(os.path.join(d, "trace_w2.log"), "w") as f:
            f.write("noise\n" + json.dumps(line) + "\n")
        with pytest.raises(ValueError, match="timed workload 'mlp_up_shard_h12288_2x2x2'"):
            R.report(d, "gpt_block_h2048_t8192", 2, d, "0" * 16)
        assert sorted(os.listdir(d)) == ["trace_w2.log"]


def test_forced_plan_runs_add_only_what_the_tuned_runs_lack():
    """Counter runs with another plan forced fill in the kernels (and launch
    grids) the tuned plans' runs did not launch; what those runs measured stays."""
    main = {"kernels": {"k1": {"launches": 2, "hbm_bytes_per_launch": 10.0,
                               "by_grid": {"64": {"launches": 2, "hbm_bytes_per_launch": 10.0}}}}}
    alt = {"kernels": {"k1": {"launches": 3, "hbm_bytes_per_launch": 99.0,
                              "by_grid": {"64": {"launches": 1, "hbm_bytes_per_launch": 98.0},
                                          "128": {"launches": 2, "hbm_bytes_per_launch": 30.0}}},
                       "k2": {"launches": 1, "hbm_bytes_per_launch": 7.0,
                              "by_grid": {"32": {"launches": 1, "hbm_bytes_per_launch": 7.0}}}}}
    R.merge_traffic(main, alt, "p576")
    k1, k2 = main["kernels"]["k1"], main["kernels"]["k2"]
    assert k1["hbm_bytes_per_launch"] == 10.0 and k1["by_grid"]["64"]["hbm_bytes_per_launch"] == 10.0
    assert k1["by_grid"]["128"] == {"launches": 2, "hbm_bytes_per_launch": 30.0, "run": "p576"}
    assert "run" not in k1 and "run" not in k1["by_grid"]["64"]
    assert k2["run"] == "p576" and k2["hbm_bytes_per_launch"] == 7.0
