"""Summarize rocprofv3 output of this library's kernels as short text.

Reads a rocprofv3 rocpd database (<name>_results.db) and prints, per kernel
(optionally per kernel and grid size), the dispatch count and the average,
minimum, maximum and total duration; for counter runs (--pmc) it prints the
per-dispatch averages of each counter. With --traffic it combines a
FETCH_SIZE run and a WRITE_SIZE run into HBM bytes per launch of each kernel,
scaled by what the same counters read for a plain copy of known size. With
--mfma it turns a run with SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE into
each kernel's engine clock and MFMA busy fraction, and, with
SQ_INSTS_VALU_MFMA_MOPS_BF16 (bf16 MFMA operations / 512), the flops the
hardware executed per launch.
With --report it writes the three summaries of one workload (kernel trace,
HBM traffic, MFMA utilisation) into a directory as short text files, each
with the commands that produced its inputs, and records the traffic figures
in a JSON file keyed by workload and by a hash of the device sources.
Usage:

  python -m sharded_fc_layer_amd.rocprof_summary RESULTS.db [--by-grid] [--pmc]
  python -m sharded_fc_layer_amd.rocprof_summary --traffic FETCH.db WRITE.db \
      --copy-kernel REGEX --copy-bytes N [--json OUT --workload NAME --source-hash H]
  python -m sharded_fc_layer_amd.rocprof_summary --mfma MFMA.db
  python -m sharded_fc_layer_amd.rocprof_summary --report DIR --workload NAME --prof-dir P \
      --source-hash H --json profiles/traffic.json
"""
from __future__ import annotations

import argparse
import re
import sqlite3
import sys
from collections import defaultdict


def short(name: str) -> str:
    name = re.sub(r"^void ", "", name)
    name = name.replace("fcs::(anonymous namespace)::", "")
    return re.sub(r"\(.*\)$", "", name)


def kernel_rows(db: str):
    con = sqlite3.connect(db)
    cur = con.cursor()
    rows = cur.execute("select name, duration, grid_x, grid_y, grid_z, id from kernels order by start").fetchall()
    return con, rows


def summarize(db: str, by_grid: bool, out=sys.stdout):
    con, rows = kernel_rows(db)
    agg = defaultdict(list)
    for name, dur, gx, gy, gz, _ in rows:
        key = (short(name), gx) if by_grid else (short(name), None)
        agg[key].append(dur / 1000.0)  # ns -> us
    total = sum(sum(v) for v in agg.values())
    out.write(f"{'kernel':<66} {'grid':>8} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} "
              f"{'total_ms':>10} {'pct':>6}\n")
    for (k, g), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        out.write(f"{k:<66} {str(g or '-'):>8} {len(v):>6} {sum(v) / len(v):>10.2f} {min(v):>10.2f} "
                  f"{max(v):>10.2f} {sum(v) / 1000:>10.3f} {100 * sum(v) / total:>6.2f}\n")


def summarize_pmc(db: str, out=sys.stdout):
    con = sqlite3.connect(db)
    cur = con.cursor()
    cols = [d[0] for d in cur.execute("select * from counters_collection limit 1").description]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    q = f"select {name_col}, counter_name, value, dispatch_id from counters_collection"
    agg = defaultdict(lambda: defaultdict(dict))
    for kname, cname, val, disp in cur.execute(q):
        d = agg[short(kname)][cname]
        d[disp] = d.get(disp, 0.0) + float(val)
    out.write(f"{'kernel':<66} {'counter':<22} {'dispatches':>10} {'avg_per_dispatch':>18}\n")
    for k, cs in sorted(agg.items()):
        for c, per in sorted(cs.items()):
            vals = list(per.values())
            out.write(f"{k:<66} {c:<22} {len(vals):>10} {sum(vals) / len(vals):>18.1f}\n")


def counter_per_dispatch(db: str, counter: str, by_grid: bool = False):
    """{kernel: [value per dispatch]} for one counter (summed over dimensions);
    with by_grid, {kernel: {grid size in threads: [value per dispatch]}}."""
    con = sqlite3.connect(db)
    cur = con.cursor()
    cols = [d[0] for d in cur.execute("select * from counters_collection limit 1").description]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    grid_col = "grid_size_x" if "grid_size_x" in cols else "0"
    per = defaultdict(lambda: defaultdict(float))
    grid = {}
    for kname, cname, val, disp, gx in cur.execute(
            f"select {name_col}, counter_name, value, dispatch_id, {grid_col} from counters_collection"):
        if cname == counter:
            per[short(kname)][disp] += float(val)
            grid[(short(kname), disp)] = int(gx)
    if not by_grid:
        return {k: list(v.values()) for k, v in per.items()}
    out = defaultdict(lambda: defaultdict(list))
    for k, v in per.items():
        for disp, val in v.items():
            out[k][grid[(k, disp)]].append(val)
    return {k: dict(v) for k, v in out.items()}


# MI355X: 8 XCDs (one GRBM each), 256 CUs x 4 SIMDs; dense bf16 peak 2.5 PFLOP/s at 2.4 GHz
XCDS, SIMDS, PEAK_TFLOPS, PEAK_GHZ = 8, 1024, 2500.0, 2.4
PROBE_MIN_NS = 1_000_000  # probe launches shorter than 1 ms are clock samples


def mfma_util(db: str, out=sys.stdout):
    """Per kernel: engine clock (GRBM_GUI_ACTIVE, summed over the XCDs, per XCD,
    over the dispatch duration), MFMA busy fraction (SQ_VALU_MFMA_BUSY_CYCLES
    over SIMDs x engine cycles), and the bf16 rate those two imply."""
    con = sqlite3.connect(db)
    cur = con.cursor()
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))
    dur = defaultdict(dict)
    for kname, cname, val, disp, d in cur.execute(
            "select kernel_name, counter_name, value, dispatch_id, duration from counters_collection"):
        k = short(kname)
        per[k][disp][cname] += float(val)
        dur[k][disp] = float(d)
    res = {}
    out.write(f"{'kernel':<66} {'dispatches':>10} {'avg_us':>9} {'clock_GHz':>9} {'mfma_busy':>9} "
              f"{'implied_TFLOP/s':>15} {'hw_GFLOP/launch':>15}\n")
    for k, disps in sorted(per.items()):
        rows = [(c, dur[k][d]) for d, c in disps.items()
                if c.get("GRBM_GUI_ACTIVE", 0) > 0 and "SQ_VALU_MFMA_BUSY_CYCLES" in c and dur[k][d] > 0]
        if k.startswith("mfma_probe_kernel"):
            # the short launches between a step's GEMMs are clock samples, too
            # short for the counters' clock; only the long probe launches count
            rows = [(c, d) for c, d in rows if d >= PROBE_MIN_NS]
        # kernels without MFMA work (copies, the split-K sum) are short next to
        # the counters' sampling, so their clock would not mean anything
        if not rows or not any(c["SQ_VALU_MFMA_BUSY_CYCLES"] > 0 for c, _ in rows):
            continue
        cyc = [c["GRBM_GUI_ACTIVE"] / XCDS for c, _ in rows]
        clock = sum(cy / d for cy, (_, d) in zip(cyc, rows)) / len(rows)
        busy = sum(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * cy) for cy, (c, _) in zip(cyc, rows)) / len(rows)
        avg_us = sum(d for _, d in rows) / len(rows) / 1e3
        implied = busy * PEAK_TFLOPS * clock / PEAK_GHZ
        mops = [c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16") for c, _ in rows]
        hw = sum(mops) * 512 / len(mops) if all(m is not None for m in mops) else None
        res[k] = {"dispatches": len(rows), "avg_us": avg_us, "clock_ghz": clock, "mfma_busy": busy,
                  "implied_tflops": implied, "hw_flops_per_launch": hw}
        hw_s = f"{hw / 1e9:>15.3f}" if hw is not None else f"{'-':>15}"
        out.write(f"{k:<66} {len(rows):>10} {avg_us:>9.1f} {clock:>9.3f} {busy:>9.3f} {implied:>15.1f} {hw_s}\n")
    return res


def traffic(fetch_db: str, write_db: str, copy_kernel: str, copy_bytes: int, out=sys.stdout):
    """HBM bytes per launch, each counter scaled by its reading on the copy."""
    fetch = counter_per_dispatch(fetch_db, "FETCH_SIZE")
    write = counter_per_dispatch(write_db, "WRITE_SIZE")
    pat = re.compile(copy_kernel)
    cf = [v for k, vs in fetch.items() if pat.search(k) for v in vs]
    cw = [v for k, vs in write.items() if pat.search(k) for v in vs]
    if not cf or not cw:
        raise SystemExit(f"copy kernel {copy_kernel!r} not found in the counter runs")
    # counters are in KiB per dispatch; the copy reads and writes copy_bytes
    f_scale = copy_bytes / (1024.0 * max(cf))
    w_scale = copy_bytes / (1024.0 * max(cw))
    res = {"copy_kernel": copy_kernel, "copy_bytes": copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale,
           "kernels": {}}
    out.write(f"copy calibration: FETCH_SIZE {max(cf):.0f} KiB, WRITE_SIZE {max(cw):.0f} KiB for "
              f"{copy_bytes / 2**30:.3f} GiB each -> scale fetch {f_scale:.4f}, write {w_scale:.4f}\n")
    out.write(f"{'kernel':<66} {'launches':>8} {'fetch_MB':>10} {'write_MB':>10} {'hbm_MB/launch':>14}\n")
    fetch_g = counter_per_dispatch(fetch_db, "FETCH_SIZE", by_grid=True)
    write_g = counter_per_dispatch(write_db, "WRITE_SIZE", by_grid=True)
    for k in sorted(set(fetch) & set(write)):
        if pat.search(k):
            continue
        f = sum(fetch[k]) / len(fetch[k]) * 1024 * f_scale
        w = sum(write[k]) / len(write[k]) * 1024 * w_scale
        rec = {"launches": len(fetch[k]), "fetch_bytes_per_launch": f, "write_bytes_per_launch": w,
               "hbm_bytes_per_launch": f + w, "by_grid": {}}
        # per launch grid (threads): a kernel that several GEMMs share
        # gets a figure per GEMM shape
        for g in sorted(set(fetch_g.get(k, {})) & set(write_g.get(k, {}))):
            fv, wv = fetch_g[k][g], write_g[k][g]
            fg = sum(fv) / len(fv) * 1024 * f_scale
            wg = sum(wv) / len(wv) * 1024 * w_scale
            rec["by_grid"][str(g)] = {"launches": len(fv), "hbm_bytes_per_launch": fg + wg}
        res["kernels"][k] = rec
        out.write(f"{k:<66} {len(fetch[k]):>8} {f / 1e6:>10.1f} {w / 1e6:>10.1f} {(f + w) / 1e6:>14.1f}\n")
    return res


def merge_traffic(main: dict, other: dict, label: str) -> dict:
    """Adds to `main` (traffic()'s result) what `other` measured and it did
    not: kernels it lacks, and launch grids missing from a kernel it has.
    A record taken from `other` gets "run": label. Each run's figures stay
    scaled by that run's own copy calibration."""
    for k, rec in other["kernels"].items():
        mine = main["kernels"].get(k)
        if mine is None:
            main["kernels"][k] = dict(rec, run=label)
            continue
        for g, grec in rec.get("by_grid", {}).items():
            if g not in mine.setdefault("by_grid", {}):
                mine["by_grid"][g] = dict(grec, run=label)
    return main


def _bench_line(path: str):
    """The JSON line bench.py printed in a run's log (None if there is none)."""
    import json
    try:
        with open(path) as f:
            for line in f:
                line = line.strip()
                if line.startswith("{") and '"metric"' in line:
                    return json.loads(line)
    except OSError:
        return None
    return None


def main_launch_extent(r: dict):
    """(output rows, output cols, reduction) of the launch that a plan record's
    kernel names: the whole product, or for a tail-split plan ("tail": "m<rows>"
    or "n<cols>") its unsplit part, whose launch is the named kernel (the tail
    runs in another launch)."""
    M, K, N = r["M"], r["K"], r["N"]
    rows, cols, red = {"fwd": (M, N, K), "bwd_data": (M, K, N), "bwd_weight": (K, N, M)}[r["op"]]
    t = r.get("tail")
    if t:
        if t[0] == "m":
            rows = int(t[1:])
        elif t[0] == "n":
            cols = int(t[1:])
        else:
            raise ValueError(f"bad tail field {t!r}")
    return rows, cols, red


def analytical_flops(bench: dict):
    """{kernel: mean 2 M N K per call} from a bench line's per-call plan records
    (of the kernel's own launch: the unsplit part of a tail-split plan)."""
    per = defaultdict(list)
    for r in (bench or {}).get("plans", []):
        rows, cols, red = main_launch_extent(r)
        per[r["kernel"]].append(2 * rows * cols * red)
    return {k: sum(v) / len(v) for k, v in per.items()}


def algorithmic_bytes(bench: dict):
    """{kernel: mean compulsory HBM bytes per call}: both bf16 inputs read once,
    the bf16 output written once (of the kernel's own launch, as above)."""
    per = defaultdict(list)
    for r in (bench or {}).get("plans", []):
        rows, cols, red = main_launch_extent(r)
        per[r["kernel"]].append(2 * (rows * red + red * cols + rows * cols))
    return {k: sum(v) / len(v) for k, v in per.items()}


def report(out_dir: str, workload: str, number: int, prof: str, source_hash: str, json_path: str = None,
           copy_kernel: str = "elementwise", copy_bytes: int = 1 << 30, alt_plans=()):
    """The three summaries of workload `workload` (bench.py --workload
    `number`) from the runs under `prof`, named as the commands in each file's
    header say. `alt_plans`: plan ids of further counter-run pairs made with
    bench.py --force-plan (fetch_w<n>_p<id>, write_w<n>_p<id>); the traffic
    records take from them the kernels and launch grids that the tuned plans'
    runs did not launch (another tuning may pick them)."""
    import io
    import json
    import os
    w, tag = workload, f"w{number}"
    plans = os.path.join(prof, f"plans_{tag}.txt")
    bench_cmd = f"python3 bench.py --workload {number} --plans {plans}"
    runs = {
        "tune": f"{bench_cmd} --no-cpu-baseline --no-extra            # tunes, saves the plans",
        "trace": f"rocprofv3 --kernel-trace --stats -d {prof} -o trace_{tag} -- {bench_cmd} --no-cpu-baseline --no-extra",
        "fetch": f"rocprofv3 --pmc FETCH_SIZE -d {prof} -o fetch_{tag} -- {bench_cmd} --no-cpu-baseline --no-extra "
                 f"--no-clock --copy-calibration --steps 5 --warmup 2",
        "write": f"rocprofv3 --pmc WRITE_SIZE -d {prof} -o write_{tag} -- {bench_cmd} --no-cpu-baseline --no-extra "
                 f"--no-clock --copy-calibration --steps 5 --warmup 2",
        **{f"fetch_p{i}": f"rocprofv3 --pmc FETCH_SIZE -d {prof} -o fetch_{tag}_p{i} -- {bench_cmd} --no-cpu-baseline "
                          f"--no-extra --no-clock --copy-calibration --steps 5 --warmup 2 --force-plan {i}"
           for i in alt_plans},
        **{f"write_p{i}": f"rocprofv3 --pmc WRITE_SIZE -d {prof} -o write_{tag}_p{i} -- {bench_cmd} --no-cpu-baseline "
                          f"--no-extra --no-clock --copy-calibration --steps 5 --warmup 2 --force-plan {i}"
           for i in alt_plans},
        "mfma": f"rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                f"GRBM_GUI_ACTIVE -d {prof} -o mfma_{tag} -- {bench_cmd} --no-cpu-baseline --no-extra "
                f"--steps 5 --warmup 2",
    }
    me = "python3 -m sharded_fc_layer_amd.rocprof_summary"
    trace_bench = _bench_line(os.path.join(prof, f"trace_{tag}.log"))
    mfma_bench = _bench_line(os.path.join(prof, f"mfma_{tag}.log"))
    for run, rec in (("trace", trace_bench), ("mfma", mfma_bench)):
        ran = ((rec or {}).get("config") or {}).get("workload")
        if ran is not None and ran != w:
            raise ValueError(f"the {run} run of --workload {number} timed workload {ran!r}, not {w!r}")
    plan_lines = []
    try:
        with open(plans) as f:
            plan_lines = [l.rstrip("\n") for l in f if l.strip()]
    except OSError:
        pass
    n_calls = len((trace_bench or {}).get("plans", []))

    def header(title, keys, tool):
        h = [f"# {title}, workload {w} ({n_calls} GEMMs per step)", f"# kernel source hash: {source_hash}", "#",
             "# Commands (run from the repository root on one MI355X; TMPDIR=/tmp):"]
        h += [f"#   {runs[k]}" for k in keys]
        h += [f"#   {tool}", "#"]
        return h

    # kernel trace
    buf = io.StringIO()
    summarize(os.path.join(prof, f"trace_{tag}_results.db"), False, buf)
    lines = header("rocprofv3 kernel trace", ["tune", "trace"],
                   f"{me} {os.path.join(prof, f'trace_{tag}_results.db')}")
    lines += ["# The profiled run loads the saved plans, so it contains no tuning launches:",
              "# warm-up and timed steps, steps with per-call HIP events, and the clock pass (a short",
              "# mfma_probe_kernel launch after every GEMM, and one long launch of it).",
              "# The plans (fc_plans_save format: arch op M K N x_order w_order out_dtype plan tuned_ms):"]
    lines += [f"#   {l}" for l in plan_lines] + ["#"]
    lines += buf.getvalue().rstrip("\n").splitlines()
    if trace_bench:
        lines += ["#", f"# bench.py line of the traced run: value {trace_bench['value']} TFLOP/s, ms_per_step "
                       f"{trace_bench['ms_per_step']}, roofline kernel {trace_bench['roofline']['kernel']} at "
                       f"{trace_bench['roofline']['achieved']} TFLOP/s over {trace_bench['roofline']['avg_launch_us']} "
                       f"us per launch (HIP events)"]
    with open(os.path.join(out_dir, f"kernel_trace__{w}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # traffic
    buf = io.StringIO()
    tr = traffic(os.path.join(prof, f"fetch_{tag}_results.db"), os.path.join(prof, f"write_{tag}_results.db"),
                 copy_kernel, copy_bytes, buf)
    alt_bufs = []
    for i in alt_plans:
        b = io.StringIO()
        alt = traffic(os.path.join(prof, f"fetch_{tag}_p{i}_results.db"),
                      os.path.join(prof, f"write_{tag}_p{i}_results.db"), copy_kernel, copy_bytes, b)
        new_k = sorted(k for k in alt["kernels"] if k not in tr["kernels"])
        merge_traffic(tr, alt, f"p{i}")
        alt_bufs.append((i, b.getvalue(), new_k))
    alt_opt = f" --alt-plans {','.join(str(i) for i in alt_plans)}" if alt_plans else ""
    alt_keys = [k for i in alt_plans for k in (f"fetch_p{i}", f"write_p{i}")]
    lines = header("HBM traffic per launch", ["tune", "fetch", "write"] + alt_keys,
                   f"{me} --report profiles --workload {w} --workload-number {number} --prof-dir {prof} "
                   f"--source-hash {source_hash} --json profiles/traffic.json{alt_opt}")
    lines += ["# The copy reference is one torch elementwise kernel (out = in * 1) over 2^29 bf16",
              "# values: it reads and writes exactly 1 GiB. Each counter is scaled by",
              "# (1 GiB / what it read for that copy). FETCH_SIZE counts L2 misses to the data",
              "# fabric (MALL or HBM).", "#"]
    lines += buf.getvalue().rstrip("\n").splitlines()
    for i, text, new_k in alt_bufs:
        lines += ["#", f"# counter runs with plan {i} forced where it applies (bench.py --force-plan {i}); the",
                  "# traffic records take from them the kernels and launch grids the tuned plans did not launch:",
                  f"# {', '.join(new_k) if new_k else 'no new kernel'}"]
        lines += text.rstrip("\n").splitlines()
    alg = algorithmic_bytes(trace_bench)
    lines.append("#")
    for k, rec in sorted(tr["kernels"].items()):
        if k in alg:
            lines.append(f"# {k}: {rec['hbm_bytes_per_launch'] / 1e6:.1f} MB per launch measured vs "
                         f"{alg[k] / 1e6:.1f} MB algorithmic (A + B read once, C written once) = "
                         f"{rec['hbm_bytes_per_launch'] / alg[k]:.2f}x")
    with open(os.path.join(out_dir, f"hbm_traffic__{w}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if json_path:
        rec = {}
        try:
            with open(json_path) as f:
                rec = json.load(f)
        except (OSError, ValueError):
            rec = {}
        if rec.get("source_hash") != source_hash or "workloads" not in rec:
            rec = {"source_hash": source_hash, "workloads": {}}
        rec["workloads"][w] = tr
        with open(json_path, "w") as f:
            json.dump(rec, f, indent=1)

    # MFMA utilisation
    buf = io.StringIO()
    mu = mfma_util(os.path.join(prof, f"mfma_{tag}_results.db"), buf)
    lines = header("rocprofv3 MFMA utilisation", ["tune", "mfma"],
                   f"{me} --mfma {os.path.join(prof, f'mfma_{tag}_results.db')}")
    lines += ["# clock_GHz = GRBM_GUI_ACTIVE / 8 XCDs / dispatch duration; mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES /",
              "# (1024 SIMDs x engine cycles); implied_TFLOP/s = mfma_busy x 2500 x clock / 2.4 GHz (the dense bf16",
              "# rate those two allow). Kernels without MFMA work are left out. The counter run serialises",
              "# dispatches with gaps between them, so clocks run higher and the step slower than in the bench.",
              "# mfma_probe_kernel is the MFMA-only probe: its launches of 1 ms or more (the bench's warm-up and",
              "# timed probe); the few-microsecond launches between the GEMMs (clock samples) are left out.", "#"]
    lines += buf.getvalue().rstrip("\n").splitlines()
    an = analytical_flops(trace_bench)
    lines += ["#", "# hardware flop count (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) against the analytical 2 M N K per launch",
              "# (analytical: bench.py's per-call records of the traced run; ratio > 1 is MFMA work on padding)"]
    for k, r in sorted(mu.items()):
        if k in an and r.get("hw_flops_per_launch"):
            lines.append(f"#   {k:<58} analytical {an[k] / 1e9:>10.3f} GFLOP  hardware "
                         f"{r['hw_flops_per_launch'] / 1e9:>10.3f} GFLOP  ratio {r['hw_flops_per_launch'] / an[k]:.4f}")
    if mfma_bench:
        c = mfma_bench.get("clock") or {}
        pr = c.get("mfma_probe") or {}
        lines += ["#", f"# bench.py line of the counter run: value {mfma_bench['value']} TFLOP/s, ms_per_step "
                       f"{mfma_bench['ms_per_step']}"]
        if pr:
            lines.append(f"# its MFMA-only probe: {pr.get('tflops')} TFLOP/s, shader-clock counter {pr.get('clock_GHz')} "
                         f"GHz, {pr.get('flop_per_clock_per_cu')} bf16 flop per clock per CU; step clock "
                         f"{c.get('clock_GHz')} GHz from the probe launches between the GEMMs")
    with open(os.path.join(out_dir, f"mfma_util__{w}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db", nargs="?")
    ap.add_argument("--by-grid", action="store_true")
    ap.add_argument("--pmc", action="store_true")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"))
    ap.add_argument("--mfma", metavar="MFMA_DB")
    ap.add_argument("--copy-kernel", default="elementwise")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--json", default=None)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--source-hash", default=None)
    ap.add_argument("--report", metavar="DIR", default=None)
    ap.add_argument("--prof-dir", default="prof", help="directory of the rocprofv3 runs (-d of their commands)")
    ap.add_argument("--workload-number", type=int, default=5)
    ap.add_argument("--alt-plans", default="", help="comma-separated plan ids of --force-plan counter runs")
    a = ap.parse_args()
    if a.report:
        alt = [int(x) for x in a.alt_plans.split(",") if x.strip()]
        report(a.report, a.workload, a.workload_number, a.prof_dir, a.source_hash, a.json, a.copy_kernel,
               a.copy_bytes, alt)
    elif a.traffic:
        res = traffic(a.traffic[0], a.traffic[1], a.copy_kernel, a.copy_bytes)
        if a.json:
            import json
            res["workload"] = a.workload
            res["source_hash"] = a.source_hash
            with open(a.json, "w") as f:
                json.dump(res, f, indent=1)
    elif a.mfma:
        mfma_util(a.mfma)
    elif a.pmc:
        summarize_pmc(a.db)
    else:
        summarize(a.db, a.by_grid)


if __name__ == "__main__":
    main()
