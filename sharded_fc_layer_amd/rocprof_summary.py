"""Summarize rocprofv3 output of this library's kernels as short text.

Reads a rocprofv3 rocpd database (<name>_results.db) and prints, per kernel
(optionally per kernel and grid size), the dispatch count and the average,
minimum, maximum and total duration; for counter runs (--pmc) it prints the
per-dispatch averages of each counter. Usage:

  python -m sharded_fc_layer_amd.rocprof_summary RESULTS.db [--by-grid] [--pmc]
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("--by-grid", action="store_true")
    ap.add_argument("--pmc", action="store_true")
    a = ap.parse_args()
    if a.pmc:
        summarize_pmc(a.db)
    else:
        summarize(a.db, a.by_grid)


if __name__ == "__main__":
    main()
