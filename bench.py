#!/usr/bin/env python3
"""Throughput of one GPU's FC-layer shard GEMMs (forward + both backward
products) on an MI355X, through the library's C ABI.

A step is one pass of the hot path over one batch of synthetic input: for
every FC layer of the workload, forward Y = X.W, backward-data dX = dY.W^T
and backward-weight dW = X^T.dY, issued back to back on one HIP stream
(bf16 in, fp32 accumulate, bf16 out) in training-step order (the forwards
layer by layer, then the backward products in reverse), with the plans
fc_tune picked (tuning runs before the timed region). Inputs are seeded
synthetic bf16 (N(0, 1) activations, N(0, 0.02) weights, N(0, 1e-3) output
gradients), resident in HBM before timing.

Default workload: one GPU's shard of a 405B-like layer (hidden 16384, FFN
53248, 128 heads) on a virtual 2 x 4 x 2 grid with 8192 tokens per shard,
plus a 16384 x 16032 vocabulary-projection shard: QKV 8192 -> 12288,
out-projection 8192 -> 4096, MLP up 8192 -> 13312, MLP down 26624 -> 4096,
vocabulary 16384 -> 16032, i.e. 15 GEMMs per step.

Prints ONE JSON line. `value` is TFLOP/s (2 M K N per GEMM, summed over the
step, divided by the mean step time); the mean of the last 8 steps, the
median, min and max are given beside it. `roofline` reports the dominant
kernel (largest summed time) against the dense bf16 MFMA peak, from HIP
events recorded on the launch stream around each of its launches.
`clock` gives the engine clock sampled during a second pass of the step, the
empirical per-CU MFMA rate of the MFMA-only probe kernel, and the step's
fraction of the clock-scaled peak. `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "sharded_fc_layer_amd", "csrc")
# every source with device code (the C-ABI layer, fcshard_api.hip, is host code only)
KERNEL_SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                        if f.endswith((".hip", ".h", ".inc")) and f != "fcshard_api.hip")


def kernel_source_hash(sources=None) -> str:
    """Hash of the device code (comments and whitespace removed): counter figures
    taken on other code are stale; comment edits leave them valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sorted(sources or KERNEL_SOURCES):
        with open(f, encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(os.path.basename(f).encode() + b"\0" + " ".join(text.split()).encode() + b"\0")
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, grids=None):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter
    runs, or None when none were taken for it or the kernel sources changed since.
    With `grids` (the launch grid, in threads, of each of this run's calls of
    the kernel), the mean over those calls of the counter runs' figure for
    each grid, so that a kernel several GEMMs share is weighed by this run's
    own calls; the kernel's overall mean if a grid was not profiled."""
    import json as _json
    try:
        with open(TRAFFIC_FILE) as f:
            rec = _json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    k = rec.get("workloads", {}).get(workload, {}).get("kernels", {}).get(kernel)
    if k is None:
        return None
    by = k.get("by_grid") or {}
    if grids and all(str(g) in by for g in grids):
        return sum(by[str(g)]["hbm_bytes_per_launch"] for g in grids) / len(grids)
    return k.get("hbm_bytes_per_launch")

WORKLOAD_NAMES = {
    1: "single_fc_256x512x2048",
    2: "gpt_block_h2048_t8192",
    3: "mlp_up_shard_h12288_2x2x2",
    4: "skinny_shard_h16384_gx8_gy8",
    5: "llm405b_like_layer_2x4x2_plus_vocab",
}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", type=int, default=5, choices=sorted(WORKLOAD_NAMES))
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    p.add_argument("--no-extra", action="store_true", help="skip the large-shard context workloads")
    p.add_argument("--no-tune", action="store_true", help="use the default plans")
    p.add_argument("--plans", default=None,
                   help="plan file: loaded if it exists (no tuning in this run), else written after tuning")
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="CPU oracle timing: the sample doubles until one pass takes at least half of this")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run one plain 1 GiB device copy (a known-size reference for HBM counters)")
    p.add_argument("--no-clock", action="store_true", help="skip the clock pass and the MFMA-only probe")
    p.add_argument("--force-plan", type=int, default=None,
                   help="after loading or tuning the plans, run every product with this plan id where it "
                        "applies (counter runs: the kernels that other tunings pick)")
    p.add_argument("--probe-iters", type=int, default=60000,
                   help="MFMA-only probe: rounds of 64 MFMAs per wave (60000: about 0.5 s)")
    return p.parse_args()


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


class Layer:
    """Device buffers of one FC shard and the three calls of a step."""

    def __init__(self, g, X, W, dY, torch, F, xo=0, wo=0):
        self.g, self.F = g, F
        self.X, self.W, self.dY = X, W, dY  # X, W stored in orders xo, wo (0 row-, 1 column-major)
        self.xo, self.wo = xo, wo
        self.Y = torch.empty((g.M, g.N), dtype=torch.bfloat16, device="cuda")
        self.dX = torch.empty((g.M, g.K), dtype=torch.bfloat16, device="cuda")
        self.dW = torch.empty((g.K, g.N), dtype=torch.bfloat16, device="cuda")
        self.dW32 = None  # set: dW is added into this fp32 buffer (gradient accumulation)

    def calls(self):
        F = self.F
        if self.dW32 is not None:
            dw = lambda: F.fc_bwd_weight(self.X, self.dY, self.xo, out=self.dW32,  # noqa: E731
                                         out_dtype=F.OUT_F32_ACC)
        else:
            dw = lambda: F.fc_bwd_weight(self.X, self.dY, self.xo, out=self.dW)  # noqa: E731
        return [
            ("fwd", F.OP_FWD, lambda: F.fc_fwd(self.X, self.W, self.xo, self.wo, out=self.Y)),
            ("bwd_data", F.OP_BWD_DATA, lambda: F.fc_bwd_data(self.dY, self.W, self.wo, out=self.dX)),
            ("bwd_weight", F.OP_BWD_WEIGHT, dw),
        ]


    def stamp_args(self, code):
        """fc_stamped's operands, orders and output for product `code` (None
        when the step accumulates dW in fp32: the stamped form is bf16 only)."""
        F = self.F
        if code == F.OP_FWD:
            return self.X, self.W, self.xo, self.wo, self.Y
        if code == F.OP_BWD_DATA:
            return self.dY, self.W, 0, self.wo, self.dX
        return None if self.dW32 is not None else (self.X, self.dY, self.xo, 0, self.dW)


def make_layers(workload, torch, F, I, host_inputs, xo=0, wo=0):
    """Device buffers of every FC shard of a workload: the seeded host inputs
    (host_inputs=True; X and W stored in orders xo, wo), or draws of the same
    distributions on the device."""
    import numpy as np
    layers = []
    for gi, g in enumerate(I.WORKLOADS[workload], start=1):
        if host_inputs:
            d = I.make_inputs(workload, gi)
            dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to("cuda").view(torch.bfloat16)  # noqa: E731
            layers.append(Layer(g, dev(I.stored(d["X"], xo)), dev(I.stored(d["W"], wo)), dev(d["dY"]), torch, F,
                                xo, wo))
            del d
        else:
            gen = torch.Generator(device="cuda").manual_seed(1000 * workload + gi)
            rn = lambda r, c, s: (torch.randn((r, c), device="cuda", generator=gen) * s).to(torch.bfloat16)  # noqa
            X = rn(g.M, g.K, g.sx) if xo == 0 else rn(g.K, g.M, g.sx)
            W = rn(g.K, g.N, g.sw) if wo == 0 else rn(g.N, g.K, g.sw)
            layers.append(Layer(g, X, W, rn(g.M, g.N, g.sdy), torch, F, xo, wo))
    return layers


class ClockSampler:
    """Samples the engine (gfx) clock and the socket power of the device in a
    background thread, through amdsmi (read-only metrics; no GPU work)."""

    def __init__(self, torch, interval_s=0.005):
        import amdsmi
        self.smi, self.interval = amdsmi, interval_s
        amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
        handles = amdsmi.amdsmi_get_processor_handles()
        if not handles:
            raise RuntimeError("amdsmi sees no GPU")
        self.h = handles[0]
        props = torch.cuda.get_device_properties(0)
        bus = getattr(props, "pci_bus_id", None)
        if bus is not None and len(handles) > 1:
            for h in handles:  # the handle whose PCI bus is torch's device 0
                if int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == int(bus):
                    self.h = h
                    break
        self.samples, self._stop, self._thread = [], False, None

    def read(self):
        m = self.smi.amdsmi_get_gpu_metrics_info(self.h)
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 10000]
        clk = sum(clks) / len(clks) if clks else m.get("current_gfxclk")
        pw = m.get("current_socket_power")
        return (float(clk) if isinstance(clk, (int, float)) else None,
                float(pw) if isinstance(pw, (int, float)) and 0 < pw < 10000 else None)

    def _run(self):
        import threading  # noqa: F401
        while not self._stop:
            try:
                self.samples.append((time.perf_counter(),) + self.read())
            except Exception:  # a failed read leaves a gap, not an error
                pass
            time.sleep(self.interval)

    def start(self):
        import threading
        self.samples, self._stop = [], False
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self):
        self._stop = True
        self._thread.join()
        clk = [c for _, c, _ in self.samples if c]
        pw = [p for _, _, p in self.samples if p]
        return {"samples": len(self.samples), "clock_mhz_mean": sum(clk) / len(clk) if clk else None,
                "clock_mhz_min": min(clk) if clk else None, "clock_mhz_max": max(clk) if clk else None,
                "socket_power_w_mean": sum(pw) / len(pw) if pw else None}

    def close(self):
        try:
            self.smi.amdsmi_shut_down()
        except Exception:
            pass


def clock_and_probe(layers, steps, args, torch, F):
    """The engine clock during the step, the MFMA-only probe (the GEMM kernels'
    MFMA stream alone: the empirical bf16 flop per clock per CU), and the
    step's fraction of the clock-scaled peak: compute units x that rate x the
    step's clock.

    The clock is read on the GPU itself: in a second pass of the step, a
    short launch of the probe kernel (16 rounds of 64 MFMAs per wave, a few
    microseconds) follows every GEMM, and each of its blocks reads the
    shader-clock counter against the constant-rate counter; the chip's clock
    moves on a millisecond scale, so that is the clock the GEMM ran at. The
    step's clock is the mean over GEMMs weighted by their flops. Socket power
    is sampled through amdsmi meanwhile."""
    import numpy as np
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    pr = F.fc_mfma_probe(args.probe_iters)
    wall_mhz = pr["wall_clock_mhz"]
    probe_ghz = pr["counter_ratio"] * wall_mhz / 1e3
    rate = pr["flops"] / (pr["ms"] / 1e3)
    per_cu = rate / (pr["compute_units"] * probe_ghz * 1e9)  # bf16 flop per clock per CU
    res = {"mfma_probe": {"ms": round(pr["ms"], 3), "tflops": round(rate / 1e12, 2),
                          "compute_units": pr["compute_units"], "clock_GHz": round(probe_ghz, 4),
                          "flop_per_clock_per_cu": round(per_cu, 1),
                          "frac_of_4096_per_clock": round(per_cu / 4096, 4),
                          "kernel": "mfma_probe_kernel: 64 v_mfma_f32_16x16x32_bf16 per round, 256 AGPR "
                                    "accumulators per wave, one wave per SIMD, no loads / LDS / barriers"}}
    calls = step_calls(layers)
    clocks = torch.zeros((steps * len(calls), cus, 4), dtype=torch.int64, device="cuda")
    for _ in range(3):
        for _, (_, _, fn) in calls:
            fn()
    torch.cuda.synchronize()
    try:
        smp = ClockSampler(torch)
        smp.start()
    except Exception as e:  # no power readings: the clock comes from the GPU anyway
        smp, res["power"] = None, f"unavailable ({type(e).__name__})"
    for s in range(steps):
        for i, (_, (_, _, fn)) in enumerate(calls):
            fn()
            F.fc_mfma_probe_launch(clocks[s * len(calls) + i], iters=16)
    torch.cuda.synchronize()
    if smp:
        smp_res = smp.stop()
        smp.close()
        res["power"] = {"socket_power_w_mean": smp_res["socket_power_w_mean"], "samples": smp_res["samples"],
                        "amdsmi_gfxclk_mhz_mean": smp_res["clock_mhz_mean"],
                        "note": "amdsmi's clock figure is context only: under load it reads below the "
                                "shader-clock counter and the GRBM counter"}
    c = clocks.cpu().numpy().astype(np.float64)
    ghz = ((c[..., 1] - c[..., 0]) / (c[..., 3] - c[..., 2])).mean(axis=1) * wall_mhz / 1e3
    ghz = ghz.reshape(steps, len(calls))
    w = np.array([L.g.flops for L, _ in calls], dtype=np.float64)
    step_ghz = float((ghz.mean(axis=0) * w).sum() / w.sum())
    res["per_call_clock_GHz"] = {f"{L.g.name} {op}": round(float(v), 4)
                                 for (L, (op, _, _)), v in zip(calls, ghz.mean(axis=0))}
    peak = cus * per_cu * step_ghz * 1e9 / 1e12
    res.update({"clock_GHz": round(step_ghz, 4), "clock_scaled_peak": round(peak, 1),
                "clock_source": "shader-clock counter / constant-rate counter, read by a short probe launch "
                                "after every GEMM of a second pass of the step (flop-weighted mean)"})
    ik = stamp_pass(layers, steps, wall_mhz, per_cu, cus, torch, F)
    if "clock_GHz" in ik:
        ik["clock_scaled_peak"] = round(cus * per_cu * ik["clock_GHz"] * 1e9 / 1e12, 1)
    res["in_kernel"] = ik
    return res


def stamp_pass(layers, steps, wall_mhz, per_cu, cus, torch, F):
    """The engine clock and the main-loop cycles inside the GEMM kernels.

    The step runs `steps` more times with every product whose plan has a
    stamped form issued through fc_stamped_call: the same plan, result and
    main-loop instruction stream, with each block reading the shader-clock
    and constant-rate counters at entry and exit and the shader clock around
    its main loop. Products without a stamped form run as usual. Per product:
    the clock while its blocks ran, the loop's cycles per 64-value stage
    against the bare MFMA stream's (4 waves x 128 MFMAs of 16 x 16 x 32 per
    stage at the probe's flop per clock), and the prologue and epilogue."""
    import numpy as np
    calls = step_calls(layers)
    plan = []
    for L, (op, code, fn) in calls:
        a = L.stamp_args(code)
        bufs, ok = [], False
        if a is not None:
            rows, cols = a[4].shape
            nb = ((rows + 255) // 256) * ((cols + 255) // 256)
            bufs = [torch.zeros((nb, F.STAMP_SLOTS), dtype=torch.int64, device="cuda") for _ in range(steps)]
            try:
                F.fc_stamped(code, a[0], a[1], a[2], a[3], out=a[4], stamps=bufs[0])
                ok = True
            except F.FcError as e:
                if e.status != F.FC_E_UNSUPPORTED:
                    raise
        plan.append((L, op, fn, a, bufs, ok))
    torch.cuda.synchronize()
    for s in range(steps):
        for L, op, fn, a, bufs, ok in plan:
            if ok:
                F.fc_stamped(F.OP_FWD if op == "fwd" else F.OP_BWD_DATA if op == "bwd_data" else F.OP_BWD_WEIGHT,
                             a[0], a[1], a[2], a[3], out=a[4], stamps=bufs[s])
            else:
                fn()
    torch.cuda.synchronize()
    floor = 4 * 128 * 16 * 16 * 32 * 2 / per_cu  # cycles per stage of the bare MFMA stream
    per_call, w_all, w_ok, clk = {}, 0.0, 0.0, 0.0
    for L, op, fn, a, bufs, ok in plan:
        w_all += L.g.flops
        if not ok:
            per_call[f"{L.g.name} {op}"] = "no stamped form for its plan"
            continue
        host = [b.cpu().numpy() for b in bufs]
        r = F.summarize_stamps(np.concatenate(host), wall_mhz)
        per_launch = [F.summarize_stamps(h, wall_mhz, compute_units=cus) for h in host]
        per_call[f"{L.g.name} {op}"] = {
            "clock_GHz": round(r["clock_GHz"], 4), "loop_cycles_per_stage": round(r["loop_cycles_per_stage"], 1),
            "loop_vs_mfma_stream": round(floor / r["loop_cycles_per_stage"], 4),
            "loop_share_of_block": round(r["stages"] * r["loop_cycles_per_stage"] / r["block_cycles"], 4),
            "cu_occupancy": round(float(np.mean([x["cu_occupancy"] for x in per_launch])), 4),
            "launch_span_us": round(float(np.mean([x["launch_span_us"] for x in per_launch])), 2),
            "stages": r["stages"], "prologue_cycles": round(r["prologue_cycles"]),
            "epilogue_cycles": round(r["epilogue_cycles"]), "block_cycles": round(r["block_cycles"])}
        w_ok += L.g.flops
        clk += L.g.flops * r["clock_GHz"]
    if w_ok == 0:
        return {"note": "no product of the step has a stamped form"}
    loops = [v for v in per_call.values() if isinstance(v, dict)]
    wts = [L.g.flops for L, op, fn, a, bufs, ok in plan if ok]
    avg = lambda key: round(float(np.average([v[key] for v in loops], weights=wts)), 4)  # noqa: E731
    return {
        "clock_GHz": round(clk / w_ok, 4),
        "loop_vs_mfma_stream": avg("loop_vs_mfma_stream"),
        "loop_share_of_block": avg("loop_share_of_block"),
        "cu_occupancy": avg("cu_occupancy"),
        "mfma_stream_cycles_per_stage": round(floor, 1),
        "stamped_flop_fraction": round(w_ok / w_all, 4),
        "per_call": per_call,
        "source": "fc_stamped_call: per-block shader-clock / constant-rate counter readings inside the GEMM "
                  "kernels, flop-weighted over the step's products",
    }


def step_calls(layers):
    """Training-step order: forwards layer by layer, then backwards in reverse."""
    fw = [(L, c) for L in layers for c in L.calls()[:1]]
    bw = [(L, c) for L in reversed(layers) for c in L.calls()[1:]]
    return fw + bw


def step_flops(layers):
    return sum(3 * L.g.flops for L in layers)


def run_timed(layers, steps, warmup, torch):
    calls = step_calls(layers)
    for _ in range(warmup):
        for _, (_, _, fn) in calls:
            fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for s in range(steps):
        for _, (_, _, fn) in calls:
            fn()
        ev[s + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = [ev[s].elapsed_time(ev[s + 1]) for s in range(steps)]
    total_ms = ev[0].elapsed_time(ev[steps])
    return total_ms / steps, per_step, wall


def run_per_launch(layers, steps, torch, F):
    """Per-call HIP events on the launch stream: {kernel: [durations ms]}."""
    calls = step_calls(layers)
    stream = torch.cuda.current_stream()
    recs = []
    for _ in range(steps):
        for L, (opname, op, fn) in calls:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            recs.append((L, opname, op, a, b))
    torch.cuda.synchronize()
    out = {}
    for L, opname, op, a, b in recs:
        g = L.g
        desc = F.fc_plan_describe(op, g.M, g.K, g.N)
        key = desc["kernel"]
        # one kernel launch per call: no split (reduce launch), transpose copy,
        # reduction padding (pad_rows launches) or tail split
        single = desc["split"] == 1 and desc["copy"] == 0 and desc["pad"] == 0 and "tail" not in desc
        e = out.setdefault(key, {"ms": [], "flops": [], "bytes": [], "grids": [], "single_launch": True})
        e["ms"].append(a.elapsed_time(b))
        # launch grid in threads (a single launch: 256 x bn tiles, 256 threads each)
        rows, cols = {"fwd": (g.M, g.N), "bwd_data": (g.M, g.K), "bwd_weight": (g.K, g.N)}[opname]
        bn = 192 if desc.get("tile") == "256x192" else 256
        e["grids"].append(-(-rows // 256) * -(-cols // bn) * 256 if key.startswith("gemm_w4") else None)
        e["flops"].append(g.flops)
        # compulsory HBM bytes: both bf16 inputs once, the bf16 output once
        e["bytes"].append(2 * (g.M * g.K + g.K * g.N + g.M * g.N))
        e["single_launch"] = e["single_launch"] and single
        e.setdefault("by_call", {}).setdefault((g.name, opname), []).append(a.elapsed_time(b))
    return out


def plans_of(layers, F, kern=None):
    """The plan each call runs; with per-call timings, its mean time and rate inside the step."""
    by_call = {}
    for v in (kern or {}).values():
        for key, ms in v.get("by_call", {}).items():
            by_call.setdefault(key, []).extend(ms)
    res = []
    for L in layers:
        g = L.g
        for opname, op, _ in L.calls():
            d = F.fc_plan_describe(op, g.M, g.K, g.N)
            rec = {"gemm": g.name, "op": opname, "M": g.M, "K": g.K, "N": g.N, "kernel": d["kernel"],
                   "split": d["split"], "copy": d["copy"], "pad": d["pad"]}
            if "tail" in d:  # the kernel runs the unsplit part; the tail is another launch
                rec["tail"] = d["tail"]
            ms = by_call.get((g.name, opname))
            if ms:
                avg = sum(ms) / len(ms)
                rec["avg_us"] = round(avg * 1e3, 2)
                rec["tflops"] = round(g.flops / (avg / 1e3) / 1e12, 1)
            res.append(rec)
    return res


def cpu_baseline(workload, target_s, I):
    """The oracle as it stands, on sampled output rows of the workload."""
    import numpy as np
    import oracle
    try:
        cores = ctypes.CDLL("libgomp.so.1").omp_get_max_threads()
    except OSError:
        cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    gemms = I.WORKLOADS[workload]
    inputs = [I.make_inputs(workload, gi) for gi in range(1, len(gemms) + 1)]

    def one(gi, op, rows):
        g, d = gemms[gi], inputs[gi]
        if op == "fwd":
            oracle.fc_fwd(d["X"], 0, d["W"], 0, g.M, g.K, g.N, rows=rows)
            return 2 * len(rows) * g.K * g.N
        if op == "bwd_data":
            oracle.fc_bwd_data(d["dY"], d["W"], 0, g.M, g.K, g.N, rows=rows)
            return 2 * len(rows) * g.N * g.K
        oracle.fc_bwd_weight(d["X"], 0, d["dY"], g.M, g.K, g.N, rows=rows)
        return 2 * len(rows) * g.M * g.N

    ops = ["fwd", "bwd_data", "bwd_weight"]

    def one_pass(rows_each):
        t = time.perf_counter()
        fl = 0
        for gi in range(len(gemms)):
            for op in ops:
                n_out_rows = gemms[gi].K if op == "bwd_weight" else gemms[gi].M
                rows = np.linspace(0, n_out_rows - 1, min(rows_each, n_out_rows)).astype(np.int64)
                fl += one(gi, op, rows)
        return fl, time.perf_counter() - t

    # double the sample until one pass takes at least half the target time
    rows_each = 8
    while True:
        flops, dt = one_pass(rows_each)
        if dt >= 0.5 * target_s or rows_each >= 8192:
            break
        rows_each *= 2
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows_each} full output rows of each of the {3 * len(gemms)} GEMMs of the workload "
                      f"({flops / 1e9:.1f} GFLOP in {dt:.1f} s; fp64 plain loops, OpenMP)",
            "seconds": dt, "cpu": cpu}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        return 2
    import numpy as np
    import torch

    from sharded_fc_layer_amd import fcshard as F
    from sharded_fc_layer_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    F.lib()  # fails loudly if the HIP library is missing
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)

    log(f"device {props.name} {getattr(props, 'gcnArchName', '')}; workload {args.workload}")
    t = time.perf_counter()
    layers = make_layers(args.workload, torch, F, I, host_inputs=True)
    log(f"inputs resident ({time.perf_counter() - t:.1f} s)")
    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration: 1 GiB read + 1 GiB write")
    tune_s = 0.0
    if args.plans and os.path.exists(args.plans):
        F.fc_plans_load(args.plans)
        log(f"loaded plans from {args.plans}")
    elif not args.no_tune:
        t = time.perf_counter()
        for L in layers:
            F.fc_tune(L.g.M, L.g.K, L.g.N)
        torch.cuda.synchronize()
        tune_s = time.perf_counter() - t
        log(f"tuned {len(layers)} shapes in {tune_s:.1f} s")
        if args.plans:
            F.fc_plans_save(args.plans)
    if args.force_plan is not None:
        forced = sum(F.fc_set_plan(op, L.g.M, L.g.K, L.g.N, L.xo, L.wo, F.OUT_BF16, args.force_plan) == F.FC_OK
                     for L in layers for op in (F.OP_FWD, F.OP_BWD_DATA, F.OP_BWD_WEIGHT))
        log(f"plan {args.force_plan} forced on {forced} of {3 * len(layers)} products")

    ms, per_step, wall = run_timed(layers, args.steps, args.warmup, torch)
    flops = step_flops(layers)
    value = flops / (ms / 1e3) / 1e12
    log(f"{ms:.3f} ms/step, {value:.1f} TFLOP/s")

    kern = run_per_launch(layers, args.steps, torch, F)
    # the dominant kernel among those whose every call launches that kernel
    # alone (no transpose copy, split-K reduction or reduction padding), so
    # that the per-call events time exactly that kernel
    single = {k: v for k, v in kern.items() if v["single_launch"]} or kern
    dom = max(single.items(), key=lambda kv: sum(kv[1]["ms"]))
    dname, drec = dom
    d_avg_ms = float(np.mean(drec["ms"]))
    d_avg_flops = float(np.mean(drec["flops"]))
    achieved = d_avg_flops / (d_avg_ms / 1e3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(dname, WORKLOAD_NAMES[args.workload], drec["grids"]), "kernel": dname,
                "launches": len(drec["ms"]), "avg_launch_us": round(d_avg_ms * 1e3, 2),
                "avg_gflop_per_launch": round(d_avg_flops / 1e9, 3),
                "algorithmic_bytes_per_launch": int(np.mean(drec["bytes"])),
                "single_launch_plans": drec["single_launch"]}
    per_kernel = {k: {"launches": len(v["ms"]), "avg_us": round(float(np.mean(v["ms"])) * 1e3, 2),
                      "tflops": round(float(np.sum(v["flops"]) / (np.sum(v["ms"]) / 1e3) / 1e12), 1)}
                  for k, v in kern.items()}

    last8 = per_step[-8:] if len(per_step) >= 10 else per_step
    result = {
        "metric": "bf16 TFLOP/s of FC fwd+bwd shard GEMMs on 1 MI355X; % of MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "tokens": I.WORKLOADS[args.workload][0].M,
                   "gemms": [[g.name, g.M, g.K, g.N] for g in I.WORKLOADS[args.workload]],
                   "products_per_gemm": ["fwd", "bwd_data", "bwd_weight"], "orders": "X row, W row",
                   "out_dtype": "bf16", "step_gflop": round(flops / 1e9, 2)},
        "pct_of_mfma_peak": round(100 * value / MFMA_BF16_PEAK_TFLOPS, 2),
        "step_ms_stats": {"mean_last8": round(float(np.mean(last8)), 4), "median": round(float(np.median(per_step)), 4),
                          "min": round(float(np.min(per_step)), 4), "max": round(float(np.max(per_step)), 4)},
        "roofline": roofline,
        "per_kernel": per_kernel,
        "plans": plans_of(layers, F, kern),
        "tune_s": round(tune_s, 2),
        "kernel_source_hash": kernel_source_hash(),
        "device": props.name,
    }

    if not args.no_clock:
        c = clock_and_probe(layers, args.steps, args, torch, F)
        result["clock"] = c
        result["clock_GHz"] = c["clock_GHz"]
        result["clock_scaled_peak"] = c["clock_scaled_peak"]
        result["frac_clock"] = round(value / c["clock_scaled_peak"], 4)
        if "clock_scaled_peak" in c["in_kernel"]:
            # the same against the clock measured inside the kernels
            result["frac_in_kernel_clock"] = round(value / c["in_kernel"]["clock_scaled_peak"], 4)
        log(f"clock {c['clock_GHz']} GHz; probe {c['mfma_probe']}; clock-scaled peak {c['clock_scaled_peak']} "
            f"TFLOP/s; frac_clock {result['frac_clock']}; power {c.get('power')}")

    if not args.no_extra:
        del layers
        torch.cuda.empty_cache()
        context = {}
        for w in (2, 3, 5):  # every other workload of one or more FC shards, row-major
            if w == args.workload:
                continue
            Ls = make_layers(w, torch, F, I, host_inputs=True)
            if not args.no_tune:
                for L in Ls:
                    F.fc_tune(L.g.M, L.g.K, L.g.N)
            wms, wsteps, _ = run_timed(Ls, 10, 3, torch)
            wf = step_flops(Ls)
            context[WORKLOAD_NAMES[w]] = {
                "tflops": round(wf / (wms / 1e3) / 1e12, 1), "ms_per_step": round(wms, 3),
                "mean_last8_ms": round(float(np.mean(wsteps[-8:])), 3),
                "pct_of_mfma_peak": round(100 * wf / (wms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 1),
                "gemms_per_step": 3 * len(Ls)}
            log(f"workload {w}: {context[WORKLOAD_NAMES[w]]}")
            del Ls
            torch.cuda.empty_cache()
        result["workload_context"] = context
        # the layout sweep: the skinny shard in each storage-order pair
        sweep = {}
        for xo, wo in I.ORDER_PAIRS:
            Ls = make_layers(4, torch, F, I, host_inputs=True, xo=xo, wo=wo)
            if not args.no_tune:
                for L in Ls:
                    F.fc_tune(L.g.M, L.g.K, L.g.N, xo, wo)
            wms, _, _ = run_timed(Ls, 10, 3, torch)
            wf = step_flops(Ls)
            key = f"X {'row' if xo == 0 else 'col'}, W {'row' if wo == 0 else 'col'}"
            sweep[key] = {"tflops": round(wf / (wms / 1e3) / 1e12, 1), "ms_per_step": round(wms, 3),
                          "plans": [F.fc_plan_describe(op, L.g.M, L.g.K, L.g.N, xo, wo)["kernel"]
                                    for L in Ls for op in (F.OP_FWD, F.OP_BWD_DATA, F.OP_BWD_WEIGHT)]}
            log(f"workload 4 {key}: {sweep[key]['tflops']} TFLOP/s")
            del Ls
            torch.cuda.empty_cache()
        result["layout_sweep_context"] = {"workload": WORKLOAD_NAMES[4], "gemms_per_step": 3, "by_orders": sweep}
        # the GPT-block step with every dW added into an fp32 gradient buffer
        # (accumulation over micro-batches), for context
        Ls = make_layers(2, torch, F, I, host_inputs=True)
        for L in Ls:
            L.dW32 = torch.zeros((L.g.K, L.g.N), dtype=torch.float32, device="cuda")
            if not args.no_tune:
                F.fc_tune(L.g.M, L.g.K, L.g.N)
                F.fc_tune(L.g.M, L.g.K, L.g.N, out_dtype=F.OUT_F32_ACC)
        wms, _, _ = run_timed(Ls, 10, 3, torch)
        wf = step_flops(Ls)
        result["dw_accumulate_context"] = {
            "workload": WORKLOAD_NAMES[2],
            "tflops": round(wf / (wms / 1e3) / 1e12, 1), "ms_per_step": round(wms, 3),
            "dw_dtype": "fp32, added into (FC_OUT_F32_ACCUMULATE)",
            "dw_extra_bytes_per_step": int(sum(6 * L.g.K * L.g.N for L in Ls))}
        log(f"dW accumulate: {result['dw_accumulate_context']}")
        del Ls
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds, I)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
