"""Overlap and interference on one GPU: a shard GEMM on the compute stream while
a copy the size of a collective's message runs on a second stream.

The pages overlap non-blocking collectives with computation and report what it
saves per batch (sciencestack.ai/paper/2502.08145, Figure 5; pith.science/paper/
2502.08145, "What carries the argument"). On one GPU the collective itself
cannot run, but the part of it that competes with the GEMM can: a ring step
reads and writes its chunk in HBM on compute units, as RCCL's kernels do. This
module stands a plain device copy of S bytes (read S, write S) in for the
message and measures, for one GEMM:

* the GEMM alone, the copy alone, and both started together on two streams;
* the GEMM's slow-down: its time under the copy / its time alone;
* the time the copy adds, t_both - t_gemm, and the hidden fraction of the copy,
  (t_gemm + t_copy - t_both) / t_copy: 1 when the copy is free, 0 when the two
  serialise, below 0 when running them together is slower than one after the
  other.

With CU masks (copy_cus > 0), the copy's stream runs on a few compute units
spread over the chip and the GEMM's stream on the others, the way a runtime
can reserve compute units for communication; the GEMM alone on every compute
unit is timed beside it.

Each timing is the median of `reps` runs, the configurations taken in turn, with the L2s and the MALL flushed before each run (the GEMM's operands
come from HBM, as in a training step). The
GEMM's output under the copy must equal its output alone, bit for bit.

Usage: python -m sharded_fc_layer_amd.overlap [--shape M,K,N] [--op fwd] [--mbytes 151,403]
"""
from __future__ import annotations

import argparse
import json
import statistics
import sys
from typing import Dict, List, Sequence

from . import fcshard as F

OPS = {"fwd": F.OP_FWD, "bwd_data": F.OP_BWD_DATA, "bwd_weight": F.OP_BWD_WEIGHT}


class _Bufs:
    def __init__(self, torch, M: int, K: int, N: int, copy_bytes: int, host_inputs=None):
        if host_inputs is not None:  # bf16 bit patterns (uint16), logical row-major
            import numpy as np

            def dev(bits):
                return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)

            self.X, self.W, self.dY = dev(host_inputs["X"]), dev(host_inputs["W"]), dev(host_inputs["dY"])
        else:
            g = torch.Generator(device="cuda").manual_seed(5)
            self.X = torch.randn((M, K), device="cuda", generator=g).to(torch.bfloat16)
            self.W = (torch.randn((K, N), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
            self.dY = (torch.randn((M, N), device="cuda", generator=g) * 1e-3).to(torch.bfloat16)
        self.Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        self.dX = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
        self.dW = torch.empty((K, N), dtype=torch.bfloat16, device="cuda")
        n = max(1, copy_bytes // 2)
        self.src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        self.dst = torch.empty_like(self.src)
        self.flush_a = torch.ones(1 << 28, dtype=torch.bfloat16, device="cuda")  # 512 MB
        self.flush_b = torch.empty_like(self.flush_a)

    def gemm(self, op: str, stream) -> None:
        s = stream.cuda_stream
        if op == "fwd":
            F.fc_fwd(self.X, self.W, out=self.Y, stream=s)
        elif op == "bwd_data":
            F.fc_bwd_data(self.dY, self.W, out=self.dX, stream=s)
        else:
            F.fc_bwd_weight(self.X, self.dY, out=self.dW, stream=s)


def _hip_runtime():
    """ctypes handle of the HIP runtime this process already uses (torch's):
    loading another copy would start a second runtime."""
    import ctypes
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                return ctypes.CDLL(line.split()[-1])
    raise RuntimeError("no HIP runtime is loaded")


def cu_masked_stream(torch, cus: Sequence[int]):
    """A stream (default priority) whose kernels run only on compute units `cus`."""
    import ctypes
    n = torch.cuda.get_device_properties(0).multi_processor_count
    words = (n + 31) // 32
    mask = (ctypes.c_uint32 * words)()
    for c in cus:
        mask[c // 32] |= 1 << (c % 32)
    h = ctypes.c_void_p()
    rc = _hip_runtime().hipExtStreamCreateWithCUMask(ctypes.byref(h), ctypes.c_uint32(words), mask)
    if rc != 0:
        raise RuntimeError(f"hipExtStreamCreateWithCUMask returned {rc}")
    return torch.cuda.ExternalStream(h.value)


def measure(M: int, K: int, N: int, op: str, copy_mbytes: Sequence[float], reps: int = 7,
            tune: bool = True, copy_cus: int = 0, host_inputs=None, return_output: bool = False) -> List[Dict]:
    """One record per message size (see the module docstring). With copy_cus > 0
    the copy's stream runs on that many compute units, spread over the chip,
    and the GEMM's stream on the others (CU-masked streams). host_inputs: the
    operands as bf16 bit patterns ({"X", "W", "dY"}, logical row-major; default
    torch.randn on the device). return_output: each record also holds, under
    "output", the GEMM's output written while the copy ran, as a host tensor."""
    import torch
    if op not in OPS:
        raise ValueError(f"op must be one of {sorted(OPS)}")
    if tune:
        F.fc_tune(M, K, N)
    plan = F.fc_plan_describe(OPS[op], M, K, N)
    if copy_cus > 0:
        n = torch.cuda.get_device_properties(0).multi_processor_count
        copy_set = sorted({(i * 33) % n for i in range(copy_cus)})  # 33 is coprime with the CU count
        main = cu_masked_stream(torch, [c for c in range(n) if c not in copy_set])
        side = cu_masked_stream(torch, copy_set)
    else:
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream()  # default priority
    full = torch.cuda.current_stream()
    out = []
    for mb in copy_mbytes:
        b = _Bufs(torch, M, K, N, int(mb * 1e6), host_inputs)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]

        def flush():
            b.flush_b.copy_(b.flush_a)
            torch.cuda.synchronize()

        def run(gemm: bool, copy: bool, main=main):
            flush()
            ev[0].record(main)
            side.wait_event(ev[0])
            if gemm:
                b.gemm(op, main)
            ev[1].record(main)
            if copy:
                with torch.cuda.stream(side):
                    ev[2].record(side)
                    b.dst.copy_(b.src)
                    ev[3].record(side)
            else:
                ev[2].record(side)
                ev[3].record(side)
            main.wait_stream(side)
            ev[4].record(main)
            torch.cuda.synchronize()
            return (ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3]), ev[0].elapsed_time(ev[4]))

        run(True, True)  # warm-up
        res = {"fwd": b.Y, "bwd_data": b.dX, "bwd_weight": b.dW}[op]
        run(True, False)
        ref = res.clone()  # written with no copy running
        # the three configurations interleaved, so that clock drift hits them alike
        alone, copy_alone, both, whole = [], [], [], []
        for _ in range(reps):
            alone.append(run(True, False))
            if copy_cus > 0:
                whole.append(run(True, False, main=full))  # the GEMM on every compute unit
            copy_alone.append(run(False, True))
            both.append(run(True, True))
        # the output of the last run, written while the copy ran
        same = bool(torch.equal(ref.view(torch.int16), res.view(torch.int16)))
        t_g = statistics.median(a[0] for a in alone)
        t_c = statistics.median(c[1] for c in copy_alone)
        t_g_under = statistics.median(x[0] for x in both)
        t_c_under = statistics.median(x[1] for x in both)
        t_both = statistics.median(x[2] for x in both)
        out.append({"M": M, "K": K, "N": N, "op": op, "kernel": plan["kernel"], "copy_MB": mb,
                    "gemm_ms": round(t_g, 4), "copy_ms": round(t_c, 4),
                    "copy_GBs": round(2 * mb * 1e6 / (t_c * 1e-3) / 1e9, 1),
                    "gemm_under_copy_ms": round(t_g_under, 4), "copy_under_gemm_ms": round(t_c_under, 4),
                    "both_ms": round(t_both, 4), "added_ms": round(t_both - t_g, 4), "copy_cus": copy_cus,
                    "gemm_all_cus_ms": round(statistics.median(x[0] for x in whole), 4) if whole else None,
                    "gemm_slowdown": round(t_g_under / t_g, 4),
                    "hidden_fraction": round((t_g + t_c - t_both) / t_c, 4), "output_identical": same})
        if return_output:
            out[-1]["output"] = res.cpu()
        del b
        torch.cuda.empty_cache()
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--shape", default="8192,6144,24576", help="M,K,N")
    ap.add_argument("--op", default="fwd", choices=sorted(OPS))
    ap.add_argument("--mbytes", default="101,151,403", help="message sizes in MB")
    ap.add_argument("--reps", type=int, default=15)
    ap.add_argument("--copy-cus", type=int, default=0,
                    help="run the copy on this many compute units and the GEMM on the rest (0: no masks)")
    a = ap.parse_args(argv)
    M, K, N = (int(v) for v in a.shape.split(","))
    for r in measure(M, K, N, a.op, [float(v) for v in a.mbytes.split(",")], a.reps, copy_cus=a.copy_cus):
        print(json.dumps(r), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
