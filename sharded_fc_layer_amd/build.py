"""Build libfcshard.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m sharded_fc_layer_amd.build  (or __graft_entry__.build()).
Each .hip source is compiled to an object in parallel, then linked into a
shared library next to this file.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfcshard.so")
BUILD_DIR = os.path.join(ROOT, "_build")

# largest first, so that the parallel build starts them first
SOURCES = ["gemm_w4_ring256.hip", "gemm_w4_ring192.hip", "gemm_w4_ring256b.hip", "gemm_w4_ring192b.hip",
           "gemm_w4.hip", "gemm_pipe.hip", "gemm_bf16.hip", "aux_kernels.hip", "mfma_probe.hip", "fcshard_api.hip"]

# packed-fp32 instructions are switched off for all device code
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: set HIPCC or install ROCm")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libfcshard.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmd = [cc, *HIPCC_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        if verbose:
            sys.stderr.write(r.stderr)
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    try:  # every symbol must resolve (a kernel instance without a host stub would not)
        ctypes.CDLL(tmp)
    except OSError as e:
        os.remove(tmp)
        raise RuntimeError(f"the linked library does not load: {e}") from None
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
