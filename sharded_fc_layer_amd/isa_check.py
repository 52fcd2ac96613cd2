"""Accumulator-hazard check of the built library's gfx950 machine code.

The one-wave-per-SIMD kernels issue their MFMAs as inline asm with the
accumulators pinned to AGPRs, so the compiler does not insert the wait states
that a nearby non-MFMA access of those accumulators needs. This module takes
the gfx950 code objects out of libfcshard.so (the `.hip_fatbin` section holds
one offload bundle per source file), disassembles them with the ROCm LLVM
tools and scans every kernel, in program order, for:

1. a non-MFMA write of an AGPR (``v_accvgpr_write`` / ``v_accvgpr_mov``)
   followed within ``WRITE_WINDOW`` issue slots by an MFMA that reads it as
   its accumulator input;
2. an MFMA result read or overwritten by a non-MFMA instruction within
   ``READ_WINDOW`` slots, unless an ``s_waitcnt`` on ``vmcnt`` in between
   stalls the wave: at the places the kernels do this (after their main
   loops), that wait covers loads issued during the last MFMAs, which take
   hundreds of cycles;
3. a VALU write of a VGPR followed within ``VALU_WINDOW`` slots by an MFMA
   that reads it as an operand (the accumulator zeroing builds its zero
   operand with VALU moves right before its asm MFMAs).

``s_nop N`` counts N + 1 slots. The scan follows fall-through order only,
and covers the kernels whose MFMAs are inline asm (``ASM_KERNELS``); the
compiler inserts the wait states of its own MFMA builtins.
Usage: ``python -m sharded_fc_layer_amd.isa_check [libfcshard.so]``.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile
from typing import Dict, List

HERE = os.path.dirname(os.path.abspath(__file__))
LLVM = os.environ.get("ROCM_LLVM", "/opt/rocm/llvm/bin")
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
WRITE_WINDOW = 6   # slots between an AGPR write and an MFMA reading it
READ_WINDOW = 18   # slots between an MFMA and a non-MFMA access of its result
VALU_WINDOW = 2    # slots between a VALU write of a VGPR and an MFMA reading it
ASM_KERNELS = re.compile(r"gemm_w4k64r?(_stamped)?_kernel")


def tools_available() -> bool:
    return all(os.path.exists(os.path.join(LLVM, t)) for t in ("llvm-objcopy", "clang-offload-bundler",
                                                                "llvm-objdump"))


def code_objects(lib: str) -> List[bytes]:
    """The gfx950 ELF code objects inside the library, one per source file with device code."""
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fatbin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", f".hip_fatbin={fat}", lib,
                        os.path.join(d, "stripped")], check=True, capture_output=True)
        data = open(fat, "rb").read()
        starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
        out = []
        for k, s in enumerate(starts):
            part = os.path.join(d, f"bundle{k}")
            open(part, "wb").write(data[s:starts[k + 1] if k + 1 < len(starts) else len(data)])
            elf = os.path.join(d, f"co{k}.elf")
            r = subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                                f"--targets={TARGET}", f"--input={part}", f"--output={elf}"], capture_output=True)
            if r.returncode == 0 and os.path.getsize(elf) > 0:
                out.append(open(elf, "rb").read())
        return out


def disassemble(elf: bytes) -> str:
    with tempfile.NamedTemporaryFile(suffix=".elf") as f:
        f.write(elf)
        f.flush()
        r = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", f.name],
                           check=True, capture_output=True, text=True)
        return r.stdout


def _agprs(tok: str) -> set:
    m = re.match(r"a\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"a(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _vgprs(tok: str) -> set:
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def scan(text: str) -> Dict[str, dict]:
    """Per kernel: MFMA count and the hazards found (list of strings)."""
    res: Dict[str, dict] = {}
    name = None
    wr: list = []   # (agprs, slots since a non-MFMA write)
    mw: list = []   # (agprs, slots since an MFMA wrote them)
    vw: list = []   # (vgprs, slots since a VALU write)

    def age(n):
        nonlocal wr, mw, vw
        wr = [(r, s + n) for r, s in wr if s + n < WRITE_WINDOW]
        mw = [(r, s + n) for r, s in mw if s + n < READ_WINDOW]
        vw = [(r, s + n) for r, s in vw if s + n < VALU_WINDOW]

    for line in text.split("\n"):
        m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
        if m:
            name = m.group(1)
            res[name] = {"mfma": 0, "hazards": []}
            wr, mw, vw = [], [], []
            continue
        if name is None:
            continue
        t = line.split("//")[0].strip()
        if not t or t.endswith(":"):
            continue
        parts = t.replace(",", " ").split()
        op, ops = parts[0], parts[1:]
        if op == "s_nop":
            age(int(ops[0], 0) + 1 if ops else 1)
            continue
        if op.startswith("s_waitcnt") and "vmcnt" in t and "vmcnt(63)" not in t:
            mw = []
            age(1)
            continue
        if op.startswith("v_mfma"):
            res[name]["mfma"] += 1
            srcc = _agprs(ops[3]) if len(ops) > 3 else set()
            for r, s in wr:
                if r & srcc:
                    res[name]["hazards"].append(f"MFMA reads a{min(r & srcc)} {s} slots after a write: {t}")
            srcv = set().union(*[_vgprs(o) for o in ops[1:4]]) if len(ops) > 1 else set()
            for r, s in vw:
                if r & srcv:
                    res[name]["hazards"].append(f"MFMA reads v{min(r & srcv)} {s} slots after a VALU write: {t}")
            age(1)
            dst = _agprs(ops[0]) if ops else set()
            if dst:
                mw.append((dst, 0))
            continue
        if op.startswith("v_"):
            touched = set().union(*[_agprs(o) for o in ops]) if ops else set()
            for r, s in mw:
                if r & touched:
                    res[name]["hazards"].append(f"{t} accesses a{min(r & touched)} {s} slots after an MFMA wrote it")
            age(1)
            dst = _agprs(ops[0]) if ops else set()
            if dst:
                wr.append((dst, 0))
            vdst = _vgprs(ops[0]) if ops else set()
            if vdst:
                vw.append((vdst, 0))
            continue
        age(1)
    return res


def check(lib: str) -> Dict[str, dict]:
    """Scan results of the inline-asm MFMA kernels of the library."""
    out: Dict[str, dict] = {}
    for elf in code_objects(lib):
        out.update({k: v for k, v in scan(disassemble(elf)).items() if ASM_KERNELS.search(k)})
    return out


def main(argv=None) -> int:
    argv = sys.argv[1:] if argv is None else argv
    lib = argv[0] if argv else os.path.join(HERE, "libfcshard.so")
    res = check(lib)
    bad = {k: v for k, v in res.items() if v["hazards"]}
    n_mfma = sum(1 for v in res.values() if v["mfma"])
    print(f"{len(res)} inline-asm MFMA kernels ({n_mfma} with MFMAs), {len(bad)} with hazards")
    for k, v in bad.items():
        print(k)
        for h in v["hazards"][:5]:
            print("   ", h)
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main())
