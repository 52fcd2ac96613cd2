"""Host sanitizer runs (AddressSanitizer, UndefinedBehaviorSanitizer and
LeakSanitizer), no GPU needed:

* the CPU oracle (oracle/oracle.c) under tests/sanitize/oracle_driver.c,
  built with gcc;
* the C-ABI layer's host code (csrc/fcshard_api.hip, included by
  tests/sanitize/abi_driver.hip), built with hipcc with the sanitizers on
  the host side only and linked with the library's other objects.

Each driver checks its own results and exits non-zero on a failed check;
any sanitizer report ends the run with an error as well.
"""
from __future__ import annotations

import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Wno-unknown-pragmas", "-o", exe,
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert "sanitized oracle run: ok" in r.stdout


def _library_objects():
    """The library's objects other than the C-ABI layer, rebuilt when a source is newer."""
    from sharded_fc_layer_amd import build
    objs = {s: os.path.join(build.BUILD_DIR, s + ".o") for s in build.SOURCES if s != "fcshard_api.hip"}
    sources = glob.glob(os.path.join(build.CSRC, "*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    newest = max(os.path.getmtime(p) for p in sources)
    if any(not os.path.exists(o) or os.path.getmtime(o) < newest for o in objs.values()):
        build.build()
    return list(objs.values())


def test_abi_host_code_under_sanitizers(tmp_path):
    from sharded_fc_layer_amd import build
    objs = _library_objects()
    obj = str(tmp_path / "abi_driver.o")
    exe = str(tmp_path / "abi_driver")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all"]
    _run([build.hipcc(), *flags, "-I", os.path.join(ROOT, "include"), "-I", build.CSRC, "-c",
          os.path.join(HERE, "abi_driver.hip"), "-o", obj])
    # host link with the sanitizer runtimes (device code is already embedded)
    linker = "/opt/rocm/llvm/bin/clang++"
    if not os.path.exists(linker):
        pytest.skip("ROCm clang++ not found")
    link = [linker, "-fsanitize=address,undefined", "-o", exe, obj, *objs,
            "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    _run(link)
    r = _run([exe], env=ENV, timeout=300)
    assert "sanitized ABI run: ok" in r.stdout
