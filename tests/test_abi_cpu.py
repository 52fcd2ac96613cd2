"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects malformed arguments before touching a device."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

from sharded_fc_layer_amd import fcshard as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(F.LIB_PATH):
        from sharded_fc_layer_amd import build
        build.build()
    return F.lib()


def test_header_declares_the_boundary():
    names = F.header_functions()
    for n in ("fc_fwd", "fc_bwd_data", "fc_bwd_weight", "fc_tune", "fc_status_str", "fc_release",
              "fc_set_plan", "fc_plan_describe", "fc_plan_count", "fc_plans_save", "fc_plans_load"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", F.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, re.M))
    for n in F.header_functions():
        assert n in exported, n
        assert hasattr(L, n)


def test_enum_values_match_header():
    text = open(F.HEADER).read()
    for name, val in [("FC_OK", F.FC_OK), ("FC_E_INVALID", F.FC_E_INVALID), ("FC_E_UNSUPPORTED", F.FC_E_UNSUPPORTED),
                      ("FC_E_HIP", F.FC_E_HIP), ("FC_E_NOMEM", F.FC_E_NOMEM),
                      ("FC_E_TOO_LARGE", F.FC_E_TOO_LARGE), ("FC_ROW_MAJOR", F.ROW),
                      ("FC_COL_MAJOR", F.COL), ("FC_OUT_BF16", F.OUT_BF16), ("FC_OUT_F32", F.OUT_F32),
                      ("FC_OUT_F32_ACCUMULATE", F.OUT_F32_ACC),
                      ("FC_OP_FWD", F.OP_FWD), ("FC_OP_BWD_DATA", F.OP_BWD_DATA),
                      ("FC_OP_BWD_WEIGHT", F.OP_BWD_WEIGHT)]:
        assert re.search(rf"\b{name}\s*=\s*{val}\b", text), name


def test_status_strings(L):
    for s in range(6):
        assert F.status_str(s).startswith("FC_")
    assert F.status_str(99) == "unknown fc_status"
    assert F.fc_plan_count() == 640


def test_null_and_bad_dimensions_rejected_without_a_device(L):
    fake = ctypes.c_void_p(0x100000)
    # NULL operands
    assert L.fc_fwd(None, 0, fake, 0, fake, 0, 8, 8, 8, None) == F.FC_E_INVALID
    assert L.fc_bwd_data(fake, None, 0, fake, 0, 8, 8, 8, None) == F.FC_E_INVALID
    assert L.fc_bwd_weight(fake, 0, fake, None, 0, 8, 8, 8, None) == F.FC_E_INVALID
    assert L.fc_bwd_weight_noalloc(fake, 0, None, fake, 0, 8, 8, 8, None) == F.FC_E_INVALID
    assert L.fc_bwd_weight_noalloc(a_ := ctypes.c_void_p(0x100000), 0, ctypes.c_void_p(0x200000),
                                   ctypes.c_void_p(0x300000), 0, 8, 0, 8, None) == F.FC_E_INVALID
    assert F.fc_noalloc_scratch_bytes() == 64 << 20
    # dimensions < 1 and bad enums are caught before any HIP call
    a, b, c = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000)
    assert L.fc_fwd(a, 0, b, 0, c, 0, 0, 8, 8, None) == F.FC_E_INVALID
    assert L.fc_fwd(a, 0, b, 0, c, 0, 8, -1, 8, None) == F.FC_E_INVALID
    assert L.fc_fwd(a, 2, b, 0, c, 0, 8, 8, 8, None) == F.FC_E_INVALID
    assert L.fc_fwd(a, 0, b, 0, c, 7, 8, 8, 8, None) == F.FC_E_INVALID
    # misaligned and overlapping outputs
    assert L.fc_fwd(a, 0, b, 0, ctypes.c_void_p(0x300001), 0, 8, 8, 8, None) == F.FC_E_INVALID
    assert L.fc_fwd(a, 0, b, 0, ctypes.c_void_p(0x300002), 1, 8, 8, 8, None) == F.FC_E_INVALID
    assert L.fc_fwd(a, 0, b, 0, ctypes.c_void_p(0x300002), 2, 8, 8, 8, None) == F.FC_E_INVALID  # fp32 alignment
    assert L.fc_fwd(a, 0, b, 0, c, 3, 8, 8, 8, None) == F.FC_E_INVALID
    assert L.fc_fwd(a, 0, b, 0, ctypes.c_void_p(0x100010), 0, 8, 8, 8, None) == F.FC_E_INVALID
    assert L.fc_tune(0, 8, 8, 0, 0, 0, 0, None) == F.FC_E_INVALID
    assert L.fc_set_plan(0, 8, 8, 8, 0, 0, 0, F.fc_plan_count()) == F.FC_E_INVALID
    assert L.fc_plan_describe(0, 8, 8, 8, 0, 0, 0, None, 0) == F.FC_E_INVALID


def test_binding_fails_loudly_when_library_missing(monkeypatch):
    monkeypatch.setattr(F, "_lib", None)
    monkeypatch.setattr(F, "LIB_PATH", os.path.join(ROOT, "does_not_exist", "libfcshard.so"))
    with pytest.raises(RuntimeError, match="missing"):
        F.lib()
