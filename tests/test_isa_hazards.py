"""The accumulator-hazard check of the built library's machine code (CPU).

The scanner is pinned first on small disassembly listings with and without
the hazards it looks for (the first one is the form a real miscompile took:
an accumulator copy two instructions after the MFMA writing it). Then every
inline-asm MFMA kernel of the built library must come out clean.
"""
from __future__ import annotations

import os

import pytest

from sharded_fc_layer_amd import isa_check as C

HEAD = "0000000000001000 <_ZN3fcs12_GLOBAL__N_117gemm_w4k64_kernelILb0ELb0ELb0ELi256EEEvNS_8GemmArgsE>:\n"
MFMA = "\tv_mfma_f32_16x16x32_bf16 a[124:127], v[78:81], v[66:69], a[124:127]   // 000000001000: D3B5807C\n"


def _listing(*body: str) -> str:
    return HEAD + MFMA + "".join("\t" + b + "\n" for b in body)


def _hazards(text: str):
    return next(iter(C.scan(text).values()))["hazards"]


def test_read_right_after_the_mfma_is_found():
    h = _hazards(_listing("s_cbranch_scc0 65533", "s_waitcnt lgkmcnt(14)", "v_accvgpr_read_b32 v4, a124"))
    assert len(h) == 1 and "a124" in h[0]


def test_enough_wait_states_clear_it():
    assert not _hazards(_listing("s_nop 7", "s_nop 7", "s_nop 3", "v_accvgpr_read_b32 v4, a124"))
    assert _hazards(_listing("s_nop 7", "s_nop 7", "v_accvgpr_read_b32 v4, a124"))  # 16 + 1 slots: too few


def test_a_vmcnt_wait_clears_it():
    assert not _hazards(_listing("s_waitcnt vmcnt(0) lgkmcnt(0)", "v_accvgpr_read_b32 v4, a125"))


def test_other_registers_are_not_flagged():
    assert not _hazards(_listing("v_accvgpr_read_b32 v4, a123", "v_accvgpr_mov_b32 a0, a128"))


def test_write_right_before_an_mfma_is_found():
    text = HEAD + "\tv_accvgpr_write_b32 a3, 0\n\ts_nop 1\n" + \
        "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[2:5], v[6:9], a[0:3]\n"
    h = _hazards(text)
    assert len(h) == 1 and "a3" in h[0]
    text_ok = HEAD + "\tv_accvgpr_write_b32 a3, 0\n\ts_nop 7\n" + \
        "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[2:5], v[6:9], a[0:3]\n"
    assert not _hazards(text_ok)


def test_valu_write_of_an_mfma_operand_is_found():
    """The form a real fault took: the zero operand of the accumulator-zeroing
    MFMAs moved into place by VALU instructions right before them, so the
    first MFMA read stale values and left garbage in an accumulator."""
    text = HEAD + "\tv_mov_b64_e32 v[4:5], s[30:31]\n" + \
        "\tv_mfma_f32_16x16x32_bf16 a[252:255], v[2:5], v[2:5], 0\n"
    h = _hazards(text)
    assert len(h) == 1 and "v4" in h[0] and "VALU" in h[0]
    assert _hazards(HEAD + "\tv_mov_b32_e32 v3, 0\n\ts_nop 0\n"
                    "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[2:5], v[2:5], 0\n")  # 1 slot: too few
    assert not _hazards(HEAD + "\tv_mov_b32_e32 v3, 0\n\ts_nop 1\n"
                        "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[2:5], v[2:5], 0\n")
    assert not _hazards(HEAD + "\tv_mov_b32_e32 v9, 0\n"
                        "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[2:5], v[2:5], 0\n")  # another register


LIB = os.path.join(os.path.dirname(C.HERE), "sharded_fc_layer_amd", "libfcshard.so")


@pytest.mark.skipif(not C.tools_available(), reason="ROCm LLVM tools not found")
@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_built_library_is_clean():
    res = C.check(LIB)
    # two-slot kernels (2 tile widths) and ring kernels (padded and head forms), 8 layouts/outputs each
    assert len(res) >= 60 and all(v["mfma"] > 0 for v in res.values())
    bad = {k: v["hazards"][:3] for k, v in res.items() if v["hazards"]}
    assert not bad, bad
