"""The stamped products (fc_stamped_call, a measurement aid): the same bits
as the hot call of the same plan, exact against the oracle, and counter
readings that are ordered and consistent (the stage count the kernel ran,
an engine clock in range, loop cycles per stage at or above the MFMA
floor); plans without a stamped form are refused before anything runs."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from sharded_fc_layer_amd import fcshard as F
from sharded_fc_layer_amd import inputs as I

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

ROW, COL = I.ROW, I.COL
RING = 512  # family 8 (ring, 3 A + 2 B tiles), 256 x 256 tiles, one slice, no copy
RING_B = 576  # family 9 (the mirrored ring, 2 A + 3 B tiles), otherwise the same
RING_SPLIT2 = 516  # the same with the reduction split in two


def log(msg: str) -> None:
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def dev(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def host(t) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.fixture(autouse=True)
def _clean_plans():
    yield
    torch.cuda.synchronize()
    F.fc_release()


# (M, K, N): reductions of 128 stages (head 2), 64 (head 4), 7 (padded form),
# 1000 values (15 whole stages and a partial one, in front of two virtual
# stages: padded form) and ragged outputs
SHAPES = [(512, 8192, 768), (768, 4096, 512), (520, 448, 264), (256, 1000, 264)]


def _operands(op, c):
    if op == F.OP_FWD:
        return c["X"], c["W"], c["xo"], c["wo"]
    if op == F.OP_BWD_DATA:
        return c["dY"], c["W"], ROW, c["wo"]
    return c["X"], c["dY"], c["xo"], ROW


def _hot(op, c):
    if op == F.OP_FWD:
        return F.fc_fwd(c["X"], c["W"], c["xo"], c["wo"])
    if op == F.OP_BWD_DATA:
        return F.fc_bwd_data(c["dY"], c["W"], c["wo"])
    return F.fc_bwd_weight(c["X"], c["dY"], c["xo"])


def _oracle(op, d, xo, wo, M, K, N):
    if op == F.OP_FWD:
        return oracle.fc_fwd(I.stored(d["X"], xo), xo, I.stored(d["W"], wo), wo, M, K, N)[0]
    if op == F.OP_BWD_DATA:
        return oracle.fc_bwd_data(d["dY"], I.stored(d["W"], wo), wo, M, K, N)[0]
    return oracle.fc_bwd_weight(I.stored(d["X"], xo), xo, d["dY"], M, K, N)[0]


@pytest.mark.parametrize("plan", [RING, RING_B])
@pytest.mark.parametrize("shape", SHAPES)
def test_stamped_products_are_the_hot_calls(shape, plan):
    M, K, N = shape
    d = I.make_integer_inputs(M, K, N, seed=M + K + N)
    wall_mhz = F.fc_mfma_probe(16)["wall_clock_mhz"]
    for xo, wo in ((ROW, ROW), (COL, COL), (ROW, COL)):
        c = {"X": dev(I.stored(d["X"], xo)), "W": dev(I.stored(d["W"], wo)), "dY": dev(d["dY"]),
             "xo": xo, "wo": wo}
        for op in (F.OP_FWD, F.OP_BWD_DATA, F.OP_BWD_WEIGHT):
            red = {F.OP_FWD: K, F.OP_BWD_DATA: N, F.OP_BWD_WEIGHT: M}[op]
            F.fc_set_plan(op, M, K, N, xo, wo, F.OUT_BF16, plan)
            desc = F.fc_plan_describe(op, M, K, N, xo, wo, F.OUT_BF16)
            what = f"op {op} shape {shape} orders {xo}{wo}: {desc['kernel']} pad={desc['pad']}"
            log(what)
            A, B, ao, bo = _operands(op, c)
            G, stamps = F.fc_stamped(op, A, B, ao, bo)
            H = _hot(op, c)
            torch.cuda.synchronize()
            assert np.array_equal(host(G), host(H)), f"{what}: stamped and hot call differ"
            if red <= 1000:  # the whole output against the oracle (small reductions)
                want = oracle.round_bf16(_oracle(op, d, xo, wo, M, K, N))
                assert np.array_equal(host(G), want), f"{what}: not exact"
            s = stamps.cpu().numpy()
            rows, cols = G.shape
            assert s.shape == (((rows + 255) // 256) * ((cols + 255) // 256), F.STAMP_SLOTS)
            # counter readings in order within every block
            for a, b in ((0, 2), (2, 3), (3, 4), (4, 5)):
                assert np.all(s[:, b] >= s[:, a]), f"{what}: slot {b} before slot {a}"
            assert np.all(s[:, 6] > s[:, 1]), f"{what}: no wall time"
            assert desc["kernel"].endswith(", 3>" if plan == RING else ", 2>"), what
            padded = ", -1, " in desc["kernel"]
            whole = red // 64
            if red % 64:  # the partial stage and the virtual ones in front of the whole stages
                assert padded and desc["ktail"] == red % 64, what
                want_stages = whole + 6 - whole % 6
            else:
                want_stages = whole + ((6 - whole % 6) % 6 if padded else 0)
            assert np.all(s[:, 7] == want_stages), f"{what}: stages {set(s[:, 7].tolist())} vs {want_stages}"
            r = F.summarize_stamps(s, wall_mhz)
            log(f"  clock {r['clock_GHz']:.3f} GHz, loop {r['loop_cycles_per_stage']:.0f} cycles/stage, "
                f"prologue {r['prologue_cycles']:.0f}, epilogue {r['epilogue_cycles']:.0f}")
            assert 0.3 < r["clock_GHz"] < 3.5, what
            # 128 MFMAs of 16 x 16 x 32 per wave and stage: at least ~2048 cycles
            assert 1800 < r["loop_cycles_per_stage"] < 100000, what
            F.fc_set_plan(op, M, K, N, xo, wo, F.OUT_BF16, -1)


def test_plans_without_a_stamped_form_are_refused():
    M, K, N = 512, 4096, 512
    d = I.make_integer_inputs(M, K, N, seed=3)
    X, W = dev(d["X"]), dev(d["W"])
    F.fc_set_plan(F.OP_FWD, M, K, N, ROW, ROW, F.OUT_BF16, RING_SPLIT2)
    stamps = torch.full((4, F.STAMP_SLOTS), -7, dtype=torch.int64, device="cuda")
    out = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(F.FcError) as e:
        F.fc_stamped(F.OP_FWD, X, W, out=out, stamps=stamps)
    assert e.value.status == F.FC_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((stamps == -7).all()) and bool((out == 3.0).all()), "something ran"
    # a stamps buffer too small for the launch's blocks
    F.fc_set_plan(F.OP_FWD, M, K, N, ROW, ROW, F.OUT_BF16, RING)
    with pytest.raises(F.FcError) as e:
        F.fc_stamped(F.OP_FWD, X, W, stamps=torch.zeros((3, F.STAMP_SLOTS), dtype=torch.int64, device="cuda"))
    assert e.value.status == F.FC_E_INVALID
