"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

* exact: integer-valued inputs make every fp32 partial sum exact in any
  order, so fp32 outputs must equal the oracle bit for bit and bf16 outputs
  must equal the oracle's nearest-even rounding of the exact value - for every
  product, storage order, output type, odd shape and every plan the tuner can
  pick;
* tolerance: N(0, sigma) inputs on ragged shapes and on the five workloads at
  full size (sampled outputs computed one by one by the oracle), with the
  plans fc_tune picks, as the benchmark runs them: max |G - O| <= 1e-2 S
  elementwise (S = |A|.|B|) and relative Frobenius error <= 5e-3;
* determinism: the same plan twice gives the same bits.
"""
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
OPS = ["fwd", "bwd_data", "bwd_weight"]
ALL_ORDERS = [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)]
RING = 512  # family 8 (ring, 3 A + 2 B tiles), 256 x 256 tiles, one slice, no copy
RING_B = 576  # family 9 (the mirrored ring, 2 A + 3 B tiles), otherwise the same
ELEM_TOL, FRO_TOL = 1e-2, 5e-3


def log(msg: str) -> None:
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def dev(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def host(t) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class Case:
    """Inputs of one shard on the device in given storage orders."""

    def __init__(self, d, xo, wo):
        self.d, self.xo, self.wo = d, xo, wo
        self.M, self.K = d["X"].shape
        self.N = d["W"].shape[1]
        self.X = dev(I.stored(d["X"], xo))
        self.W = dev(I.stored(d["W"], wo))
        self.dY = dev(d["dY"])

    def gpu(self, op, out_dtype):
        if op == "fwd":
            return F.fc_fwd(self.X, self.W, self.xo, self.wo, out_dtype=out_dtype)
        if op == "bwd_data":
            return F.fc_bwd_data(self.dY, self.W, self.wo, out_dtype=out_dtype)
        return F.fc_bwd_weight(self.X, self.dY, self.xo, out_dtype=out_dtype)

    def oracle(self, op, rows=None, cols=None):
        d, M, K, N = self.d, self.M, self.K, self.N
        if op == "fwd":
            return oracle.fc_fwd(I.stored(d["X"], self.xo), self.xo, I.stored(d["W"], self.wo), self.wo, M, K, N,
                                 rows, cols)
        if op == "bwd_data":
            return oracle.fc_bwd_data(d["dY"], I.stored(d["W"], self.wo), self.wo, M, K, N, rows, cols)
        return oracle.fc_bwd_weight(I.stored(d["X"], self.xo), self.xo, d["dY"], M, K, N, rows, cols)


def op_code(op):
    return {"fwd": F.OP_FWD, "bwd_data": F.OP_BWD_DATA, "bwd_weight": F.OP_BWD_WEIGHT}[op]


def assert_exact(G: np.ndarray, O: np.ndarray, out_dtype: int, what: str):
    if out_dtype == F.OUT_F32:
        want = O.astype(np.float32)
        assert np.array_equal(want.astype(np.float64), O), "oracle value not exact in fp32"
        bad = np.argwhere(G.view(np.uint32) != want.view(np.uint32))
    else:
        want = oracle.round_bf16(O)
        bad = np.argwhere(G != want)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}"


def assert_close(G: np.ndarray, O: np.ndarray, S: np.ndarray, out_dtype: int, what: str):
    Gv = I.bf16_bits_to_f32(G) if out_dtype == F.OUT_BF16 else G
    r = oracle.compare(Gv, O, S, ELEM_TOL, FRO_TOL)
    log(f"  {what}: max_err_ratio={r['max_err_ratio']:.3g} rel_fro={r['rel_fro']:.3g}")
    assert r["pass"], f"{what}: {r}"


@pytest.fixture(autouse=True)
def _clean_plans():
    yield
    torch.cuda.synchronize()
    F.fc_release()


# ------------------------------------------------------------- exact parity

EXACT_SHAPES = [(1, 1, 1), (7, 33, 17), (33, 7, 65), (130, 257, 129), (8, 16, 24), (264, 520, 136),
                (256, 512, 256), (520, 136, 1032)]


@pytest.mark.parametrize("shape", EXACT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_exact_integer_default_plans(shape):
    M, K, N = shape
    d = I.make_integer_inputs(M, K, N, seed=1)
    for xo, wo in ALL_ORDERS:
        c = Case(d, xo, wo)
        for op in OPS:
            O, _ = c.oracle(op)
            for dt in (F.OUT_BF16, F.OUT_F32):
                what = f"{op} {shape} orders={xo}{wo} dtype={dt}"
                log(what)
                G = host(c.gpu(op, dt))
                torch.cuda.synchronize()
                assert_exact(G, O, dt, what)


def test_exact_power_of_two_scaled_inputs():
    # integers times powers of two: still exact; exercises exponent handling
    M, K, N = 136, 264, 72
    d = I.make_integer_inputs(M, K, N, seed=2, pow2=(-6, 3, -2))
    c = Case(d, ROW, ROW)
    for op in OPS:
        O, _ = c.oracle(op)
        for dt in (F.OUT_BF16, F.OUT_F32):
            assert_exact(host(c.gpu(op, dt)), O, dt, f"{op} pow2 dtype={dt}")


# (320, 576, 192): every reduction length (576, 192, 320) is a multiple of 64,
# so the kernels that take 32-value reduction stages in pairs run too, with
# ragged output tiles and two- and four-way reduction splits. (384, 1024, 384):
# every reduction a multiple of 128 (64-value stages in pairs), ragged tiles.
# (352, 608, 224): every reduction length is 32 more than a multiple of 64;
# split slices of 320 + 288 and of 192 + 192 + 192 + 32. (384, 1024, 328):
# forward and backward-weight outputs ragged against the 256- and 192-column
# block tiles (328 = 192 + 136), the second wave column of a 192-column tile
# partly outside the matrix. (512, 640, 1024): the ring kernel's head forms
# (reductions of 6 q + 2 or 6 q + 4 64-value stages, q >= 1) in all three
# products: 10 stages (head of 4) forward, 16 (4) backward-data, 8 (2)
# backward-weight, and the split slices of 8 + 8 (2) and 4 x 4 (padded).
# (392, 800, 136): reductions of 12 and 6 whole stages and a partial one,
# which the ring kernels run in front of five virtual stages (800 = 12 x 64 +
# 32, 392 = 6 x 64 + 8), and of 2 whole stages and 8 values (136); split
# slices of 448 + 352 and 256 + 136. (352, 608, 224) has 5 whole stages and a
# partial one (no virtual stage), (200, 1032, 72) 1 whole stage and 8 values.
@pytest.mark.parametrize("shape", [(264, 520, 136), (200, 1032, 72), (9, 130, 17), (320, 576, 192),
                                   (384, 1024, 384), (352, 608, 224), (384, 1024, 328), (512, 640, 1024),
                                   (392, 800, 136)],
                         ids=lambda s: "x".join(map(str, s)))
def test_exact_integer_every_plan(shape):
    M, K, N = shape
    d = I.make_integer_inputs(M, K, N, seed=3)
    n_plans = F.fc_plan_count()
    for xo, wo in ALL_ORDERS:
        c = Case(d, xo, wo)
        for op in OPS:
            O, _ = c.oracle(op)
            for dt in (F.OUT_BF16, F.OUT_F32):
                ran = 0
                for pid in range(n_plans):
                    st = F.fc_set_plan(op_code(op), M, K, N, xo, wo, dt, pid)
                    if st == F.FC_E_UNSUPPORTED:
                        continue
                    assert st == F.FC_OK, F.status_str(st)
                    desc = F.fc_plan_describe(op_code(op), M, K, N, xo, wo, dt)
                    assert desc["plan"] == pid
                    what = f"{op} {shape} orders={xo}{wo} dtype={dt} plan={pid} {desc['kernel']} pad={desc['pad']}"
                    log(what)
                    G = host(c.gpu(op, dt))
                    torch.cuda.synchronize()
                    assert_exact(G, O, dt, what)
                    ran += 1
                assert ran >= 1
                F.fc_set_plan(op_code(op), M, K, N, xo, wo, dt, -1)


# Output grids of more than 16 x 16 block tiles, so the block map's every
# case runs: full 16 x 16 super-tiles (an 8 x 4 sub-block per XCD), right
# edges 2 and 8 tiles wide, bottom bands of 1 and 2 tile rows; with 256- and
# 192-column tiles (18 and 24 tile columns). Forward (the M x N output) on the
# ring and two-slot plans, exact on every element.
@pytest.mark.parametrize("shape", [(4352, 128, 4608), (4608, 128, 4096)], ids=lambda s: "x".join(map(str, s)))
def test_exact_block_map_large_grids(shape):
    M, K, N = shape
    d = I.make_integer_inputs(M, K, N, seed=14)
    c = Case(d, ROW, ROW)
    O, _ = c.oracle("fwd")
    ran = 0
    for pid in range(F.fc_plan_count()):
        if F.fc_set_plan(F.OP_FWD, M, K, N, ROW, ROW, F.OUT_BF16, pid) != F.FC_OK:
            continue
        desc = F.fc_plan_describe(F.OP_FWD, M, K, N, ROW, ROW, F.OUT_BF16)
        if not desc["kernel"].startswith("gemm_w4k64") or desc["split"] != 1 or desc["copy"] != 0:
            continue
        what = f"fwd {shape} plan={pid} {desc['kernel']} tile={desc['tile']}"
        log(what)
        G = host(c.gpu("fwd", F.OUT_BF16))
        torch.cuda.synchronize()
        assert_exact(G, O, F.OUT_BF16, what)
        ran += 1
    assert ran >= 4


# Tail plans: output grids of 16 x 20 tiles (the last 4 tile columns split)
# and 20 x 16 tiles (the last 4 tile rows), for each product (its output is
# M x N, M x K or K x N); reductions of 1024 (two slices of 8 stages, head
# forms) and of 1000 (15 whole stages and 40 values unsplit; slices of 512 and
# 488 values, the second ending with a partial stage). Exact for every
# storage order, bf16 and fp32 outputs and an accumulating output.
TAIL_CASES = [("fwd", (4096, 1024, 5120)), ("fwd", (5120, 1024, 4096)), ("bwd_data", (4096, 5120, 1024)),
              ("bwd_weight", (1024, 4096, 5120)), ("bwd_weight", (1024, 5120, 4096)),
              ("fwd", (4096, 1000, 5120)), ("bwd_weight", (1000, 5120, 4096))]


@pytest.mark.parametrize("op,shape", TAIL_CASES, ids=[f"{o}-{'x'.join(map(str, s))}" for o, s in TAIL_CASES])
def test_exact_tail_split_plans(op, shape):
    M, K, N = shape
    d = I.make_integer_inputs(M, K, N, seed=15)
    rng = np.random.default_rng(15)
    O = None
    ran = 0
    for xo, wo in ALL_ORDERS:
        c = Case(d, xo, wo)
        if O is None:
            O, S = c.oracle(op)
        for dt in (F.OUT_BF16, F.OUT_F32, F.OUT_F32_ACC):
            for pid in range(F.fc_plan_count()):
                if F.fc_set_plan(op_code(op), M, K, N, xo, wo, dt, pid) != F.FC_OK:
                    continue
                desc = F.fc_plan_describe(op_code(op), M, K, N, xo, wo, dt)
                if "tail" not in desc:
                    continue
                what = f"{op} {shape} orders={xo}{wo} dtype={dt} plan={pid} {desc['kernel']} tail={desc['tail']}"
                log(what)
                if dt == F.OUT_F32_ACC:
                    C_old = rng.integers(-64, 65, size=O.shape).astype(np.float32)
                    want, _ = oracle.accumulate(C_old, O, S)
                    G = host(gpu_acc(c, op, C_old))
                    assert_exact(G, want, F.OUT_F32, what)
                else:
                    G = host(c.gpu(op, dt))
                    torch.cuda.synchronize()
                    assert_exact(G, O, dt, what)
                ran += 1
            F.fc_set_plan(op_code(op), M, K, N, xo, wo, dt, -1)
        del c
    assert ran >= 8


@pytest.mark.parametrize("exhaustive,warm", [(True, True), (False, False)], ids=["exhaustive-warm", "quick-flushed"])
def test_tuned_plans_exact(exhaustive, warm):
    """fc_tune in both candidate sets and both cache modes (its close
    candidates re-timed in rounds) picks plans that are exact on integer data,
    for every product and storage order, on ragged sizes."""
    M, K, N = 520, 1032, 264
    d = I.make_integer_inputs(M, K, N, seed=21)
    for xo, wo in ALL_ORDERS:
        c = Case(d, xo, wo)
        F.fc_tune(M, K, N, xo, wo, F.OUT_BF16, exhaustive=exhaustive, warm_caches=warm)
        for op in OPS:
            desc = F.fc_plan_describe(op_code(op), M, K, N, xo, wo, F.OUT_BF16)
            assert desc.get("tuned_ms", 0) > 0, desc
            what = f"tuned {op} orders={xo}{wo} plan={desc['plan']} {desc['kernel']}"
            log(what)
            O, _ = c.oracle(op)
            G = host(c.gpu(op, F.OUT_BF16))
            torch.cuda.synchronize()
            assert_exact(G, O, F.OUT_BF16, what)
        del c
    F.fc_release()


def test_ring_partial_stage_needs_a_whole_stage_before_it():
    """A ring kernel runs a reduction's partial last stage only after at least
    one whole 64-value stage (its trailing prefetches reload the last whole
    one): forward reductions of 8 and 40 values refuse the ring plans, one of
    72 (a whole stage and 8 values) runs them exactly, with no workspace."""
    M, N = 264, 136
    for K, applies in ((8, False), (40, False), (72, True)):
        d = I.make_integer_inputs(M, K, N, seed=K)
        c = Case(d, ROW, ROW)
        O, _ = c.oracle("fwd")
        for pid in (RING, RING_B):
            st = F.fc_set_plan(F.OP_FWD, M, K, N, ROW, ROW, F.OUT_BF16, pid)
            if not applies:
                assert st == F.FC_E_UNSUPPORTED, (K, pid, F.status_str(st))
                continue
            assert st == F.FC_OK, (K, pid, F.status_str(st))
            desc = F.fc_plan_describe(F.OP_FWD, M, K, N, ROW, ROW, F.OUT_BF16)
            assert desc["ktail"] == K % 64 and desc["ws"] == 0 and desc["pad"] == 0, desc
            what = f"fwd {(M, K, N)} plan={pid} {desc['kernel']}"
            log(what)
            G = host(c.gpu("fwd", F.OUT_BF16))
            torch.cuda.synchronize()
            assert_exact(G, O, F.OUT_BF16, what)
        F.fc_set_plan(F.OP_FWD, M, K, N, ROW, ROW, F.OUT_BF16, -1)
        del c


def test_default_plans_need_no_workspace():
    """Untuned shapes run a plan that needs no workspace, also where the
    one-wave-per-SIMD kernels could only run the reduction padded (K = 2040 is
    not a multiple of 64), and right after fc_release (no workspace at all).
    Exact on whole sampled rows and columns of integer-valued data."""
    M, K, N = 4096, 2040, 4096
    F.fc_release()
    for xo, wo in ALL_ORDERS:
        for op in OPS:
            for dt in (F.OUT_BF16, F.OUT_F32):
                desc = F.fc_plan_describe(op_code(op), M, K, N, xo, wo, dt)
                # (a plan whose operands are both output-contiguous pads the
                # reduction with no workspace: rows past K read zeros)
                assert desc["ws"] == 0, f"{op} orders={xo}{wo} dtype={dt}: {desc}"
    d = I.make_integer_inputs(M, K, N, seed=13)
    rng = np.random.default_rng(13)
    for xo, wo in ((ROW, ROW), (COL, ROW)):
        c = Case(d, xo, wo)
        for op in OPS:
            desc = F.fc_plan_describe(op_code(op), M, K, N, xo, wo, F.OUT_BF16)
            what = f"default plan {op} orders={xo}{wo} {desc['kernel']} pad={desc['pad']}"
            log(what)
            Gt = c.gpu(op, F.OUT_BF16)
            torch.cuda.synchronize()
            n_r, n_c = Gt.shape
            rows, cols = _sample(n_r, 6, rng), _sample(n_c, 6, rng)
            O, _ = c.oracle(op, rows, None)
            assert_exact(host(Gt[torch.from_numpy(rows).cuda()]), O, F.OUT_BF16, what + " rows")
            O, _ = c.oracle(op, None, cols)
            assert_exact(host(Gt[:, torch.from_numpy(cols).cuda()].contiguous()), O, F.OUT_BF16, what + " cols")
        del c


# ------------------------------------------------ accumulating fp32 output

def _out_shape(op, M, K, N):
    return {"fwd": (M, N), "bwd_data": (M, K), "bwd_weight": (K, N)}[op]


def gpu_acc(c: Case, op: str, C_old: np.ndarray):
    """The product added into a device copy of C_old (fp32)."""
    out = torch.from_numpy(np.ascontiguousarray(C_old, dtype=np.float32)).to("cuda")
    acc = F.OUT_F32_ACC
    if op == "fwd":
        F.fc_fwd(c.X, c.W, c.xo, c.wo, out=out, out_dtype=acc)
    elif op == "bwd_data":
        F.fc_bwd_data(c.dY, c.W, c.wo, out=out, out_dtype=acc)
    else:
        F.fc_bwd_weight(c.X, c.dY, c.xo, out=out, out_dtype=acc)
    return out


@pytest.mark.parametrize("shape", [(264, 520, 136), (384, 1024, 384), (352, 608, 224)],
                         ids=lambda s: "x".join(map(str, s)))
def test_accumulate_exact_every_plan(shape):
    """Every plan, split-K ones included, adds the exact product to the old values."""
    M, K, N = shape
    d = I.make_integer_inputs(M, K, N, seed=8)
    rng = np.random.default_rng(8)
    acc = F.OUT_F32_ACC
    for xo, wo in ALL_ORDERS:
        c = Case(d, xo, wo)
        for op in OPS:
            O, S = c.oracle(op)
            C_old = rng.integers(-64, 65, size=_out_shape(op, M, K, N)).astype(np.float32)
            want, _ = oracle.accumulate(C_old, O, S)
            ran = 0
            for pid in range(F.fc_plan_count()):
                st = F.fc_set_plan(op_code(op), M, K, N, xo, wo, acc, pid)
                if st == F.FC_E_UNSUPPORTED:
                    continue
                assert st == F.FC_OK, F.status_str(st)
                desc = F.fc_plan_describe(op_code(op), M, K, N, xo, wo, acc)
                what = f"acc {op} {shape} orders={xo}{wo} plan={pid} {desc['kernel']} split={desc['split']}"
                log(what)
                G = host(gpu_acc(c, op, C_old))
                assert_exact(G, want, F.OUT_F32, what)
                ran += 1
            assert ran >= 1
            F.fc_set_plan(op_code(op), M, K, N, xo, wo, acc, -1)


@pytest.mark.parametrize("shape", [(777, 1000, 555), (513, 2056, 257), (1024, 2048, 1536)],
                         ids=lambda s: "x".join(map(str, s)))
def test_accumulate_tolerance_tuned(shape):
    M, K, N = shape
    d = I.make_random_inputs(M, K, N, seed=9)
    rng = np.random.default_rng(9)
    F.fc_tune(M, K, N, ROW, ROW, F.OUT_F32_ACC)
    c = Case(d, ROW, ROW)
    for op in OPS:
        O, S = c.oracle(op)
        C_old = (rng.standard_normal(_out_shape(op, M, K, N)) * float(np.median(S))).astype(np.float32)
        want, S2 = oracle.accumulate(C_old, O, S)
        desc = F.fc_plan_describe(op_code(op), M, K, N, ROW, ROW, F.OUT_F32_ACC)
        assert_close(host(gpu_acc(c, op, C_old)), want, S2, F.OUT_F32,
                     f"acc {op} {shape} {desc['kernel']} split={desc['split']}")


def test_accumulated_micro_batches_equal_the_whole_batch():
    """dW accumulated over micro-batches of tokens = dW of the whole batch."""
    M, K, N = 2048, 1024, 768
    d = I.make_random_inputs(M, K, N, seed=10)
    O, S = Case(d, ROW, ROW).oracle("bwd_weight")
    dW = torch.zeros((K, N), dtype=torch.float32, device="cuda")
    for lo, hi in ((0, 768), (768, 2048)):
        part = {"X": np.ascontiguousarray(d["X"][lo:hi]), "W": d["W"], "dY": np.ascontiguousarray(d["dY"][lo:hi])}
        c = Case(part, ROW, ROW)
        F.fc_bwd_weight(c.X, c.dY, ROW, out=dW, out_dtype=F.OUT_F32_ACC)
    assert_close(host(dW), O, S, F.OUT_F32, "two micro-batches vs the whole batch")
    with pytest.raises(ValueError, match="existing output"):
        F.fc_bwd_weight(c.X, c.dY, ROW, out_dtype=F.OUT_F32_ACC)


# ------------------------------------------------------------ maximum sizes

def test_operands_of_2_gib_and_more():
    """X of 2 GiB and more is past the fast kernels' buffer descriptors: those
    plans do not apply and the simple kernel (64-bit addressing) runs the
    products that read X; backward-data writes a dX of 2 GiB and more.
    Integer-valued data, exact on sampled outputs."""
    M, K, N = 131080, 8192, 264  # X: 2.0002 GiB
    log(f"generating {M}x{K} integer inputs")
    d = {"X": I.integer_bf16_chunked([31, 1], (M, K)), "W": I.integer_bf16_chunked([31, 2], (K, N)),
         "dY": I.integer_bf16_chunked([31, 3], (M, N))}
    c = Case(d, ROW, ROW)
    rng = np.random.default_rng(31)
    for plans in ("default", "tuned"):
        if plans == "tuned":
            # the quick search still has candidates where only the simple kernel applies
            F.fc_tune(M, K, N)
        for op in OPS:
            desc = F.fc_plan_describe(op_code(op), M, K, N)
            what = f"max-size {plans} {op} {desc['kernel']} split={desc['split']}"
            log(what)
            if op != "bwd_data":
                assert desc["kernel"].startswith("gemm_bf16_kernel"), what
            if plans == "tuned":
                assert desc.get("tuned_ms", 0) > 0, what
            Gt = c.gpu(op, F.OUT_BF16)
            rows, cols = _sample(Gt.shape[0], 24, rng), _sample(Gt.shape[1], 96, rng)
            O, _ = c.oracle(op, rows, cols)
            G = host(Gt[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
            assert_exact(G, O, F.OUT_BF16, what)
            del Gt
    del c
    torch.cuda.empty_cache()


# --------------------------------------------------------- tolerance parity

@pytest.mark.parametrize("dt", [F.OUT_BF16, F.OUT_F32])
def test_workload1_full(dt):
    d = I.make_inputs(1, 1)
    c = Case(d, ROW, ROW)
    for op in OPS:
        O, S = c.oracle(op)
        assert_close(host(c.gpu(op, dt)), O, S, dt, f"workload1 {op} dtype={dt}")


@pytest.mark.parametrize("shape", [(777, 1000, 555), (1000, 264, 1304), (513, 2056, 257), (64, 4104, 72)],
                         ids=lambda s: "x".join(map(str, s)))
def test_ragged_tolerance_all_orders(shape):
    M, K, N = shape
    d = I.make_random_inputs(M, K, N, seed=4)
    for xo, wo in ALL_ORDERS:
        c = Case(d, xo, wo)
        # both timing modes of the tuner: flushed caches (default) and warm caches
        F.fc_tune(M, K, N, xo, wo, F.OUT_BF16, warm_caches=(xo == wo))
        for op in OPS:
            O, S = c.oracle(op)
            desc = F.fc_plan_describe(op_code(op), M, K, N, xo, wo, F.OUT_BF16)
            assert_close(host(c.gpu(op, F.OUT_BF16)), O, S, F.OUT_BF16,
                         f"{op} {shape} orders={xo}{wo} {desc['kernel']} split={desc['split']} copy={desc['copy']}")


def _sample(n: int, k: int, rng) -> np.ndarray:
    pick = set(rng.choice(n, min(k, n), replace=False).tolist())
    pick.update({0, n - 1, max(0, n - 2)})
    return np.array(sorted(pick), dtype=np.int64)


def _check_sampled(c, op, what, rng):
    """Run op twice (bitwise equal), compare sampled outputs with the oracle."""
    log(what)
    Gt = c.gpu(op, F.OUT_BF16)
    G2 = c.gpu(op, F.OUT_BF16)
    torch.cuda.synchronize()
    assert torch.equal(Gt.view(torch.int16), G2.view(torch.int16)), "not deterministic"
    n_r, n_c = Gt.shape
    # whole sampled rows and whole sampled columns: every tile row and every
    # tile column of the output is touched
    rows, cols = _sample(n_r, 8, rng), _sample(n_c, 8, rng)
    O, S = c.oracle(op, rows, None)
    assert_close(host(Gt[torch.from_numpy(rows).cuda()]), O, S, F.OUT_BF16, what + " rows")
    O, S = c.oracle(op, None, cols)
    assert_close(host(Gt[:, torch.from_numpy(cols).cuda()].contiguous()), O, S, F.OUT_BF16, what + " cols")


FULL = [(2, 1, [(ROW, ROW)]), (2, 2, [(ROW, ROW)]), (2, 3, [(ROW, ROW)]), (2, 4, [(ROW, ROW)]),
        (3, 1, [(ROW, ROW)]), (4, 1, I.ORDER_PAIRS),
        (5, 1, [(ROW, ROW)]), (5, 2, [(ROW, ROW)]), (5, 3, [(ROW, ROW)]), (5, 4, [(ROW, ROW)]),
        (5, 5, [(ROW, ROW)])]


@pytest.mark.parametrize("workload,gemm,orders", FULL,
                         ids=[f"w{w}g{g}" for w, g, _ in FULL])
def test_full_size_sampled(workload, gemm, orders):
    """Full-size shard, tuned plans as in the benchmark, sampled outputs."""
    g = I.WORKLOADS[workload][gemm - 1]
    log(f"workload {workload} gemm {gemm} {g}")
    d = I.make_inputs(workload, gemm)
    rng = np.random.default_rng([workload, gemm])
    for xo, wo in orders:
        c = Case(d, xo, wo)
        F.fc_tune(g.M, g.K, g.N, xo, wo, F.OUT_BF16)
        for op in OPS:
            desc = F.fc_plan_describe(op_code(op), g.M, g.K, g.N, xo, wo, F.OUT_BF16)
            what = (f"w{workload}g{gemm} {op} orders={xo}{wo} {desc['kernel']} split={desc['split']} "
                    f"copy={desc['copy']} pad={desc['pad']}")
            _check_sampled(c, op, what, rng)
        if g.N % 64:
            # backward-data reduces over N, here not a multiple of 64: also force
            # both ring plans (three A tiles and three B tiles), which run the
            # partial last stage themselves, and the first with dY, W or both
            # copied to padded rows (copy bits 1, 2, 3), whatever the tuner picked
            forced = 0
            for pid, copy in ((RING, 0), (RING_B, 0), (RING + 16, 1), (RING + 32, 2), (RING + 48, 3)):
                if F.fc_set_plan(F.OP_BWD_DATA, g.M, g.K, g.N, xo, wo, F.OUT_BF16, pid) != F.FC_OK:
                    continue
                desc = F.fc_plan_describe(F.OP_BWD_DATA, g.M, g.K, g.N, xo, wo, F.OUT_BF16)
                assert desc["ktail"] == g.N % 64 and desc["copy"] == copy, desc
                assert desc["pad"] == (0 if copy == 0 else g.N + 64 - g.N % 64), desc
                assert (desc["ws"] == 0) == (copy == 0), desc
                _check_sampled(c, "bwd_data", f"w{workload}g{gemm} bwd_data forced plan={pid} {desc['kernel']} "
                                              f"ktail={desc['ktail']} copy={copy} pad={desc['pad']}", rng)
                forced += 1
            assert forced == 5, "a ring plan does not apply"
        del c
        torch.cuda.empty_cache()


# -------------------------------------------------------------- ABI on GPU

def test_overlapping_output_rejected_on_device():
    X = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    st = F.lib().fc_fwd(X.data_ptr(), 0, W.data_ptr(), 0, X.data_ptr(), 0, 64, 64, 64, None)
    assert st == F.FC_E_INVALID


def test_binding_rejects_host_output_and_takes_stream_objects():
    """Host outputs are refused; outputs it allocates for a side stream are allocated on that stream."""
    X = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="CUDA/HIP"):
        F.fc_fwd(X, W, out=torch.empty((64, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="CUDA/HIP"):
        F.fc_bwd_weight(X, W, out=torch.empty((64, 64), dtype=torch.bfloat16))
    X1, W1 = X + 1, W + 1
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())  # the operands are written on the current stream
    Y = F.fc_fwd(X1, W1, stream=s)
    Y2 = F.fc_fwd(X1, W1, stream=s.cuda_stream)  # a raw handle works the same
    s.synchronize()
    want = torch.full((64, 64), 64.0, dtype=torch.bfloat16, device="cuda")
    assert torch.equal(Y, want) and torch.equal(Y2, want)


def test_runs_on_a_side_stream_and_tuned_equals_cold_plan_bits():
    M, K, N = 1024, 768, 1280
    d = I.make_random_inputs(M, K, N, seed=5)
    c = Case(d, ROW, ROW)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        cold = c.gpu("fwd", F.OUT_BF16)
    s.synchronize()
    desc = F.fc_plan_describe(F.OP_FWD, M, K, N)
    F.fc_set_plan(F.OP_FWD, M, K, N, ROW, ROW, F.OUT_BF16, desc["plan"])
    warm = c.gpu("fwd", F.OUT_BF16)
    torch.cuda.synchronize()
    assert torch.equal(cold.view(torch.int16), warm.view(torch.int16))
    O, S = c.oracle("fwd")
    assert_close(host(cold), O, S, F.OUT_BF16, "side stream fwd")
