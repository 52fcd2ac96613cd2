"""Pins of the CPU oracle to facts outside itself (CPU only).

The oracle computes the plain products of one FC layer's shard
(sciencestack.ai/paper/2502.08145, Figure 1) in fp64 over bf16 inputs. The
pages print no worked numbers, so the oracle is pinned to:

* exact rational brute force (fractions.Fraction) on tiny shapes, every
  storage order and every op;
* closed forms: identity, power-of-two diagonal, permutation, all-ones, zero;
* invariants: dW . 1 = X^T (dY . 1), 1^T Y = (1^T X) W, explicit-transpose
  equivalences, scaling and additivity, sampled = full;
* a library fp64 product (numpy.matmul) on the workload shapes;
* the virtual-grid split reassembling the unsharded product
  (pith.science/paper/2502.08145, "What carries the argument"; "If this is
  right": single-axis grids reduce to FSDP / tensor-parallel splits);
* the bf16 output rounding against exhaustive and brute-force references.

The planted-mistake tests at the end rebuild the oracle from a mutated copy of
its source and check that these pins reject every mutant.
"""
from __future__ import annotations

import math
import os
import tempfile
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import grid
from sharded_fc_layer_amd import inputs as I

ROW, COL = I.ROW, I.COL
U53 = 2.0 ** -53


def vals(bits: np.ndarray) -> np.ndarray:
    """fp64 values of bf16 bits via the input module's decoder (not the oracle's)."""
    return I.bf16_bits_to_f32(bits).astype(np.float64)


def logical_operands(op: str, d: dict):
    """Logical operands (A, B) of C = A . B for each op, as fp64 arrays."""
    X, W, dY = vals(d["X"]), vals(d["W"]), vals(d["dY"])
    if op == "fwd":
        return X, W
    if op == "bwd_data":
        return dY, W.T
    if op == "bwd_weight":
        return X.T, dY
    raise ValueError(op)


def run_oracle(orc, op: str, d: dict, xo: int, wo: int, rows=None, cols=None):
    M, K = d["X"].shape
    N = d["W"].shape[1]
    Xs, Ws = I.stored(d["X"], xo), I.stored(d["W"], wo)
    if op == "fwd":
        return orc.fc_fwd(Xs, xo, Ws, wo, M, K, N, rows, cols)
    if op == "bwd_data":
        return orc.fc_bwd_data(np.ascontiguousarray(d["dY"]), Ws, wo, M, K, N, rows, cols)
    return orc.fc_bwd_weight(Xs, xo, np.ascontiguousarray(d["dY"]), M, K, N, rows, cols)


def exact_product(A: np.ndarray, B: np.ndarray):
    """Exact rational C = A . B and S = |A| . |B| (as Fractions)."""
    R = A.shape[1]
    Af = [[Fraction(float(v)) for v in row] for row in A]
    Bf = [[Fraction(float(v)) for v in row] for row in B]
    C = [[sum((Af[i][r] * Bf[r][j] for r in range(R)), Fraction(0)) for j in range(B.shape[1])]
         for i in range(A.shape[0])]
    S = [[sum((abs(Af[i][r] * Bf[r][j]) for r in range(R)), Fraction(0)) for j in range(B.shape[1])]
         for i in range(A.shape[0])]
    return C, S


OPS = ["fwd", "bwd_data", "bwd_weight"]
ORDERS = [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)]
TINY = [(1, 1, 1), (1, 2, 3), (2, 3, 5), (3, 5, 8), (5, 8, 17), (8, 17, 3), (17, 3, 33),
        (33, 1, 2), (2, 33, 1), (7, 33, 17)]


def brute_force_ok(orc, shapes=TINY, seed=0) -> bool:
    """Every op x order x shape within 2 R u S of the exact rational result."""
    for (M, K, N) in shapes:
        d = I.make_random_inputs(M, K, N, seed=seed, sx=1.0, sw=0.5, sdy=2.0)
        for op in OPS:
            A, B = logical_operands(op, d)
            C, S = exact_product(A, B)
            R = A.shape[1]
            for xo, wo in ORDERS:
                O, So = run_oracle(orc, op, d, xo, wo)
                for i in range(A.shape[0]):
                    for j in range(B.shape[1]):
                        s = float(S[i][j])
                        if abs(Fraction(float(O[i, j])) - C[i][j]) > Fraction(2 * R * U53) * S[i][j]:
                            return False
                        if abs(So[i, j] - s) > 2 * R * U53 * s:
                            return False
    return True


def test_brute_force_exact_rational():
    assert brute_force_ok(oracle.default())


# ---------------------------------------------------------------- closed forms

def test_identity_weight_reproduces_input():
    for M, K in [(5, 7), (16, 16), (33, 9)]:
        d = I.make_random_inputs(M, K, K, seed=1)
        d["W"] = I.f32_to_bf16_bits(np.eye(K, dtype=np.float32))
        for xo, wo in ORDERS:
            Y, S = run_oracle(oracle.default(), "fwd", d, xo, wo)
            assert np.array_equal(Y, vals(d["X"]))
            assert np.array_equal(S, np.abs(vals(d["X"])))
        # dX = dY . I^T = dY
        d2 = I.make_random_inputs(M, K, K, seed=2)
        d2["W"] = I.f32_to_bf16_bits(np.eye(K, dtype=np.float32))
        for wo in (ROW, COL):
            dX, _ = run_oracle(oracle.default(), "bwd_data", d2, ROW, wo)
            assert np.array_equal(dX, vals(d2["dY"]))


def test_identity_input_gives_weight_gradient_dy():
    M = K = 12
    d = I.make_random_inputs(M, K, 9, seed=3)
    d["X"] = I.f32_to_bf16_bits(np.eye(M, dtype=np.float32))
    for xo in (ROW, COL):
        dW, _ = run_oracle(oracle.default(), "bwd_weight", d, xo, ROW)
        assert np.array_equal(dW, vals(d["dY"]))


def test_power_of_two_diagonal_scales_columns():
    K = 11
    d = I.make_random_inputs(6, K, K, seed=4)
    e = np.arange(K) - 5
    d["W"] = I.f32_to_bf16_bits(np.diag(2.0 ** e).astype(np.float32))
    for xo, wo in ORDERS:
        Y, _ = run_oracle(oracle.default(), "fwd", d, xo, wo)
        assert np.array_equal(Y, vals(d["X"]) * (2.0 ** e)[None, :])


def test_permutation_weight_permutes_columns():
    K = 10
    rng = np.random.default_rng(5)
    p = rng.permutation(K)
    P = np.zeros((K, K), dtype=np.float32)
    P[p, np.arange(K)] = 1.0  # W[p[j], j] = 1  ->  Y[:, j] = X[:, p[j]]
    d = I.make_random_inputs(7, K, K, seed=5)
    d["W"] = I.f32_to_bf16_bits(P)
    for xo, wo in ORDERS:
        Y, _ = run_oracle(oracle.default(), "fwd", d, xo, wo)
        assert np.array_equal(Y, vals(d["X"])[:, p])


def test_all_ones_weight_gives_row_sums():
    d = I.make_random_inputs(9, 40, 3, seed=6)
    d["W"] = I.f32_to_bf16_bits(np.ones((40, 3), dtype=np.float32))
    Y, _ = run_oracle(oracle.default(), "fwd", d, ROW, ROW)
    X = vals(d["X"])
    for i in range(9):
        # bf16 values span few binades: every partial sum is exact in fp64
        assert np.all(Y[i] == math.fsum(X[i]))


def test_zero_in_zero_out():
    d = I.make_random_inputs(4, 6, 5, seed=7)
    d["X"] = np.zeros_like(d["X"])
    for op in ("fwd", "bwd_weight"):
        O, S = run_oracle(oracle.default(), op, d, ROW, ROW)
        assert not O.any() and not S.any()


def test_scale_equals_value_for_nonnegative_inputs():
    d = I.make_random_inputs(8, 9, 10, seed=8)
    for k in d:
        d[k] = d[k] & np.uint16(0x7FFF)  # clear the sign bits
    for op in OPS:
        O, S = run_oracle(oracle.default(), op, d, ROW, ROW)
        assert np.array_equal(O, S)


# ------------------------------------------------------------------ invariants

def test_weight_gradient_row_sum_invariant():
    """dW . 1_N = X^T (dY . 1_N)."""
    M, K, N = 64, 48, 40
    d = I.make_random_inputs(M, K, N, seed=9)
    X, dY = vals(d["X"]), vals(d["dY"])
    for xo in (ROW, COL):
        dW, _ = run_oracle(oracle.default(), "bwd_weight", d, xo, ROW)
        lhs = np.array([math.fsum(r) for r in dW])
        rhs = X.T @ np.array([math.fsum(r) for r in dY])
        scale = np.abs(X).T @ np.abs(dY).sum(1)
        assert np.all(np.abs(lhs - rhs) <= 1e-12 * scale)


def test_forward_column_sum_invariant():
    """1_M^T Y = (1_M^T X) W."""
    M, K, N = 50, 30, 44
    d = I.make_random_inputs(M, K, N, seed=10)
    X, W = vals(d["X"]), vals(d["W"])
    for xo, wo in ORDERS:
        Y, _ = run_oracle(oracle.default(), "fwd", d, xo, wo)
        lhs = np.array([math.fsum(c) for c in Y.T])
        rhs = np.array([math.fsum(c) for c in X.T]) @ W
        scale = np.abs(X).sum(0) @ np.abs(W)
        assert np.all(np.abs(lhs - rhs) <= 1e-12 * scale)


def test_backward_ops_equal_forward_of_explicit_transposes():
    """dX = fwd(dY, W^T) and dW = fwd(X^T, dY), bit for bit."""
    M, K, N = 13, 21, 17
    d = I.make_random_inputs(M, K, N, seed=11)
    orc = oracle.default()
    WT = np.ascontiguousarray(d["W"].T)
    XT = np.ascontiguousarray(d["X"].T)
    for wo in (ROW, COL):
        dX, S1 = run_oracle(orc, "bwd_data", d, ROW, wo)
        Y, S2 = orc.fc_fwd(np.ascontiguousarray(d["dY"]), ROW, I.stored(WT, wo), wo, M, N, K)
        assert np.array_equal(dX, Y) and np.array_equal(S1, S2)
    for xo in (ROW, COL):
        dW, S1 = run_oracle(orc, "bwd_weight", d, xo, ROW)
        Y, S2 = orc.fc_fwd(I.stored(XT, xo), xo, np.ascontiguousarray(d["dY"]), ROW, K, M, N)
        assert np.array_equal(dW, Y) and np.array_equal(S1, S2)


def test_scaling_and_additivity():
    M, K, N = 9, 14, 6
    orc = oracle.default()
    d = I.make_integer_inputs(M, K, N, seed=12)
    Y, _ = run_oracle(orc, "fwd", d, ROW, ROW)
    d4 = dict(d)
    d4["X"] = I.f32_to_bf16_bits(vals(d["X"]).astype(np.float32) * 4)
    Y4, _ = run_oracle(orc, "fwd", d4, ROW, ROW)
    assert np.array_equal(Y4, 4 * Y)
    d2 = I.make_integer_inputs(M, K, N, seed=13)
    dsum = dict(d)
    dsum["W"] = I.f32_to_bf16_bits((vals(d["W"]) + vals(d2["W"])).astype(np.float32))
    Y2, _ = run_oracle(orc, "fwd", {**d, "W": d2["W"]}, ROW, ROW)
    Ys, _ = run_oracle(orc, "fwd", dsum, ROW, ROW)
    assert np.array_equal(Ys, Y + Y2)


def test_sampled_outputs_equal_full_outputs():
    M, K, N = 37, 29, 41
    d = I.make_random_inputs(M, K, N, seed=14)
    rows = [0, 5, 36, 17]
    for op in OPS:
        n_r = {"fwd": M, "bwd_data": M, "bwd_weight": K}[op]
        n_c = {"fwd": N, "bwd_data": K, "bwd_weight": N}[op]
        cols = [n_c - 1, 0, 3]
        rr = [r % n_r for r in rows]
        for xo, wo in ORDERS:
            O, S = run_oracle(oracle.default(), op, d, xo, wo)
            Os, Ss = run_oracle(oracle.default(), op, d, xo, wo, rr, cols)
            assert np.array_equal(Os, O[np.ix_(rr, cols)]) and np.array_equal(Ss, S[np.ix_(rr, cols)])


# ------------------------------------------------------- library fp64 product

def _operand_slices(op, d, rows, cols):
    """fp64 values of the selected rows of A and columns of B (A . B = the op)."""
    X, W, dY = d["X"], d["W"], d["dY"]
    if op == "fwd":
        return vals(X[rows, :]), vals(W[:, cols])
    if op == "bwd_data":
        return vals(dY[rows, :]), vals(W[cols, :]).T
    return vals(X[:, rows]).T, vals(dY[:, cols])


def _library_check(d, op, xo, wo, rows=None, cols=None):
    M, K = d["X"].shape
    N = d["W"].shape[1]
    n_r = K if op == "bwd_weight" else M
    n_c = K if op == "bwd_data" else N
    rows = np.arange(n_r) if rows is None else np.asarray(rows)
    cols = np.arange(n_c) if cols is None else np.asarray(cols)
    O, S = run_oracle(oracle.default(), op, d, xo, wo, rows, cols)
    Asel, B = _operand_slices(op, d, rows, cols)
    ref = np.matmul(Asel, B)
    R = Asel.shape[1]
    assert np.all(np.abs(O - ref) <= 4 * R * U53 * S)
    assert np.all(np.abs(S - np.matmul(np.abs(Asel), np.abs(B))) <= 4 * R * U53 * S)


def test_library_product_workload1_full():
    d = I.make_inputs(1, 1)
    for op in OPS:
        for xo, wo in ORDERS:
            _library_check(d, op, xo, wo)


@pytest.mark.slow
@pytest.mark.parametrize("workload,gemm", [(2, 1), (2, 4), (4, 1), (3, 1)])
def test_library_product_workload_rows(workload, gemm):
    d = I.make_inputs(workload, gemm)
    g = I.WORKLOADS[workload][gemm - 1]
    rng = np.random.default_rng(0)
    orders = I.ORDER_PAIRS if workload == 4 else [(ROW, ROW)]
    for op in OPS:
        n_r = g.K if op == "bwd_weight" else g.M
        n_c = g.K if op == "bwd_data" else g.N
        rows = np.sort(rng.choice(n_r, 8, replace=False))
        cols = np.sort(rng.choice(n_c, 256, replace=False))
        for xo, wo in orders:
            _library_check(d, op, xo, wo, rows, cols)


# -------------------------------------------------------- virtual-grid split

def test_workload_shard_shapes_follow_the_grid_reading():
    # hidden 12288, FFN 49152, 16384 tokens on 2x2x2 -> the 8192 x 6144 x 24576 shard
    assert grid.shard_shapes(16384, 12288, 49152, (2, 2, 2)) == {"M": 8192, "K": 6144, "N": 24576}
    g = I.WORKLOADS[3][0]
    assert (g.M, g.K, g.N) == (8192, 6144, 24576)
    # hidden 16384, FFN 53248 at Gx = Gy = 8 -> 2048 x 6656
    assert grid.shard_shapes(8192, 16384, 53248, (8, 8, 1)) == {"M": 8192, "K": 2048, "N": 6656}
    # 405B-like layer on 2x4x2: QKV, out-proj, up, down
    w5 = {g.name: (g.M, g.K, g.N) for g in I.WORKLOADS[5]}
    assert w5["qkv"] == tuple(grid.shard_shapes(16384, 16384, 3 * 16384, (2, 4, 2)).values())
    assert w5["out_proj"] == tuple(grid.shard_shapes(16384, 16384, 16384, (2, 4, 2)).values())
    assert w5["mlp_up"] == tuple(grid.shard_shapes(16384, 16384, 53248, (2, 4, 2)).values())
    assert w5["mlp_down"] == tuple(grid.shard_shapes(16384, 53248, 16384, (2, 4, 2)).values())


def _grid_vs_full(d, g, exact):
    M, K = d["X"].shape
    N = d["W"].shape[1]
    sim = grid.simulate_layer(d["X"], d["W"], d["dY"], g)
    orc = oracle.default()
    full = {"Y": run_oracle(orc, "fwd", d, ROW, ROW), "dX": run_oracle(orc, "bwd_data", d, ROW, ROW),
            "dW": run_oracle(orc, "bwd_weight", d, ROW, ROW)}
    for k, (O, S) in full.items():
        if exact:
            assert np.array_equal(sim[k], O), k
        else:
            assert np.all(np.abs(sim[k] - O) <= 1e-12 * S), k
        R = {"Y": K, "dX": N, "dW": M}[k]
        assert np.all(np.abs(sim["S_" + k] - S) <= 4 * R * U53 * S)
    return sim


def test_grid_2x2x2_workload1_integer_exact():
    g = I.WORKLOADS[1][0]
    d = I.make_integer_inputs(g.M, g.K, g.N, seed=0)
    sim = _grid_vs_full(d, (2, 2, 2), exact=True)
    assert sim["ranks"][(1, 1, 1)] == {"X": (128, 256), "W": (256, 1024), "W_piece": (128, 1024),
                                       "dY": (128, 1024)}


def test_grid_2x2x2_workload1_seeded():
    _grid_vs_full(I.make_inputs(1, 1), (2, 2, 2), exact=False)


@pytest.mark.parametrize("g", [(1, 1, 2), (1, 2, 1), (2, 1, 1), (3, 2, 2), (1, 1, 1)])
def test_grid_single_axis_and_uneven(g):
    d = I.make_integer_inputs(7, 9, 5, seed=1)
    _grid_vs_full(d, g, exact=True)
    _grid_vs_full(I.make_random_inputs(11, 10, 13, seed=2), g, exact=False)


# ------------------------------------------ accumulating output (micro-batches)

def _micro_batches(d, cuts, orc):
    M, K = d["X"].shape
    N = d["dY"].shape[1]
    C = np.zeros((K, N), dtype=np.float32)
    S = np.zeros((K, N))
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        X1, dY1 = np.ascontiguousarray(d["X"][lo:hi]), np.ascontiguousarray(d["dY"][lo:hi])
        P, S1 = orc.fc_bwd_weight(X1, ROW, dY1, hi - lo, K, N)
        V, S = oracle.accumulate(C, P, S1)
        C = V.astype(np.float32)
    return V, S


def test_accumulated_micro_batches_equal_the_whole_batch():
    # dW = X^T dY sums over tokens, so adding the micro-batches' products into
    # one output gives the whole batch's product (exact on integer data)
    orc = oracle.default()
    d = I.make_integer_inputs(24, 10, 7, seed=5)
    full, S_full = run_oracle(orc, "bwd_weight", d, ROW, ROW)
    V, S = _micro_batches(d, [0, 9, 16, 24], orc)
    assert np.array_equal(V, full)
    assert np.all(S <= S_full)  # |partial sums| never exceed the sums of |terms|
    d = I.make_random_inputs(40, 12, 9, seed=6)
    full, S_full = run_oracle(orc, "bwd_weight", d, ROW, ROW)
    V, _ = _micro_batches(d, [0, 13, 40], orc)
    # fp32 storage of the running sum between micro-batches: half an ulp of fp32
    assert np.all(np.abs(V - full) <= 2.0 ** -23 * S_full + 1e-12 * S_full)


def test_accumulate_identities():
    rng = np.random.default_rng(0)
    C = rng.standard_normal((5, 6)).astype(np.float32)
    P = rng.standard_normal((5, 6))
    S = np.abs(P) + 1.0
    V, S2 = oracle.accumulate(C, np.zeros_like(P), np.zeros_like(S))
    assert np.array_equal(V, C.astype(np.float64)) and np.array_equal(S2, np.abs(C).astype(np.float64))
    V, S2 = oracle.accumulate(np.zeros((5, 6), dtype=np.float32), P, S)
    assert np.array_equal(V, P) and np.array_equal(S2, S)


# ------------------------------------------------------------- bf16 rounding

def _nearest_even_bf16(v: float) -> int:
    """Brute force: the nearest bf16 to v, ties to the even pattern."""
    if v == 0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    f32 = np.array([v], dtype=np.float32).view(np.uint32)[0]
    c = int(f32 >> 16)
    best = None
    for b in range(max(c - 2, 0), min(c + 3, 0xFFFF) + 1):
        if (b & 0x7F80) == 0x7F80:
            continue
        bv = Fraction(float(I.bf16_bits_to_f32(np.array([b], dtype=np.uint16))[0]))
        if (bv < 0) != (v < 0) and bv != 0:
            continue
        dist = abs(bv - Fraction(v))
        key = (dist, b & 1)
        if best is None or key < best[0]:
            best = (key, b)
    return best[1]


def round_ok(orc) -> bool:
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = allbits[(allbits & 0x7F80) != 0x7F80]
    if not np.array_equal(orc.round_bf16(vals(finite)), finite):
        return False
    # midpoints between neighbours tie to the even pattern
    pos = finite[(finite < 0x7F7F) & (finite > 0)]
    lo, hi = vals(pos), vals(pos + 1)
    mid = (lo + hi) / 2
    want = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint16)
    if not np.array_equal(orc.round_bf16(mid), want):
        return False
    rng = np.random.default_rng(15)
    v = rng.standard_normal(400) * np.exp2(rng.integers(-30, 30, 400))
    got = orc.round_bf16(v)
    return all(int(g) == _nearest_even_bf16(float(x)) for g, x in zip(got, v))


def test_round_bf16_pins():
    assert round_ok(oracle.default())
    r = oracle.default().round_bf16(np.array([1e39, -1e39, 3.3895313892515355e38]))
    assert list(r) == [0x7F80, 0xFF80, 0x7F7F]


# ------------------------------------------------- planted mistakes (CPU only)

MUTANTS = {
    "drop_last_term": ("        for (int64_t r = 0; r < R; ++r) {\n            const double x",
                       "        for (int64_t r = 0; r < R - 1; ++r) {\n            const double x"),
    "untransposed_w_in_bwd_data": ("const int wt_order = (w_order == ORDER_ROW) ? ORDER_COL : ORDER_ROW;",
                                   "const int wt_order = w_order;"),
    "wrong_col_major_stride": ("p[j * R + i]", "p[j * C + i]"),
    "signed_scale": ("s[b] += ax * fabs(brow[b]);", "s[b] += ax * brow[b];"),
    "ties_away_from_zero": ("nearbyint(ldexp(a, -qexp))", "round(ldexp(a, -qexp))"),
    "sign_flip": ("o[b] += x * brow[b];", "o[b] -= x * brow[b];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        mut = oracle.Oracle(oracle.build(True, path, os.path.join(td, "libmutant.so")))
        small = [(2, 3, 5), (5, 8, 3), (3, 4, 3)]
        assert not (brute_force_ok(mut, small) and round_ok(mut)), name
