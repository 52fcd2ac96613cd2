"""Seeded random sweep of the plan space, exact against the oracle.

Each case draws a shape (dimensions from 1 to 2600, aligned or ragged), a
product, storage orders, an output type (bf16, fp32, or fp32 added into an
existing output) and a plan that applies to it from the whole plan space;
the output must equal the oracle's exactly (integer-valued inputs make
every fp32 partial sum exact in any order), run twice with the same bits,
and the default plan (no plan set) must be exact too."""
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
OPS = {"fwd": F.OP_FWD, "bwd_data": F.OP_BWD_DATA, "bwd_weight": F.OP_BWD_WEIGHT}
N_CASES = 160


def log(msg: str) -> None:
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def dev(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def host(t) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _dim(rng) -> int:
    u = rng.random()
    if u < 0.3:
        return int(rng.integers(1, 81))
    if u < 0.7:
        return int(rng.integers(80, 701))
    v = int(rng.integers(700, 2601))
    return v - v % 8 if rng.random() < 0.5 else v  # aligned or ragged


def _cases():
    rng = np.random.default_rng(20261202)
    cases = []
    while len(cases) < N_CASES:
        M, K, N = _dim(rng), _dim(rng), _dim(rng)
        if M * K * N > 3_000_000_000:
            continue
        op = list(OPS)[int(rng.integers(0, 3))]
        xo, wo = int(rng.integers(0, 2)), int(rng.integers(0, 2))
        dt = [F.OUT_BF16, F.OUT_F32, F.OUT_F32_ACC][int(rng.integers(0, 3))]
        cases.append((len(cases), M, K, N, op, xo, wo, dt, int(rng.integers(0, 1 << 30))))
    return cases


def _run(op, X, W, dY, xo, wo, dt, C_old):
    out = None if dt != F.OUT_F32_ACC else torch.from_numpy(C_old.copy()).to("cuda")
    if op == "fwd":
        r = F.fc_fwd(X, W, xo, wo, out=out, out_dtype=dt)
    elif op == "bwd_data":
        r = F.fc_bwd_data(dY, W, wo, out=out, out_dtype=dt)
    else:
        r = F.fc_bwd_weight(X, dY, xo, out=out, out_dtype=dt)
    return host(r)


@pytest.fixture(autouse=True)
def _clean_plans():
    yield
    torch.cuda.synchronize()
    F.fc_release()


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}-{c[4]}-{c[1]}x{c[2]}x{c[3]}")
def test_random_plan_exact(case):
    idx, M, K, N, op, xo, wo, dt, seed = case
    d = I.make_integer_inputs(M, K, N, seed=seed % 100000)
    X, W, dY = dev(I.stored(d["X"], xo)), dev(I.stored(d["W"], wo)), dev(d["dY"])
    if op == "fwd":
        O, S = oracle.fc_fwd(I.stored(d["X"], xo), xo, I.stored(d["W"], wo), wo, M, K, N)
    elif op == "bwd_data":
        O, S = oracle.fc_bwd_data(d["dY"], I.stored(d["W"], wo), wo, M, K, N)
    else:
        O, S = oracle.fc_bwd_weight(I.stored(d["X"], xo), xo, d["dY"], M, K, N)
    rng = np.random.default_rng(seed)
    C_old = rng.integers(-64, 65, size=O.shape).astype(np.float32) if dt == F.OUT_F32_ACC else None
    want = oracle.accumulate(C_old, O, S)[0] if C_old is not None else O
    if dt == F.OUT_BF16:
        want_bits = oracle.round_bf16(want)
    else:
        w32 = want.astype(np.float32)
        assert np.array_equal(w32.astype(np.float64), want), "oracle value not exact in fp32"
        want_bits = w32.view(np.uint32)

    def check(G, what):
        got = G if dt == F.OUT_BF16 else G.view(np.uint32)
        bad = np.argwhere(got != want_bits)
        assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}"

    # the default plan (nothing set)
    base = f"case {idx}: {op} {M}x{K}x{N} orders={xo}{wo} dtype={dt}"
    log(f"{base} default plan {F.fc_plan_describe(OPS[op], M, K, N, xo, wo, dt)['kernel']}")
    check(_run(op, X, W, dY, xo, wo, dt, C_old), base + " default plan")
    # a random plan that applies
    pids = rng.permutation(F.fc_plan_count())
    pid = next((int(p) for p in pids if F.fc_set_plan(OPS[op], M, K, N, xo, wo, dt, int(p)) == F.FC_OK), None)
    assert pid is not None, base + ": no plan applies"
    desc = F.fc_plan_describe(OPS[op], M, K, N, xo, wo, dt)
    what = f"{base} plan={pid} {desc['kernel']} split={desc['split']} copy={desc['copy']} pad={desc['pad']}" + \
           (f" tail={desc['tail']}" if "tail" in desc else "")
    log(what)
    G1 = _run(op, X, W, dY, xo, wo, dt, C_old)
    G2 = _run(op, X, W, dY, xo, wo, dt, C_old)
    torch.cuda.synchronize()
    check(G1, what)
    assert np.array_equal(G1, G2), what + ": two runs differ"
