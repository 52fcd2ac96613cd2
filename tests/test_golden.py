"""The oracle against a hand-computed worked example (CPU).

tests/golden/fc_shard_worked_example.txt holds a 2 x 3 x 2 shard: inputs exact
in bf16, and the three products (sciencestack.ai/paper/2502.08145, Figure 1)
with their tolerance scales, worked out by hand with every term written beside
its element. The oracle must reproduce each value exactly in every storage
order of X and W, and a copy of the oracle with a planted product mistake must
not.
"""
from __future__ import annotations

import os
import tempfile

import numpy as np
import pytest

import oracle
from sharded_fc_layer_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fc_shard_worked_example.txt")


def load(path: str) -> dict:
    mats, name, rows, cur = {}, None, 0, []
    for line in open(path):
        t = line.split("#")[0].split()
        if not t:
            continue
        if name is None:
            name, rows, cur = t[0], int(t[1]), []
            cols = int(t[2])
            continue
        assert len(t) == cols, f"{name}: row of {len(t)} values, expected {cols}"
        cur.append([float(v) for v in t])
        if len(cur) == rows:
            mats[name] = np.array(cur, dtype=np.float64)
            name = None
    assert name is None, f"{name} is incomplete"
    return mats


G = load(GOLDEN)


def bits(a: np.ndarray) -> np.ndarray:
    b = I.f32_to_bf16_bits(a.astype(np.float32))
    assert np.array_equal(I.bf16_bits_to_f32(b).astype(np.float64), a), "fixture input not exact in bf16"
    return b


def test_fixture_is_complete():
    assert set(G) == {"X", "W", "dY", "Y", "S_Y", "dX", "S_dX", "dW", "S_dW"}
    M, K = G["X"].shape
    N = G["W"].shape[1]
    assert G["W"].shape == (K, N) and G["dY"].shape == (M, N)
    assert G["Y"].shape == (M, N) and G["dX"].shape == (M, K) and G["dW"].shape == (K, N)


def golden_ok(orc, xo: int, wo: int) -> bool:
    """True when the oracle library `orc` reproduces every value of the example."""
    M, K = G["X"].shape
    N = G["W"].shape[1]
    X, W, dY = bits(G["X"]), bits(G["W"]), bits(G["dY"])
    Xs, Ws = I.stored(X, xo), I.stored(W, wo)
    Y, SY = orc.fc_fwd(Xs, xo, Ws, wo, M, K, N)
    dX, SdX = orc.fc_bwd_data(np.ascontiguousarray(dY), Ws, wo, M, K, N)
    dW, SdW = orc.fc_bwd_weight(Xs, xo, np.ascontiguousarray(dY), M, K, N)
    got = {"Y": Y, "S_Y": SY, "dX": dX, "S_dX": SdX, "dW": dW, "S_dW": SdW}
    return all(np.array_equal(v, G[k]) for k, v in got.items())


@pytest.mark.parametrize("xo", [I.ROW, I.COL])
@pytest.mark.parametrize("wo", [I.ROW, I.COL])
def test_oracle_reproduces_the_worked_example(xo, wo):
    assert golden_ok(oracle.default(), xo, wo)


# the product mistakes planted in the oracle's source by the pin tests
PRODUCT_MUTANTS = ["drop_last_term", "untransposed_w_in_bwd_data", "wrong_col_major_stride", "signed_scale",
                   "sign_flip"]


@pytest.mark.parametrize("name", PRODUCT_MUTANTS)
def test_worked_example_rejects_planted_mistake(name):
    from test_oracle_pins import MUTANTS
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        mut = oracle.Oracle(oracle.build(True, path, os.path.join(td, "libmutant.so")))
        assert not all(golden_ok(mut, xo, wo) for xo in (I.ROW, I.COL) for wo in (I.ROW, I.COL)), name
