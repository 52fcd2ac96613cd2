"""A shard GEMM with a concurrent copy on a second stream: the output written
while the copy runs must equal the output alone bit for bit, and both must
match the oracle within the stated bound; the timings must be consistent."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from sharded_fc_layer_amd import inputs as I

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

M, K, N = 1024, 2048, 1536


@pytest.fixture(scope="module")
def seeded():
    """N(0, 1) X, N(0, 0.02) W, N(0, 1e-3) dY and the oracle's three products."""
    d = I.make_random_inputs(M, K, N, seed=12)
    ref = {"fwd": oracle.fc_fwd(d["X"], 0, d["W"], 0, M, K, N),
           "bwd_data": oracle.fc_bwd_data(d["dY"], d["W"], 0, M, K, N),
           "bwd_weight": oracle.fc_bwd_weight(d["X"], 0, d["dY"], M, K, N)}
    return d, ref


def _check_oracle(r, ref, what):
    G = I.bf16_bits_to_f32(r["output"].view(torch.int16).numpy().view(np.uint16))
    O, S = ref
    c = oracle.compare(G, O, S)
    print(f"{what}: max_err_ratio={c['max_err_ratio']:.3g} rel_fro={c['rel_fro']:.3g}", file=sys.stderr, flush=True)
    assert c["pass"], f"{what}: {c}"


@pytest.mark.parametrize("op", ["fwd", "bwd_data", "bwd_weight"])
def test_gemm_under_a_concurrent_copy(op, seeded):
    from sharded_fc_layer_amd import overlap as O
    d, ref = seeded
    recs = O.measure(M, K, N, op, [16.0, 64.0], reps=3, host_inputs=d, return_output=True)
    for r in recs:
        print({k: v for k, v in r.items() if k != "output"}, file=sys.stderr, flush=True)
        assert r["output_identical"]
        _check_oracle(r, ref[op], f"{op} under a {r['copy_MB']} MB copy")
        assert r["gemm_ms"] > 0 and r["copy_ms"] > 0
        # both together take at least as long as the longer of the two, within noise
        assert r["both_ms"] >= 0.8 * max(r["gemm_ms"], r["copy_ms"])
        assert r["hidden_fraction"] <= 1.2


def test_gemm_beside_a_copy_on_reserved_compute_units(seeded):
    from sharded_fc_layer_amd import overlap as O
    d, ref = seeded
    for r in O.measure(M, K, N, "fwd", [16.0], reps=3, copy_cus=8, host_inputs=d, return_output=True):
        print({k: v for k, v in r.items() if k != "output"}, file=sys.stderr, flush=True)
        assert r["output_identical"] and r["copy_cus"] == 8
        _check_oracle(r, ref["fwd"], "fwd beside a copy on 8 reserved compute units")
        assert r["gemm_all_cus_ms"] > 0 and r["both_ms"] >= 0.8 * max(r["gemm_ms"], r["copy_ms"])
