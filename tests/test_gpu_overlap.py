"""A shard GEMM with a concurrent copy on a second stream: the output must not
change, and the timings must be consistent."""
from __future__ import annotations

import sys

import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("op", ["fwd", "bwd_data", "bwd_weight"])
def test_gemm_under_a_concurrent_copy(op):
    from sharded_fc_layer_amd import overlap as O
    recs = O.measure(1024, 2048, 1536, op, [16.0, 64.0], reps=3)
    for r in recs:
        print(r, file=sys.stderr, flush=True)
        assert r["output_identical"]
        assert r["gemm_ms"] > 0 and r["copy_ms"] > 0
        # both together take at least as long as the longer of the two, within noise
        assert r["both_ms"] >= 0.8 * max(r["gemm_ms"], r["copy_ms"])
        assert r["hidden_fraction"] <= 1.2


def test_gemm_beside_a_copy_on_reserved_compute_units():
    from sharded_fc_layer_amd import overlap as O
    for r in O.measure(1024, 2048, 1536, "fwd", [16.0], reps=3, copy_cus=8):
        print(r, file=sys.stderr, flush=True)
        assert r["output_identical"] and r["copy_cus"] == 8
        assert r["gemm_all_cus_ms"] > 0 and r["both_ms"] >= 0.8 * max(r["gemm_ms"], r["copy_ms"])
