"""Parity of a whole step as the benchmark issues it: every shard product of a
workload (forward layer by layer, then backward-data and backward-weight in
reverse), back to back on one stream with the tuned plans, no host
synchronization in between. In a step, split-K, transpose-copy and
padded-reduction plans take turns on the one workspace, so this checks what
checking each product alone cannot: that no call's staging disturbs
another's.

The step runs twice in a row, its outputs copied on the device between the
two (the copies are queued on the same stream); outputs start as NaN, so an
element no kernel wrote is caught. Then, for every output: no NaN left, the
two steps equal bit for bit, and whole sampled rows and whole sampled
columns within the bound of the oracle (max |G - O| <= 1e-2 S, relative
Frobenius <= 5e-3).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import bench
import oracle
from sharded_fc_layer_amd import fcshard as F
from sharded_fc_layer_amd import inputs as I

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

N_ROWS, N_COLS = 8, 8


def log(msg: str) -> None:
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def _sample(n: int, k: int, rng) -> np.ndarray:
    pick = set(rng.choice(n, min(k, n), replace=False).tolist())
    pick.update({0, n - 1})
    return np.array(sorted(pick), dtype=np.int64)


def _oracle(op, d, g, rows=None, cols=None):
    if op == "fwd":
        return oracle.fc_fwd(d["X"], 0, d["W"], 0, g.M, g.K, g.N, rows, cols)
    if op == "bwd_data":
        return oracle.fc_bwd_data(d["dY"], d["W"], 0, g.M, g.K, g.N, rows, cols)
    return oracle.fc_bwd_weight(d["X"], 0, d["dY"], g.M, g.K, g.N, rows, cols)


def _bits(t) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("workload", [2, 3, 5])
def test_step_as_issued_matches_the_oracle(workload):
    F.fc_release()
    layers = bench.make_layers(workload, torch, F, I, host_inputs=True)
    for L in layers:
        F.fc_tune(L.g.M, L.g.K, L.g.N)
    calls = bench.step_calls(layers)
    outs = {"fwd": lambda L: L.Y, "bwd_data": lambda L: L.dX, "bwd_weight": lambda L: L.dW}
    plans = []
    for L, (opname, op, _) in calls:
        desc = F.fc_plan_describe(op, L.g.M, L.g.K, L.g.N)
        plans.append(f"{L.g.name} {opname}: {desc['kernel']} split={desc['split']} copy={desc['copy']} "
                     f"pad={desc['pad']} ws={desc['ws']}")
        outs[opname](L).view(torch.int16).fill_(-1)  # 0xffff: a bf16 NaN
    log(f"workload {workload}, {len(calls)} calls per step:\n  " + "\n  ".join(plans))
    torch.cuda.synchronize()
    # step 1, device copies of its outputs, step 2: one stream, no host sync
    for _, (_, _, fn) in calls:
        fn()
    first = [outs[opname](L).clone() for L, (opname, _, _) in calls]
    for _, (_, _, fn) in calls:
        fn()
    torch.cuda.synchronize()

    rng = np.random.default_rng([77, workload])
    gi_of = {id(L): gi for gi, L in enumerate(layers, start=1)}
    for (L, (opname, _, _)), out1 in zip(calls, first):
        g = L.g
        out = outs[opname](L)
        what = f"w{workload} {g.name} {opname}"
        assert not bool(torch.isnan(out).any()), f"{what}: elements left unwritten (NaN)"
        assert torch.equal(out.view(torch.int16), out1.view(torch.int16)), f"{what}: the two steps differ"
        d = I.make_inputs(workload, gi_of[id(L)])
        n_r, n_c = out.shape
        rows, cols = _sample(n_r, N_ROWS, rng), _sample(n_c, N_COLS, rng)
        G_rows = I.bf16_bits_to_f32(_bits(out[torch.from_numpy(rows).cuda()]))
        G_cols = I.bf16_bits_to_f32(_bits(out[:, torch.from_numpy(cols).cuda()]))
        for part, G, (r_sel, c_sel) in (("rows", G_rows, (rows, None)), ("cols", G_cols, (None, cols))):
            O, S = _oracle(opname, d, g, r_sel, c_sel)
            c = oracle.compare(G, O, S)
            log(f"  {what} {part} {G.shape}: max_err_ratio={c['max_err_ratio']:.3g} rel_fro={c['rel_fro']:.3g}")
            assert c["pass"], f"{what} sampled {part}: {c}"
        del d
    del layers, first
    torch.cuda.empty_cache()
    F.fc_release()
