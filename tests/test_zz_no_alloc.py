"""The no-allocation entry point, fc_bwd_weight_noalloc, against the entry
point it varies, fc_bwd_weight: the same plan on the same inputs must give
the same bits, its staging living in the library's static device scratch
instead of the workspace. Two calls in a row, the second on a smaller shape
(so the scratch holds the first call's larger contents when the second
runs), both with split-K plans, which stage fp32 partial planes there; then
the default plan (no staging), and a plan needing more scratch than there is,
which must be refused. Every result is also checked against the oracle on
whole sampled rows and columns. The library must allocate nothing during the
calls: the device's free memory is unchanged across them."""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest

import oracle
from sharded_fc_layer_amd import fcshard as F
from sharded_fc_layer_amd import inputs as I

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _free_bytes() -> int:
    from sharded_fc_layer_amd.overlap import _hip_runtime
    free, total = ctypes.c_size_t(), ctypes.c_size_t()
    assert _hip_runtime().hipMemGetInfo(ctypes.byref(free), ctypes.byref(total)) == 0
    return free.value


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def _plan_with_split(M, K, N, split):
    for pid in range(F.fc_plan_count()):
        if F.fc_set_plan(F.OP_BWD_WEIGHT, M, K, N, 0, 0, 0, pid) != F.FC_OK:
            continue
        d = F.fc_plan_describe(F.OP_BWD_WEIGHT, M, K, N)
        if d["split"] == split and d["copy"] == 0 and d["pad"] == 0:
            return pid, d
    return None, None


def _check_oracle(dW, d, M, K, N, what):
    rng = np.random.default_rng([21, M, K, N])
    rows = np.unique(np.r_[0, K - 1, rng.choice(K, 6, replace=False)])
    cols = np.unique(np.r_[0, N - 1, rng.choice(N, 6, replace=False)])
    for part, (r, c) in (("rows", (rows, None)), ("cols", (None, cols))):
        O, S = oracle.fc_bwd_weight(d["X"], 0, d["dY"], M, K, N, r, c)
        G = dW[torch.from_numpy(rows).cuda()] if c is None else dW[:, torch.from_numpy(cols).cuda()]
        Gv = I.bf16_bits_to_f32(G.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
        res = oracle.compare(Gv, O, S)
        log(f"  {what} {part}: max_err_ratio={res['max_err_ratio']:.3g} rel_fro={res['rel_fro']:.3g}")
        assert res["pass"], f"{what} {part}: {res}"


def test_noalloc_matches_bwd_weight_on_two_calls_then_refuses_too_large():
    F.fc_release()
    cap = F.fc_noalloc_scratch_bytes()
    assert cap == 64 << 20
    # first call: the attention-out backward-weight of the GPT block (2048 x
    # 2048 output, 8192 tokens), split 4: its partial planes fill the scratch
    # exactly; second call: a smaller shape, split 2
    cases = [((8192, 2048, 2048), 4), ((1024, 512, 768), 2)]
    prepared = []
    for (M, K, N), split in cases:
        pid, desc = _plan_with_split(M, K, N, split)
        assert pid is not None, f"no split-{split} plan for {(M, K, N)}"
        assert 0 < desc["ws"] <= cap, desc
        d = I.make_random_inputs(M, K, N, seed=20 + split)
        X, dY = _dev(d["X"]), _dev(d["dY"])
        ref = F.fc_bwd_weight(X, dY)  # the existing entry point, the workspace
        out = torch.empty((K, N), dtype=torch.bfloat16, device="cuda")
        prepared.append(((M, K, N), desc, d, X, dY, ref, out))
    # set-up: the first call on the device looks up the scratch array's
    # address (the runtime loads the code object that holds it); its output
    # is overwritten below
    _, _, _, X, dY, _, out = prepared[1]
    F.fc_bwd_weight_noalloc(X, dY, out=out)
    for *_, out in prepared:
        out.view(torch.int16).fill_(-1)
    torch.cuda.synchronize()
    free0 = _free_bytes()
    for (M, K, N), desc, d, X, dY, ref, out in prepared:
        log(f"noalloc {(M, K, N)} plan={desc['plan']} {desc['kernel']} split={desc['split']} ws={desc['ws']}")
        F.fc_bwd_weight_noalloc(X, dY, out=out)
        torch.cuda.synchronize()
    assert _free_bytes() == free0, "device memory was allocated during the no-allocation calls"
    for (M, K, N), desc, d, X, dY, ref, out in prepared:
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{(M, K, N)}: differs from fc_bwd_weight"
        _check_oracle(out, d, M, K, N, f"noalloc {(M, K, N)}")
    # the default plan (no staging) at an untuned key
    M, K, N = 520, 264, 136
    d = I.make_random_inputs(M, K, N, seed=24)
    X, dY = _dev(d["X"]), _dev(d["dY"])
    ref = F.fc_bwd_weight(X, dY)
    out = F.fc_bwd_weight_noalloc(X, dY)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    # a plan needing more scratch than there is: refused, output untouched
    M, K, N = 4096, 4096, 4096
    pid, desc = _plan_with_split(M, K, N, 4)
    assert pid is not None and desc["ws"] > cap
    X = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    dY = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    out = torch.full((K, N), 3.0, dtype=torch.bfloat16, device="cuda")
    st = F.lib().fc_bwd_weight_noalloc(X.data_ptr(), 0, dY.data_ptr(), out.data_ptr(), 0, M, K, N, None)
    assert st == F.FC_E_TOO_LARGE, F.status_str(st)
    assert "scratch" in F.status_str(st)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
    F.fc_release()
