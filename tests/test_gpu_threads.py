"""Hot calls from one host thread while another thread grows the library's
workspace (fc_set_plan for ever larger split-K shapes). A growth synchronizes
the device and then frees the old workspace; a hot call keeps the plan-cache
lock from reading the workspace pointer until its kernels are enqueued, so no
kernel is handed a workspace that is freed before it runs. Every output of the
split-K plan must equal that plan's output before the growth began, bit for bit.
"""
from __future__ import annotations

import threading

import pytest

from sharded_fc_layer_amd import fcshard as F

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _plan_with(op, M, K, N, split, copy):
    """The first applicable plan id with this split and copy arm."""
    for pid in range(F.fc_plan_count()):
        if F.fc_set_plan(op, M, K, N, 0, 0, 0, pid) != F.FC_OK:
            continue
        d = F.fc_plan_describe(op, M, K, N)
        if d["split"] == split and d["copy"] == copy:
            return pid
    return None


def test_hot_calls_beside_workspace_growth():
    F.fc_release()
    M, K, N = 512, 1024, 512
    pid = _plan_with(F.OP_FWD, M, K, N, 2, 0)
    assert pid is not None
    assert F.fc_set_plan(F.OP_FWD, M, K, N, 0, 0, 0, pid) == F.FC_OK
    assert F.fc_plan_describe(F.OP_FWD, M, K, N)["ws"] > 0
    KG, NG = 1024, 2048
    pid_grow = _plan_with(F.OP_FWD, 1024, KG, NG, 4, 0)
    assert pid_grow is not None

    g = torch.Generator(device="cuda").manual_seed(11)
    X = torch.randn((M, K), device="cuda", generator=g).to(torch.bfloat16)
    W = (torch.randn((K, N), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    ref = F.fc_fwd(X, W)
    torch.cuda.synchronize()
    iters = 48
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(iters)]
    stream = torch.cuda.Stream()
    errors, statuses = [], []

    def hot():
        try:
            for o in outs:
                F.fc_fwd(X, W, out=o, stream=stream.cuda_stream)
        except Exception as e:  # reported on the main thread
            errors.append(e)

    def grow():
        for i in range(12):
            # 4 slices of fp32 partials: 32 KiB per row of M; 1 to 13 k rows
            statuses.append(F.fc_set_plan(F.OP_FWD, 1024 * (i + 2), KG, NG, 0, 0, 0, pid_grow))

    print(f"threads: split-2 plan {pid} at {M}x{K}x{N}, growth plan {pid_grow}", flush=True)
    threads = [threading.Thread(target=hot), threading.Thread(target=grow)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    assert statuses == [F.FC_OK] * 12, statuses
    assert F.fc_plan_describe(F.OP_FWD, M, K, N)["plan"] == pid
    bad = [i for i, o in enumerate(outs) if not torch.equal(o, ref)]
    F.fc_release()
    assert not bad, f"outputs {bad} differ from the plan's result before the growth"
