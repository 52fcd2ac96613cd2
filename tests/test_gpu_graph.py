"""Hot calls captured in a HIP graph: every replay reproduces the eager results
bit for bit, including plans that launch the transpose copy and the split-K
reduction (the hot path never allocates, synchronizes or clears memory)."""
from __future__ import annotations

import sys

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


def test_step_replays_bitwise():
    F.fc_release()
    g = torch.Generator(device="cuda").manual_seed(3)
    M, K, N = 1024, 1536, 768
    X = torch.randn((M, K), device="cuda", generator=g).to(torch.bfloat16)
    W = (torch.randn((K, N), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    dY = (torch.randn((M, N), device="cuda", generator=g) * 1e-3).to(torch.bfloat16)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dW = torch.empty((K, N), dtype=torch.bfloat16, device="cuda")
    # forward through a transpose-copy plan, backward-weight through split-K
    p_copy = _plan_with(F.OP_FWD, M, K, N, 1, 2)
    p_split = _plan_with(F.OP_BWD_WEIGHT, M, K, N, 4, 0)
    assert p_copy is not None and p_split is not None
    F.fc_set_plan(F.OP_FWD, M, K, N, 0, 0, 0, p_copy)
    F.fc_set_plan(F.OP_BWD_WEIGHT, M, K, N, 0, 0, 0, p_split)
    F.fc_set_plan(F.OP_BWD_DATA, M, K, N, 0, 0, 0, -1)

    def step():
        F.fc_fwd(X, W, out=Y)
        F.fc_bwd_data(dY, W, out=dX)
        F.fc_bwd_weight(X, dY, out=dW)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (Y, dX, dW)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        for t in (Y, dX, dW):  # eager work between the replays
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("Y", "dX", "dW"), ref, (Y, dX, dW)):
            same = torch.equal(a.view(torch.int16), b.view(torch.int16))
            print(f"replay {r} {name} identical={same}", file=sys.stderr, flush=True)
            assert same, f"replay {r}: {name} differs from the eager result"
    del graph
    F.fc_release()


def test_captured_graph_survives_a_workspace_growth():
    """A graph captured with a split-K plan keeps its workspace address; a later
    growth (a plan for a larger shape) retires that workspace instead of freeing
    it, so replays after the growth still match the eager result."""
    F.fc_release()
    g = torch.Generator(device="cuda").manual_seed(4)
    M, K, N = 2048, 512, 640
    X = torch.randn((M, K), device="cuda", generator=g).to(torch.bfloat16)
    dY = (torch.randn((M, N), device="cuda", generator=g) * 1e-3).to(torch.bfloat16)
    dW = torch.empty((K, N), dtype=torch.bfloat16, device="cuda")
    p_split = _plan_with(F.OP_BWD_WEIGHT, M, K, N, 4, 0)
    assert p_split is not None
    F.fc_set_plan(F.OP_BWD_WEIGHT, M, K, N, 0, 0, 0, p_split)
    F.fc_bwd_weight(X, dY, out=dW)
    torch.cuda.synchronize()
    ref = dW.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        F.fc_bwd_weight(X, dY, out=dW)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        F.fc_bwd_weight(X, dY, out=dW)
    torch.cuda.synchronize()
    before = F.fc_plan_describe(F.OP_BWD_WEIGHT, M, K, N)["ws"]
    # a split-K plan of a 16x larger output grows the workspace
    big = (M, 4 * K, 4 * N)
    p_big = _plan_with(F.OP_BWD_WEIGHT, *big, 4, 0)
    assert p_big is not None
    assert F.fc_plan_describe(F.OP_BWD_WEIGHT, *big)["ws"] > before
    # eager work that may reuse freed memory, then the replays
    junk = torch.full((64 << 20,), 7, dtype=torch.int32, device="cuda")
    for r in range(3):
        dW.zero_()
        junk.add_(1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(ref.view(torch.int16), dW.view(torch.int16))
        print(f"replay {r} after growth identical={same}", file=sys.stderr, flush=True)
        assert same
    del graph, junk
    F.fc_release()
