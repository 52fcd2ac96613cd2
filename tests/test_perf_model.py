"""The time-per-batch model of grid configurations (CPU only).

Pins, each independent of the model's own formulas:

* the ring volumes against a step-by-step simulation of the ring algorithms
  (chunks passed rank to rank, bytes counted, result checked);
* the local GEMM shapes and the collective sizes against the oracle's
  virtual-grid simulator (per-rank blocks of X, W, its Z piece and dY);
* the shard shapes of the workloads (hidden 12288 on 2x2x2, hidden 16384 at
  Gx = Gy = 8, the 405B-like layer on 2x4x2 with its vocabulary shard);
* the grid enumeration against brute force, and the node placement against
  hand-worked layouts;
* a hand-computed prediction.
"""
from __future__ import annotations

import itertools
import os
import tempfile

import numpy as np
import pytest

from oracle import grid as ogrid
from sharded_fc_layer_amd import inputs as I
from sharded_fc_layer_amd import perf_model as PM


# ------------------------------------------------------- ring algorithms, simulated

def _chunks(n, p):
    return np.array_split(np.arange(n), p)


def sim_ring_reduce_scatter(bufs):
    """Ring reduce-scatter: p - 1 steps; at step s rank r passes its running sum of
    chunk (r - s) mod p to rank r + 1. Returns per-rank arrays (rank r owns chunk
    (r + 1) mod p in full) and the elements each rank sent."""
    p = len(bufs)
    b = [x.astype(np.float64).copy() for x in bufs]
    ch = _chunks(len(b[0]), p)
    sent = [0] * p
    for s in range(p - 1):
        msgs = []
        for r in range(p):
            c = ch[(r - s) % p]
            msgs.append((r, (r + 1) % p, c, b[r][c].copy()))
        for src, dst, c, v in msgs:
            b[dst][c] += v
            sent[src] += len(c)
    return b, ch, sent


def sim_ring_all_gather(bufs, ch):
    """Ring all-gather: rank r starts owning chunk (r + 1) mod p; at step s it
    passes chunk (r + 1 - s) mod p to rank r + 1."""
    p = len(bufs)
    b = [x.copy() for x in bufs]
    sent = [0] * p
    for s in range(p - 1):
        msgs = []
        for r in range(p):
            c = ch[(r + 1 - s) % p]
            msgs.append((r, (r + 1) % p, c, b[r][c].copy()))
        for src, dst, c, v in msgs:
            b[dst][c] = v
            sent[src] += len(c)
    return b, sent


@pytest.mark.parametrize("p", [2, 3, 4, 8])
def test_ring_volumes_match_a_simulated_ring(p):
    n = 24 * p  # elements, divisible by p
    rng = np.random.default_rng(p)
    bufs = [rng.integers(-100, 100, n).astype(np.float64) for _ in range(p)]
    total = np.sum(bufs, axis=0)
    size = n * 2  # bf16 bytes
    rs, ch, sent_rs = sim_ring_reduce_scatter(bufs)
    for r in range(p):
        c = ch[(r + 1) % p]
        assert np.array_equal(rs[r][c], total[c])
    assert all(s * 2 == PM.ring_reduce_scatter_bytes(size, p) for s in sent_rs)
    ag, sent_ag = sim_ring_all_gather(rs, ch)
    for r in range(p):
        assert np.array_equal(ag[r], total)  # reduce-scatter + all-gather = all-reduce
    assert all(s * 2 == PM.ring_all_gather_bytes(size, p) for s in sent_ag)
    assert all((a + b) * 2 == PM.ring_all_reduce_bytes(size, p) for a, b in zip(sent_rs, sent_ag))


def test_single_member_groups_send_nothing():
    for f in (PM.ring_all_reduce_bytes, PM.ring_reduce_scatter_bytes, PM.ring_all_gather_bytes):
        assert f(1 << 20, 1) == 0.0


# ------------------------------------------------------- shards vs the oracle's grid

@pytest.mark.parametrize("g", [(2, 2, 2), (1, 2, 4), (4, 1, 2), (2, 3, 1)])
def test_shards_match_the_virtual_grid_simulator(g):
    Gx, Gy, Gz = g
    h, T = 24, 16  # one QKV layer: K_f = 24, N_f = 72
    model = PM.Model("tiny", h, 4 * h, 1, 0, T)
    sh = {s.name: s for s in PM.shards(model, PM.Grid(1, Gx, Gy, Gz))}["qkv"]
    d = I.make_random_inputs(T, h, 3 * h, seed=3)
    sim = ogrid.simulate_layer(d["X"], d["W"], d["dY"], g)
    for (x, y, z), r in sim["ranks"].items():
        assert r["X"] == (sh.M, sh.K) and r["W"] == (sh.K, sh.N) and r["dY"] == (sh.M, sh.N)
        sizes = {c.name: c.size for c in sh.collectives}
        # the gathered W block is the concatenation of the Gz pieces
        assert sizes["W all-gather (fwd)"] == r["W_piece"][0] * r["W_piece"][1] * 2 * Gz
        assert sizes["Y all-reduce"] == r["X"][0] * r["W"][1] * 2
        assert sizes["dX all-reduce"] == r["dY"][0] * r["W"][0] * 2
        assert sizes["dW reduce-scatter"] == r["W"][0] * r["W"][1] * 2


def test_workload_shards():
    w3 = PM.shards(PM.Model("h12288", 12288, 49152, 1, 0, 16384), PM.Grid(1, 2, 2, 2))
    assert [(s.M, s.K, s.N) for s in w3 if s.name == "mlp_up"] == [(8192, 6144, 24576)]
    w4 = PM.shards(PM.Model("h16384", 16384, 53248, 1, 0, 8192), PM.Grid(1, 8, 8, 1))
    assert [(s.M, s.K, s.N) for s in w4 if s.name == "mlp_up"] == [(8192, 2048, 6656)]
    w5 = PM.shards(PM.Model("405b-like", 16384, 53248, 126, 128256, 16384), PM.Grid(1, 2, 4, 2))
    assert {s.name: (s.M, s.K, s.N) for s in w5} == {g.name: (g.M, g.K, g.N) for g in I.WORKLOADS[5]}


def test_grids_enumerate_every_factorisation():
    for G in (1, 6, 8, 12, 16):
        brute = {(d, x, y, z) for d, x, y, z in itertools.product(range(1, G + 1), repeat=4) if d * x * y * z == G}
        got = [(g.data, g.x, g.y, g.z) for g in PM.grids(G)]
        assert len(got) == len(set(got)) and set(got) == brute
    assert len(PM.grids(8)) == 20


def test_placement_on_nodes_of_eight():
    m = PM.Machine()
    g = PM.Grid(1, 2, 2, 2)  # one node
    for ax in ("x", "y", "z"):
        assert PM.group_bandwidth(g, (ax,), m) == (m.link_gbs, "intra")
    g = PM.Grid(2, 2, 2, 2)  # two nodes: only the data groups cross
    assert PM.group_bandwidth(g, ("data",), m) == (m.inter_gbs, "inter")
    assert PM.group_bandwidth(g, ("z",), m)[1] == "intra"
    assert PM.group_bandwidth(PM.Grid(1, 8, 1, 1), ("x",), m) == (7 * m.link_gbs, "intra")
    assert PM.group_bandwidth(PM.Grid(1, 16, 1, 1), ("x",), m) == (m.inter_gbs, "inter")
    assert PM.group_bandwidth(PM.Grid(1, 4, 4, 1), ("x", "y"), m) == (m.inter_gbs, "inter")
    # x = 2 inside a node of 8: the y groups (stride 2, 4 members) stay inside
    assert PM.group_bandwidth(PM.Grid(1, 2, 4, 2), ("y",), m) == (3 * m.link_gbs, "intra")
    assert PM.group_bandwidth(PM.Grid(1, 2, 4, 2), ("z",), m) == (m.inter_gbs, "inter")


def _times(model, G, f):
    return {(op, M, K, N): f(op, M, K, N) for (M, K, N) in PM.needed_shapes(model, G) for op in PM.OPS}


def test_hand_computed_prediction():
    model = PM.Model("tiny", 64, 256, 3, 0, 1024)
    m = PM.Machine(link_gbs=100.0)
    t = _times(model, 2, lambda op, M, K, N: 1e-9 * M * K * N)
    # Gx = 2 in one node: only Y is all-reduced, over one link; nothing else has two members
    r = PM.predict(model, PM.Grid(1, 2, 1, 1), m, t)
    comm = sum(3 * 2 * (1 / 2) * (1024 * nf * 2) / 100e9 * 1e3 for nf in (192, 64, 256, 64))
    compute = sum(3 * 3 * 1e-9 * 1024 * (kf // 2) * nf for kf, nf in ((64, 192), (64, 64), (64, 256), (256, 64)))
    assert r["comm_ms"] == pytest.approx(comm, rel=1e-12)
    assert r["compute_ms"] == pytest.approx(compute, rel=1e-12)
    assert r["total_ms"] == pytest.approx(comm + compute, rel=1e-12)
    assert r["overlap_bound_ms"] == pytest.approx(max(comm, compute), rel=1e-12)
    one = PM.predict(model, PM.Grid(1, 1, 1, 1), m, _times(model, 1, lambda op, M, K, N: 1.0))
    assert one["comm_ms"] == 0.0 and one["compute_ms"] == 3 * 4 * 3


def test_rank_orders_and_reports_missing_times():
    model = PM.Model("tiny", 64, 256, 2, 64, 512)
    t = _times(model, 8, lambda op, M, K, N: 1e-9 * M * K * N)
    done, missing = PM.rank(model, 8, PM.Machine(), t)
    assert not missing and len(done) == 20
    assert [r["total_ms"] for r in done] == sorted(r["total_ms"] for r in done)
    drop = next(iter(t))
    del t[drop]
    done2, missing2 = PM.rank(model, 8, PM.Machine(), t)
    assert missing2 and all(k == drop for _, k in missing2) and len(done2) + len(missing2) == 20
    assert PM.shards(PM.Model("odd", 64, 256, 1, 0, 500), PM.Grid(1, 1, 1, 8)) is None  # 500 tokens over 8


def test_times_from_plan_file():
    lines = ["gfx950:sramecc+:xnack- 0 512 64 192 0 0 0 336 0.012500",
             "gfx950:sramecc+:xnack- 1 512 64 192 0 0 0 336",  # no time: skipped
             "gfx950:sramecc+:xnack- 2 512 64 192 1 0 0 336 0.5",  # other order: skipped
             "gfx950:sramecc+:xnack- 2 512 64 192 0 0 0 336 0.020000"]
    with tempfile.TemporaryDirectory() as d:
        p = os.path.join(d, "plans.txt")
        open(p, "w").write("\n".join(lines) + "\n")
        t = PM.times_from_plan_file(p)
    assert t == {("fwd", 512, 64, 192): 0.0125, ("bwd_weight", 512, 64, 192): 0.02}


def test_weight_state_memory():
    # 405B-like FC weights: 126 layers x (3h^2 + h^2 + 2 h f) + vocabulary h V
    h, f, V, Lr = 16384, 53248, 128256, 126
    model = PM.Model("405b-like", h, f, Lr, V, 16384)
    t = _times(model, 16, lambda op, M, K, N: 1e-9 * M * K * N)
    full = Lr * (3 * h * h + h * h + 2 * h * f) + h * V
    for g in (PM.Grid(16, 1, 1, 1), PM.Grid(1, 2, 4, 2), PM.Grid(2, 2, 2, 2)):
        r = PM.predict(model, g, PM.Machine(), t)
        assert r["weight_state_gb"] == pytest.approx(full / (g.x * g.y * g.z) * 16 / 1e9, rel=1e-12)
    done, _ = PM.rank(model, 16, PM.Machine(), t)
    fits = [r["fits"] for r in done]
    assert fits == sorted(fits, reverse=True)  # grids that fit come first
    assert not PM.predict(model, PM.Grid(16, 1, 1, 1), PM.Machine(), t)["fits"]
