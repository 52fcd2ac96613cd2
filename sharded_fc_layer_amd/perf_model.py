"""Time-per-batch model of 4D hybrid parallel training (G_data x Gx x Gy x Gz) of
a GPT-style model's fully connected layers on MI355X nodes.

What the pages fix (pith.science/paper/2502.08145, "Core claim", "What carries
the argument" and "Assumptions & free parameters"): the model predicts the
time of a configuration by summing the times of ring collectives, each
message size over a bandwidth that depends on where the process group sits in
the machine hierarchy; collectives are taken to be rings, message start-up
cost is neglected, one inter-node bandwidth serves every node pair, and the
model ranks configurations (sciencestack.ai/paper/2502.08145, Figure 2
validates it by the rank order of observed batch times). The pages do not
print the model's equations, so the textbook ring volumes stand in: per rank,
an all-reduce of S bytes sends 2 (p - 1) / p * S, a reduce-scatter or an
all-gather of an S-byte result sends (p - 1) / p * S.

Readings where the pages are silent:

* Shards follow the virtual-grid reading of the FC layer used throughout this
  package: a layer with K_f inputs and N_f outputs runs the local products at
  M = T / (G_data Gz), K = K_f / Gx, N = N_f / Gy (T tokens per batch). The
  vocabulary projection is sharded over its N_f only, across Gx Gy (K = K_f).
* Collectives per layer and batch: the Z-sharded weight block is all-gathered
  over Gz before the forward and again before the backward (Z sharding exists
  to save memory, so the gathered block is not kept); Y is all-reduced over Gx;
  dX over Gy (over Gx Gy for the vocabulary layer); dW is reduce-scattered over
  Gz and its piece all-reduced over G_data. Every message is bf16.
* Ranks are laid out with x fastest, then y, z and data. A group whose members
  share one node communicates over xGMI: the 8 GPUs of a node are fully
  connected, so a group of p members can run p - 1 rings on disjoint links and
  gets (p - 1) link bandwidths per rank. A group that spans nodes gets the
  inter-node bandwidth per GPU.
* The compute term is the sum of the three local products of every FC layer,
  each the time fc_tune measured for its plan (flushed caches, one launch),
  read from a plan file that fc_plans_save wrote. Attention's own products,
  normalisation and the optimizer are not FC shard GEMMs and are not modelled.
* Time per batch = compute + communication (no overlap), as the pages' model
  sums collective times; max(compute, communication) is reported beside it as
  the bound that perfect overlap would reach.
* Memory: a grid fits if its FC parameters per GPU (all FC weights over
  Gx Gy Gz; data parallelism replicates) times 16 bytes (bf16 weight and
  gradient, fp32 master weight, two fp32 Adam moments) fit in the GPU's HBM.
  Activations are not counted. Grids that do not fit rank after those that do.

Usage (the plan file is written on a GPU; ranking needs only the CPU):
  python -m sharded_fc_layer_amd.perf_model measure --out plans.txt [model] [--gpus G]
  python -m sharded_fc_layer_amd.perf_model rank --times plans.txt [model] [--gpus G]
  python -m sharded_fc_layer_amd.perf_model validate --times plans.txt --grid d,x,y,z [model]
"""
from __future__ import annotations

import argparse
import json
import sys
from dataclasses import dataclass
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

BF16 = 2
OPS = ("fwd", "bwd_data", "bwd_weight")
AXES = ("x", "y", "z", "data")  # fastest-varying first in the rank layout


# ------------------------------------------------------------- ring volumes

def ring_all_reduce_bytes(size: float, p: int) -> float:
    """Bytes one rank sends in a ring all-reduce of a `size`-byte buffer."""
    return 2.0 * (p - 1) / p * size if p > 1 else 0.0


def ring_reduce_scatter_bytes(size: float, p: int) -> float:
    """Bytes one rank sends in a ring reduce-scatter of a `size`-byte buffer."""
    return (p - 1) / p * size if p > 1 else 0.0


def ring_all_gather_bytes(size: float, p: int) -> float:
    """Bytes one rank sends in a ring all-gather whose gathered result is `size` bytes."""
    return (p - 1) / p * size if p > 1 else 0.0


_VOLUME = {"all_reduce": ring_all_reduce_bytes, "reduce_scatter": ring_reduce_scatter_bytes,
           "all_gather": ring_all_gather_bytes}


# ------------------------------------------------------------- grid, machine

@dataclass(frozen=True)
class Grid:
    data: int
    x: int
    y: int
    z: int

    @property
    def gpus(self) -> int:
        return self.data * self.x * self.y * self.z

    def size(self, axis: str) -> int:
        return getattr(self, axis)

    def __str__(self) -> str:
        return f"{self.data}x{self.x}x{self.y}x{self.z}"


def grids(gpus: int) -> List[Grid]:
    """Every (G_data, Gx, Gy, Gz) with product `gpus`."""
    divs = [d for d in range(1, gpus + 1) if gpus % d == 0]
    out = []
    for d in divs:
        for x in divs:
            for y in divs:
                if gpus % (d * x * y) == 0:
                    out.append(Grid(d, x, y, gpus // (d * x * y)))
    return out


@dataclass(frozen=True)
class Machine:
    gpus_per_node: int = 8
    link_gbs: float = 153.0  # one xGMI link, one direction, GB/s
    inter_gbs: float = 50.0  # per GPU between nodes, GB/s (one 400 Gb/s NIC per GPU)
    hbm_gb: float = 288.0
    bytes_per_param: int = 16  # bf16 weight + bf16 gradient + fp32 master + two fp32 Adam moments


def _coords(grid: Grid, rank: int) -> Dict[str, int]:
    c = {}
    for a in AXES:
        c[a] = rank % grid.size(a)
        rank //= grid.size(a)
    return c


def groups(grid: Grid, axes: Sequence[str]) -> List[List[int]]:
    """Ranks of every process group that spans `axes` (the other coordinates fixed)."""
    out: Dict[Tuple[int, ...], List[int]] = {}
    for r in range(grid.gpus):
        c = _coords(grid, r)
        key = tuple(c[a] for a in AXES if a not in axes)
        out.setdefault(key, []).append(r)
    return list(out.values())


def group_bandwidth(grid: Grid, axes: Sequence[str], m: Machine) -> Tuple[float, str]:
    """(GB/s per rank, "intra" | "inter") for the groups spanning `axes`."""
    gs = groups(grid, axes)
    p = len(gs[0])
    intra = all(len({r // m.gpus_per_node for r in g}) == 1 for g in gs)
    if intra:
        return m.link_gbs * max(p - 1, 1), "intra"
    return m.inter_gbs, "inter"


# ------------------------------------------------------------- model, shards

@dataclass(frozen=True)
class Model:
    name: str
    hidden: int
    ffn: int
    layers: int
    vocab: int  # 0: no vocabulary projection
    tokens: int  # tokens per batch (global)

    def fcs(self) -> List[Tuple[str, int, int]]:
        h = self.hidden
        return [("qkv", h, 3 * h), ("out_proj", h, h), ("mlp_up", h, self.ffn), ("mlp_down", self.ffn, h)]


@dataclass(frozen=True)
class Collective:
    name: str
    kind: str  # all_reduce | reduce_scatter | all_gather
    axes: Tuple[str, ...]
    size: int  # bytes of the buffer (all-reduce, reduce-scatter) or of the gathered result


@dataclass(frozen=True)
class Shard:
    name: str
    M: int
    K: int
    N: int
    count: int  # how many such layers per batch
    collectives: Tuple[Collective, ...]


def _div(a: int, b: int) -> Optional[int]:
    return a // b if a % b == 0 else None


def shards(model: Model, grid: Grid) -> Optional[List[Shard]]:
    """Local GEMM shapes and collectives of every FC layer; None if the grid does not divide the model."""
    out = []
    M = _div(model.tokens, grid.data * grid.z)
    if M is None:
        return None
    for name, kf, nf in model.fcs():
        K, N = _div(kf, grid.x), _div(nf, grid.y)
        if K is None or N is None:
            return None
        w = K * N * BF16
        cs = (Collective("W all-gather (fwd)", "all_gather", ("z",), w),
              Collective("Y all-reduce", "all_reduce", ("x",), M * N * BF16),
              Collective("W all-gather (bwd)", "all_gather", ("z",), w),
              Collective("dX all-reduce", "all_reduce", ("y",), M * K * BF16),
              Collective("dW reduce-scatter", "reduce_scatter", ("z",), w),
              Collective("dW data all-reduce", "all_reduce", ("data",), w // grid.z))
        out.append(Shard(name, M, K, N, model.layers, cs))
    if model.vocab:
        N = _div(model.vocab, grid.x * grid.y)
        K = model.hidden
        if N is None:
            return None
        w = K * N * BF16
        cs = (Collective("W all-gather (fwd)", "all_gather", ("z",), w),
              Collective("W all-gather (bwd)", "all_gather", ("z",), w),
              Collective("dX all-reduce", "all_reduce", ("x", "y"), M * K * BF16),
              Collective("dW reduce-scatter", "reduce_scatter", ("z",), w),
              Collective("dW data all-reduce", "all_reduce", ("data",), w // grid.z))
        out.append(Shard("vocab", M, K, N, 1, cs))
    return out


def collective_ms(c: Collective, grid: Grid, m: Machine) -> float:
    p = 1
    for a in c.axes:
        p *= grid.size(a)
    if p == 1:
        return 0.0
    gbs, _ = group_bandwidth(grid, c.axes, m)
    return _VOLUME[c.kind](c.size, p) / (gbs * 1e9) * 1e3


# ------------------------------------------------------------- prediction

GemmTimes = Dict[Tuple[str, int, int, int], float]  # (op, M, K, N) -> ms


def predict(model: Model, grid: Grid, m: Machine, times: GemmTimes) -> Optional[dict]:
    """Predicted time per batch of one grid, or None if the grid does not divide the model.

    Raises KeyError naming the first local GEMM that `times` lacks."""
    sh = shards(model, grid)
    if sh is None:
        return None
    compute = comm = 0.0
    parts: Dict[str, float] = {}
    for s in sh:
        for op in OPS:
            key = (op, s.M, s.K, s.N)
            if key not in times:
                raise KeyError(key)
            compute += s.count * times[key]
        for c in s.collectives:
            t = s.count * collective_ms(c, grid, m)
            comm += t
            parts[c.name] = parts.get(c.name, 0.0) + t
    params = sum(s.count * s.K * s.N for s in sh)  # this GPU's weight shards (before the Z split)
    state_gb = params / grid.z * m.bytes_per_param / 1e9
    return {"grid": str(grid), "compute_ms": compute, "comm_ms": comm, "total_ms": compute + comm,
            "overlap_bound_ms": max(compute, comm), "comm_parts_ms": parts,
            "weight_state_gb": state_gb, "fits": state_gb <= m.hbm_gb}


def rank(model: Model, gpus: int, m: Machine, times: GemmTimes) -> Tuple[List[dict], List[Tuple[str, tuple]]]:
    """Grids that divide the model, fastest predicted first, and the grids skipped for a missing GEMM time."""
    done, missing = [], []
    for g in grids(gpus):
        try:
            r = predict(model, g, m, times)
        except KeyError as e:
            missing.append((str(g), e.args[0]))
            continue
        if r is not None:
            done.append(r)
    done.sort(key=lambda r: (not r["fits"], r["total_ms"], r["grid"]))
    return done, missing


def needed_shapes(model: Model, gpus: int) -> List[Tuple[int, int, int]]:
    """The distinct local (M, K, N) over every grid that divides the model."""
    out = set()
    for g in grids(gpus):
        sh = shards(model, g)
        if sh:
            out.update((s.M, s.K, s.N) for s in sh)
    return sorted(out)


def times_from_plan_file(path: str) -> GemmTimes:
    """GEMM times from a file that fc_plans_save wrote (lines with a time field; row-major, bf16 out)."""
    t: GemmTimes = {}
    for line in open(path):
        f = line.split()
        if len(f) != 10 or f[0].startswith("#"):
            continue
        op, M, K, N, xo, wo, f32 = (int(v) for v in f[1:8])
        if xo == 0 and wo == 0 and f32 == 0:
            t[(OPS[op], M, K, N)] = float(f[9])
    return t


# ------------------------------------------------------------- GPU side

def measure(model: Model, gpus: int, out_path: str, max_elems: int = 1 << 31) -> int:
    """Tune every local GEMM the model needs at `gpus` and save the plans with their times."""
    from . import fcshard as F
    n = 0
    for (M, K, N) in needed_shapes(model, gpus):
        if max(M * K, K * N, M * N) > max_elems:
            continue
        F.fc_tune(M, K, N)
        n += 1
        print(f"[perf_model] tuned {M}x{K}x{N}", flush=True)
    F.fc_plans_save(out_path)
    return n


def validate(model: Model, grid: Grid, times_path: str, steps: int = 20, warmup: int = 5) -> dict:
    """Time one batch's FC shard GEMMs of `grid` back to back on one GPU, with the
    plans of `times_path`, against the model's compute term."""
    import torch
    from . import fcshard as F
    F.fc_plans_load(times_path)
    times = times_from_plan_file(times_path)
    sh = shards(model, grid)
    if sh is None:
        raise ValueError(f"grid {grid} does not divide the model")
    bufs = []
    g = torch.Generator(device="cuda").manual_seed(0)
    for s in sh:
        X = torch.randn((s.M, s.K), device="cuda", generator=g).to(torch.bfloat16)
        W = (torch.randn((s.K, s.N), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        dY = (torch.randn((s.M, s.N), device="cuda", generator=g) * 1e-3).to(torch.bfloat16)
        bufs.append((s, X, W, dY, torch.empty((s.M, s.N), dtype=torch.bfloat16, device="cuda"),
                     torch.empty((s.M, s.K), dtype=torch.bfloat16, device="cuda"),
                     torch.empty((s.K, s.N), dtype=torch.bfloat16, device="cuda")))

    def one_layer():  # each shape once: forward in order, then the backward products in reverse
        for s, X, W, dY, Y, dX, dW in bufs:
            F.fc_fwd(X, W, out=Y)
        for s, X, W, dY, Y, dX, dW in reversed(bufs):
            F.fc_bwd_data(dY, W, out=dX)
            F.fc_bwd_weight(X, dY, out=dW)

    for _ in range(warmup):
        one_layer()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        one_layer()
    b.record()
    torch.cuda.synchronize()
    measured = a.elapsed_time(b) / steps
    predicted = sum(times[(op, s.M, s.K, s.N)] for s in sh for op in OPS)
    return {"grid": str(grid), "gemms": 3 * len(sh), "measured_ms": measured, "predicted_ms": predicted,
            "predicted_over_measured": predicted / measured}


# ------------------------------------------------------------- CLI

def _model_args(p: argparse.ArgumentParser) -> None:
    p.add_argument("--name", default="gpt-h2048")
    p.add_argument("--hidden", type=int, default=2048)
    p.add_argument("--ffn", type=int, default=8192)
    p.add_argument("--layers", type=int, default=24)
    p.add_argument("--vocab", type=int, default=0)
    p.add_argument("--tokens", type=int, default=65536, help="tokens per batch (global)")
    p.add_argument("--gpus", type=int, default=8)


def _model(a) -> Model:
    return Model(a.name, a.hidden, a.ffn, a.layers, a.vocab, a.tokens)


def main(argv: Optional[Iterable[str]] = None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    pm = sub.add_parser("measure", help="tune the needed local GEMMs on this GPU, save plans with times")
    _model_args(pm)
    pm.add_argument("--out", required=True)
    pr = sub.add_parser("rank", help="rank the grids (CPU only)")
    _model_args(pr)
    pr.add_argument("--times", required=True)
    pr.add_argument("--link-gbs", type=float, default=Machine.link_gbs)
    pr.add_argument("--inter-gbs", type=float, default=Machine.inter_gbs)
    pr.add_argument("--json", action="store_true")
    pv = sub.add_parser("validate", help="time one grid's shard GEMM stream on this GPU vs the model")
    _model_args(pv)
    pv.add_argument("--times", required=True)
    pv.add_argument("--grid", required=True, help="d,x,y,z")
    a = ap.parse_args(argv)
    model = _model(a)
    if a.cmd == "measure":
        n = measure(model, a.gpus, a.out)
        print(f"[perf_model] {n} shapes tuned, plans and times in {a.out}")
        return 0
    if a.cmd == "validate":
        g = Grid(*(int(v) for v in a.grid.split(",")))
        print(json.dumps(validate(model, g, a.times)))
        return 0
    m = Machine(link_gbs=a.link_gbs, inter_gbs=a.inter_gbs)
    done, missing = rank(model, a.gpus, m, times_from_plan_file(a.times))
    if a.json:
        print(json.dumps({"model": model.__dict__, "gpus": a.gpus, "ranked": done,
                          "missing": [[g, list(k)] for g, k in missing]}))
        return 0
    print(f"{model.name}: hidden {model.hidden}, ffn {model.ffn}, {model.layers} layers, vocab {model.vocab}, "
          f"{model.tokens} tokens per batch, {a.gpus} GPUs")
    print(f"{'rank':>4} {'grid d x y z':>13} {'compute ms':>11} {'comm ms':>9} {'total ms':>9} {'overlap ms':>10} "
          f"{'state GB':>9}")
    for i, r in enumerate(done, 1):
        print(f"{i:4d} {r['grid']:>13} {r['compute_ms']:11.3f} {r['comm_ms']:9.3f} {r['total_ms']:9.3f} "
              f"{r['overlap_bound_ms']:10.3f} {r['weight_state_gb']:9.1f}{'' if r['fits'] else '  does not fit'}")
    for g, k in missing:
        print(f"     {g:>13} no measured time for {k}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
