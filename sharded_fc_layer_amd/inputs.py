"""Seeded synthetic inputs for the shard GEMMs of a 3D-parallel FC layer.

This module is the one piece shared by the CPU oracle's tests and the GPU
path: it draws numbers and encodes them as bf16 bit patterns. It holds none
of the method's arithmetic (no product, no reduction, no output rounding).

Workloads are the per-GPU shard shapes of a GPT-style FC layer under the
3D parallel matrix multiply (sciencestack.ai/paper/2502.08145, Figure 1:
a matrix multiply in an FC layer split over a Gx x Gy x Gz virtual grid),
in bf16 (mlsanity.com/paper/2502.08145, Abstract: bf16 training).

Shape conventions: X is M x K (tokens x input features), W is K x N
(input x output features), dY is M x N. All generators return *logical*
row-major arrays of uint16 bf16 bit patterns; `stored()` produces the
column-major storage of the same logical values.

Recipe (a reading; the pages print no data): for workload c, GEMM g and
matrix t (X = 0, W = 1, dY = 2), the logical row-major elements are cut into
chunks of 2**20; chunk j holds float32 standard normals drawn by
`numpy.random.default_rng([seed, c, g, t, j])`, scaled in float32 by the
workload's standard deviation, then rounded to bf16 to nearest-even. Chunks
are independent streams, so large shards are generated on all host cores.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

ROW = 0  # storage order: row-major
COL = 1  # storage order: column-major


@dataclass(frozen=True)
class GemmShape:
    """One FC shard: X (M x K), W (K x N), dY (M x N) and their std-devs."""

    name: str
    M: int
    K: int
    N: int
    sx: float = 1.0
    sw: float = 0.02
    sdy: float = 1e-3

    @property
    def flops(self) -> int:
        """Multiply-add count x 2 of one of the three products (all equal)."""
        return 2 * self.M * self.K * self.N


# Workloads, numbered 1..5 as listed with the benchmark. Each is a list of FC
# shards; every shard runs forward, backward-data and backward-weight.
WORKLOADS: Dict[int, List[GemmShape]] = {
    # single FC layer, 256 tokens, 512 -> 2048, dY std 0.01, seed 0
    1: [GemmShape("fc", 256, 512, 2048, 1.0, 0.02, 0.01)],
    # GPT-style block, hidden 2048, 8192 tokens (batch 4 x seq 2048)
    2: [
        GemmShape("qkv", 8192, 2048, 6144),
        GemmShape("attn_out", 8192, 2048, 2048),
        GemmShape("mlp_up", 8192, 2048, 8192),
        GemmShape("mlp_down", 8192, 8192, 2048),
    ],
    # one GPU's shard of a hidden-12288 / FFN-49152 MLP-up on a 2x2x2 grid:
    # K = 12288 / Gx, N = 49152 / Gy
    3: [GemmShape("mlp_up_shard", 8192, 6144, 24576)],
    # skinny shard of hidden 16384 / FFN 53248 at Gx = Gy = 8
    4: [GemmShape("skinny_shard", 8192, 2048, 6656)],
    # 405B-like layer (hidden 16384, FFN 53248, 128 heads) on a 2x4x2 grid:
    # K = features_in / Gx, N = features_out / Gy; vocab shard 16384 x 16032
    5: [
        GemmShape("qkv", 8192, 8192, 12288),
        GemmShape("out_proj", 8192, 8192, 4096),
        GemmShape("mlp_up", 8192, 8192, 13312),
        GemmShape("mlp_down", 8192, 26624, 4096),
        GemmShape("vocab", 8192, 16384, 16032),
    ],
}

# storage-order pairs (x_order, w_order) exercised by workload 4
ORDER_PAIRS: List[Tuple[int, int]] = [(ROW, ROW), (ROW, COL), (COL, ROW)]


CHUNK = 1 << 20


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Encode finite float32 values as bf16 bit patterns, nearest-even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("inputs must be finite")
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16_chunked(key: Sequence[int], shape: Tuple[int, int], std: float) -> np.ndarray:
    """N(0, std) bf16 bits; chunk j of the flat array comes from default_rng(key + [j])."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)

    def work(j: int) -> None:
        lo = j * CHUNK
        hi = min(n, lo + CHUNK)
        x = np.random.default_rng(list(key) + [j]).standard_normal(hi - lo, dtype=np.float32)
        x *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(x)

    nchunks = (n + CHUNK - 1) // CHUNK
    if nchunks <= 1:
        for j in range(nchunks):
            work(j)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def integer_bf16_chunked(key: Sequence[int], shape: Tuple[int, int], lo: int = -3, hi: int = 3) -> np.ndarray:
    """Integers uniform in [lo, hi] as bf16 bits (exact), for arrays too large for
    integer_bf16; chunk j of the flat array comes from default_rng(key + [j])."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)

    def work(j: int) -> None:
        a = j * CHUNK
        b = min(n, a + CHUNK)
        x = np.random.default_rng(list(key) + [j]).integers(lo, hi + 1, size=b - a, dtype=np.int8)
        out[a:b] = f32_to_bf16_bits(x.astype(np.float32))

    nchunks = (n + CHUNK - 1) // CHUNK
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def normal_bf16(rng: np.random.Generator, shape: Tuple[int, ...], std: float) -> np.ndarray:
    """float32 N(0, std) draws rounded to bf16 (std is a standard deviation)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    x *= np.float32(std)
    return f32_to_bf16_bits(x)


def integer_bf16(rng: np.random.Generator, shape: Tuple[int, ...], lo: int = -3, hi: int = 3,
                 scale_pow2: int = 0) -> np.ndarray:
    """Integers uniform in [lo, hi], times 2**scale_pow2, as bf16 bits (exact)."""
    x = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    x *= np.float32(2.0 ** scale_pow2)
    return f32_to_bf16_bits(x)


def make_inputs(workload: int, gemm_index: int, seed: int = 0,
                shape: Optional[GemmShape] = None) -> Dict[str, np.ndarray]:
    """Seeded inputs for one shard GEMM: logical row-major bf16 bit arrays.

    Returns {"X": (M,K), "W": (K,N), "dY": (M,N)}. `gemm_index` is the
    1-based position of the shard in the workload's list.
    """
    g = shape if shape is not None else WORKLOADS[workload][gemm_index - 1]
    key = [seed, workload, gemm_index]
    return {"X": normal_bf16_chunked(key + [0], (g.M, g.K), g.sx),
            "W": normal_bf16_chunked(key + [1], (g.K, g.N), g.sw),
            "dY": normal_bf16_chunked(key + [2], (g.M, g.N), g.sdy)}


def make_integer_inputs(M: int, K: int, N: int, seed: int = 0, lo: int = -3, hi: int = 3,
                        pow2: Tuple[int, int, int] = (0, 0, 0)) -> Dict[str, np.ndarray]:
    """Integer-valued inputs whose products and partial sums are exact in fp32."""
    rng = np.random.default_rng([seed, M, K, N, 7])
    return {
        "X": integer_bf16(rng, (M, K), lo, hi, pow2[0]),
        "W": integer_bf16(rng, (K, N), lo, hi, pow2[1]),
        "dY": integer_bf16(rng, (M, N), lo, hi, pow2[2]),
    }


def make_random_inputs(M: int, K: int, N: int, seed: int = 0, sx: float = 1.0, sw: float = 0.02,
                       sdy: float = 1e-3) -> Dict[str, np.ndarray]:
    """Normal inputs of an arbitrary shape (same recipe as the workloads)."""
    rng = np.random.default_rng([seed, M, K, N, 11])
    return {"X": normal_bf16(rng, (M, K), sx), "W": normal_bf16(rng, (K, N), sw),
            "dY": normal_bf16(rng, (M, N), sdy)}


def stored(logical: np.ndarray, order: int) -> np.ndarray:
    """Storage of a logical 2-D array: itself (row-major) or its transpose copy."""
    if order == ROW:
        return np.ascontiguousarray(logical)
    if order == COL:
        return np.ascontiguousarray(logical.T)
    raise ValueError(f"bad order {order}")
