"""CPU simulation of the 3D parallel matrix multiply of one FC layer.

TEST INFRASTRUCTURE ONLY (part of the oracle; see oracle/__init__.py).

The pages state that the FC layer's matrix multiply is split with Agarwal's
3D parallel matrix multiplication over a Gx x Gy x Gz virtual grid
(sciencestack.ai/paper/2502.08145, Figure 1), that the weight matrix is
further sharded along Z to save memory, and that all-gather, reduce-scatter
and all-reduce collectives move the data (pith.science/paper/2502.08145,
"What carries the argument").

The index map is not on the pages (the figure's image is missing). This
module takes the plainest reading that the shard shapes of the workloads
support:

* the reduction dimension K of the forward product is split over Gx and the
  output dimension N over Gy (an h x 4h MLP-up layer on a 2 x 2 x 2 grid gives
  the 6144 x 24576 weight shard of the workloads), and the token dimension M
  over Gz;
* rank (x, y, z) holds X[z, x] (M/Gz x K/Gx), W[x, y, z] (the z-th row piece
  of the K/Gx x N/Gy block W[x, y]) and dY[z, y] (M/Gz x N/Gy);
* forward: all-gather W[x, y] over z, local Y_part = X[z, x] . W[x, y],
  all-reduce over x gives Y[z, y];
* backward-data: local dX_part = dY[z, y] . W[x, y]^T, all-reduce over y
  gives dX[z, x];
* backward-weight: local dW_part = X[z, x]^T . dY[z, y], reduce-scatter over z
  leaves each z with its row piece of dW[x, y].

Every local product is the oracle's own plain product; the collectives are
plain fp64 sums (in axis order) and concatenations. Uneven splits follow
numpy.array_split boundaries.
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np

from . import ROW, default


def _bounds(n: int, parts: int) -> List[Tuple[int, int]]:
    """Start/stop of `parts` nearly equal consecutive pieces of range(n)."""
    edges = [0]
    q, r = divmod(n, parts)
    for p in range(parts):
        edges.append(edges[-1] + q + (1 if p < r else 0))
    return [(edges[p], edges[p + 1]) for p in range(parts)]


def _block(a: np.ndarray, rb: Tuple[int, int], cb: Tuple[int, int]) -> np.ndarray:
    return np.ascontiguousarray(a[rb[0]:rb[1], cb[0]:cb[1]])


def simulate_layer(X: np.ndarray, W: np.ndarray, dY: np.ndarray,
                   grid: Tuple[int, int, int]) -> Dict[str, np.ndarray]:
    """Run forward, backward-data and backward-weight on a virtual grid.

    X (M x K), W (K x N), dY (M x N) are logical row-major bf16 bit arrays.
    Returns the reassembled full Y, dX, dW (fp64) and their scales S_*, plus
    `ranks`, the per-rank shard shapes, for inspection.
    """
    Gx, Gy, Gz = grid
    M, K = X.shape
    K2, N = W.shape
    assert K2 == K and dY.shape == (M, N)
    orc = default()
    mz = _bounds(M, Gz)  # token pieces
    kx = _bounds(K, Gx)  # input-feature pieces
    ny = _bounds(N, Gy)  # output-feature pieces

    Y = np.zeros((M, N))
    SY = np.zeros((M, N))
    dX = np.zeros((M, K))
    SdX = np.zeros((M, K))
    dW = np.zeros((K, N))
    SdW = np.zeros((K, N))
    ranks = {}

    # storage of the Z-sharded weight: rank (x, y, z) holds rows wz[z] of W[x, y]
    w_piece = {}
    for x in range(Gx):
        for y in range(Gy):
            Wxy = _block(W, kx[x], ny[y])
            wz = _bounds(Wxy.shape[0], Gz)
            for z in range(Gz):
                w_piece[(x, y, z)] = np.ascontiguousarray(Wxy[wz[z][0]:wz[z][1], :])

    for z in range(Gz):
        for y in range(Gy):
            for x in range(Gx):
                Xzx = _block(X, mz[z], kx[x])
                dYzy = _block(dY, mz[z], ny[y])
                # all-gather over z: the full W[x, y] block from its Z pieces
                Wxy = np.ascontiguousarray(np.concatenate([w_piece[(x, y, zz)] for zz in range(Gz)], 0))
                m, k = Xzx.shape
                n = Wxy.shape[1]
                ranks[(x, y, z)] = {"X": (m, k), "W": Wxy.shape, "W_piece": w_piece[(x, y, z)].shape,
                                    "dY": dYzy.shape}
                # forward partial, summed over x (all-reduce over Gx)
                yp, sp = orc.fc_fwd(Xzx, ROW, Wxy, ROW, m, k, n)
                Y[mz[z][0]:mz[z][1], ny[y][0]:ny[y][1]] += yp
                SY[mz[z][0]:mz[z][1], ny[y][0]:ny[y][1]] += sp
                # backward-data partial, summed over y (all-reduce over Gy)
                dxp, sxp = orc.fc_bwd_data(dYzy, Wxy, ROW, m, k, n)
                dX[mz[z][0]:mz[z][1], kx[x][0]:kx[x][1]] += dxp
                SdX[mz[z][0]:mz[z][1], kx[x][0]:kx[x][1]] += sxp
                # backward-weight partial, summed over z (reduce-scatter over Gz;
                # the scatter keeps row piece z of the block on rank z, so the
                # reassembled block is the full sum)
                dwp, swp = orc.fc_bwd_weight(Xzx, ROW, dYzy, m, k, n)
                dW[kx[x][0]:kx[x][1], ny[y][0]:ny[y][1]] += dwp
                SdW[kx[x][0]:kx[x][1], ny[y][0]:ny[y][1]] += swp

    return {"Y": Y, "S_Y": SY, "dX": dX, "S_dX": SdX, "dW": dW, "S_dW": SdW, "ranks": ranks}


def shard_shapes(M: int, K: int, N: int, grid: Tuple[int, int, int]) -> Dict[str, Tuple[int, int]]:
    """Per-GPU local GEMM shapes (even split) under the reading above."""
    Gx, Gy, Gz = grid
    return {"M": M // Gz, "K": K // Gx, "N": N // Gy}
