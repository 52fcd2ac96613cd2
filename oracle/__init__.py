"""CPU oracle for the shard GEMMs of a 3D-parallel FC layer.

TEST INFRASTRUCTURE ONLY: only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module. It never imports the GPU
package (sharded_fc_layer_amd) and shares no code with it.

`oracle.c` holds the arithmetic (plain fp64 loops over exact bf16 values);
this module builds and loads it and marshals numpy arrays. `grid.py` holds the
CPU simulation of the Gx x Gy x Gz virtual-grid split.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

ROW = 0
COL = 1

def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile oracle.c (or another source, for planted-mistake tests) with gcc + OpenMP."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
               "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _u16(a: np.ndarray):
    assert a.dtype == np.uint16 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def _idx(sel: Optional[Sequence[int]], n: int) -> np.ndarray:
    if sel is None:
        return np.arange(n, dtype=np.int64)
    a = np.ascontiguousarray(np.asarray(sel, dtype=np.int64))
    if a.size and (a.min() < 0 or a.max() >= n):
        raise IndexError("sample index out of range")
    return a


class Oracle:
    """The oracle's entry points, bound to one build of oracle.c."""

    def __init__(self, lib_path: str = _LIB_PATH):
        lib = ctypes.CDLL(lib_path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        i64p = ctypes.POINTER(ctypes.c_int64)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        lib.oracle_fc_fwd.argtypes = [u16p, ci, u16p, ci, i64, i64, i64, i64p, i64, i64p, i64, f64p, f64p]
        lib.oracle_fc_bwd_data.argtypes = [u16p, u16p, ci, i64, i64, i64, i64p, i64, i64p, i64, f64p, f64p]
        lib.oracle_fc_bwd_weight.argtypes = [u16p, ci, u16p, i64, i64, i64, i64p, i64, i64p, i64, f64p, f64p]
        for f in (lib.oracle_fc_fwd, lib.oracle_fc_bwd_data, lib.oracle_fc_bwd_weight):
            f.restype = ci
        lib.oracle_round_bf16.argtypes = [f64p, i64, u16p]
        lib.oracle_round_bf16.restype = None
        self.lib = lib
        self.path = lib_path

    @staticmethod
    def _run(fn, args, n_rows_total, n_cols_total, rows, cols):
        r = _idx(rows, n_rows_total)
        c = _idx(cols, n_cols_total)
        O = np.empty((r.size, c.size), dtype=np.float64)
        S = np.empty((r.size, c.size), dtype=np.float64)
        i64p = ctypes.POINTER(ctypes.c_int64)
        f64p = ctypes.POINTER(ctypes.c_double)
        rc = fn(*args, r.ctypes.data_as(i64p), r.size, c.ctypes.data_as(i64p), c.size,
                O.ctypes.data_as(f64p), S.ctypes.data_as(f64p))
        if rc != 0:
            raise RuntimeError(f"oracle failed with code {rc}")
        return O, S

    def fc_fwd(self, X, x_order, W, w_order, M, K, N, rows=None, cols=None):
        """Y = X . W in fp64 over exact bf16 values; returns (Y[rows, cols], S)."""
        return self._run(self.lib.oracle_fc_fwd, (_u16(X), x_order, _u16(W), w_order, M, K, N),
                         M, N, rows, cols)

    def fc_bwd_data(self, dY, W, w_order, M, K, N, rows=None, cols=None):
        """dX = dY . W^T in fp64; rows index tokens m, cols index input features k."""
        return self._run(self.lib.oracle_fc_bwd_data, (_u16(dY), _u16(W), w_order, M, K, N),
                         M, K, rows, cols)

    def fc_bwd_weight(self, X, x_order, dY, M, K, N, rows=None, cols=None):
        """dW = X^T . dY in fp64; rows index input features k, cols output features n."""
        return self._run(self.lib.oracle_fc_bwd_weight, (_u16(X), x_order, _u16(dY), M, K, N),
                         K, N, rows, cols)

    def round_bf16(self, v: np.ndarray) -> np.ndarray:
        """Nearest-even bf16 bit patterns of exact fp64 values (no double rounding)."""
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.oracle_round_bf16(v.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), v.size,
                                   out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)))
        return out


_default: Optional[Oracle] = None


def default() -> Oracle:
    """The oracle built from oracle.c (rebuilt when the source is newer)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        _default = Oracle(_LIB_PATH)
    return _default


def fc_fwd(X, x_order, W, w_order, M, K, N, rows=None, cols=None) -> Tuple[np.ndarray, np.ndarray]:
    """Y = X . W (see Oracle.fc_fwd)."""
    return default().fc_fwd(X, x_order, W, w_order, M, K, N, rows, cols)


def fc_bwd_data(dY, W, w_order, M, K, N, rows=None, cols=None) -> Tuple[np.ndarray, np.ndarray]:
    """dX = dY . W^T (see Oracle.fc_bwd_data)."""
    return default().fc_bwd_data(dY, W, w_order, M, K, N, rows, cols)


def fc_bwd_weight(X, x_order, dY, M, K, N, rows=None, cols=None) -> Tuple[np.ndarray, np.ndarray]:
    """dW = X^T . dY (see Oracle.fc_bwd_weight)."""
    return default().fc_bwd_weight(X, x_order, dY, M, K, N, rows, cols)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 of exact fp64 values (see Oracle.round_bf16)."""
    return default().round_bf16(v)


def accumulate(C_old: np.ndarray, P: np.ndarray, S: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """An accumulating output: the fp32 values it held plus the exact product P.

    Gradient accumulation over micro-batches adds each micro-batch's product to
    the running fp32 sum (the pages are silent on it; this is its plain
    definition). Returns (C_old + P, |C_old| + S) in fp64: the value and the
    magnitude scale that the tolerance applies to.
    """
    C = np.asarray(C_old, dtype=np.float64)
    return C + P, np.abs(C) + S


def compare(G: np.ndarray, O: np.ndarray, S: np.ndarray, elem_tol: float = 1e-2,
            fro_tol: float = 5e-3) -> dict:
    """Tolerance check of a GPU result G (any float dtype) against (O, S).

    The bound of the shard products: the elementwise error is at most
    elem_tol times the magnitude scale S = |A|.|B| of that element, and the
    relative Frobenius error ||G - O|| / ||O|| is at most fro_tol; both must
    hold. A zero scale S demands an exact match of that element. When O is
    zero everywhere the relative error is 0 for an exact match and infinite
    otherwise. A NaN or an infinity in G is never within the bound.
    """
    G = np.asarray(G, dtype=np.float64)
    O = np.asarray(O, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    if G.shape != O.shape or S.shape != O.shape:
        raise ValueError(f"shapes differ: G {G.shape}, O {O.shape}, S {S.shape}")
    finite = bool(np.all(np.isfinite(G)))
    err = np.abs(G - O)
    bound = elem_tol * S
    with np.errstate(invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    max_ratio = float(ratio.max()) if ratio.size else 0.0
    on = float(np.linalg.norm(O))
    diff = float(np.linalg.norm(G - O)) if finite else float("inf")
    if on > 0:
        rel_fro = diff / on
    else:
        rel_fro = 0.0 if diff == 0 else float("inf")
    if not finite:
        max_ratio = float("inf")
    return {"max_err_ratio": max_ratio, "rel_fro": rel_fro,
            "pass": bool(finite and max_ratio <= 1.0 and rel_fro <= fro_tol)}
