"""Thin Python binding of libfcshard.so (the C ABI declared in include/fcshard.h).

Argument marshalling only: every product runs in the library's HIP kernels.
PyTorch supplies device memory (torch.Tensor) and the current HIP stream.
If the library is not built, every call raises: there is no fallback.

Storage conventions follow the ABI: X is M x K and W is K x N as logical
matrices, each stored row-major (ROW) or column-major (COL); a COL matrix is
passed as the tensor of its transpose (e.g. nn.Linear.weight, N x K, is W in
COL). dY, Y, dX and dW are row-major.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import List, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfcshard.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "fcshard.h")

ROW, COL = 0, 1                # fc_order
OUT_BF16, OUT_F32, OUT_F32_ACC = 0, 1, 2  # fc_out_dtype (OUT_F32_ACC: fp32 out += product)
OP_FWD, OP_BWD_DATA, OP_BWD_WEIGHT = 0, 1, 2  # fc_op
FC_OK, FC_E_INVALID, FC_E_UNSUPPORTED, FC_E_HIP, FC_E_NOMEM, FC_E_TOO_LARGE = 0, 1, 2, 3, 4, 5

_lib = None


class MfmaProbeResult(ctypes.Structure):
    """fc_mfma_probe_result of include/fcshard.h."""
    _fields_ = [("ms", ctypes.c_double), ("flops", ctypes.c_double), ("compute_units", ctypes.c_int),
                ("counter_ratio", ctypes.c_double), ("wall_clock_mhz", ctypes.c_double)]


class FcError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)}")
        self.status = status


def header_functions() -> List[str]:
    """Names of the functions that include/fcshard.h declares."""
    text = open(HEADER).read()
    return re.findall(r"^\s*(?:fc_status|int|int64_t|const char\*)\s+(fc_\w+)\s*\(", text, re.M)


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sharded_fc_layer_amd.build`")
        # torch carries its own HIP runtime. Loaded first, it also serves this
        # library's HIP dependency, so torch's memory and streams and this
        # library's calls live in one runtime; loaded after, the process would
        # hold two runtimes and this library's calls fail.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, ci, cs = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.fc_fwd.argtypes = [vp, ci, vp, ci, vp, ci, i64, i64, i64, vp]
        L.fc_bwd_data.argtypes = [vp, vp, ci, vp, ci, i64, i64, i64, vp]
        L.fc_bwd_weight.argtypes = [vp, ci, vp, vp, ci, i64, i64, i64, vp]
        L.fc_bwd_weight_noalloc.argtypes = [vp, ci, vp, vp, ci, i64, i64, i64, vp]
        L.fc_noalloc_scratch_bytes.argtypes = []
        L.fc_noalloc_scratch_bytes.restype = i64
        L.fc_tune.argtypes = [i64, i64, i64, ci, ci, ci, ci, vp]
        L.fc_set_plan.argtypes = [ci, i64, i64, i64, ci, ci, ci, ci]
        L.fc_plan_describe.argtypes = [ci, i64, i64, i64, ci, ci, ci, ctypes.c_char_p, cs]
        L.fc_plan_count.argtypes = []
        L.fc_status_str.argtypes = [ci]
        L.fc_status_str.restype = ctypes.c_char_p
        L.fc_release.argtypes = []
        L.fc_plans_save.argtypes = [ctypes.c_char_p]
        L.fc_plans_load.argtypes = [ctypes.c_char_p]
        L.fc_mfma_probe.argtypes = [i64, ctypes.POINTER(MfmaProbeResult), vp]
        L.fc_mfma_probe_launch.argtypes = [i64, ci, vp, vp]
        L.fc_stamped_call.argtypes = [ci, vp, ci, vp, ci, vp, ci, i64, i64, i64, vp, i64,
                                      ctypes.POINTER(i64), vp]
        for f in (L.fc_fwd, L.fc_bwd_data, L.fc_bwd_weight, L.fc_bwd_weight_noalloc, L.fc_tune, L.fc_set_plan, L.fc_plan_describe,
                  L.fc_plan_count, L.fc_release, L.fc_plans_save, L.fc_plans_load, L.fc_mfma_probe,
                  L.fc_mfma_probe_launch, L.fc_stamped_call):
            f.restype = ci
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().fc_status_str(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != FC_OK:
        raise FcError(status, what)


def _stream(stream) -> Optional[int]:
    """A hipStream_t handle: from a torch.cuda.Stream, an int, or torch's current stream."""
    if stream is not None:
        return int(getattr(stream, "cuda_stream", stream))
    import torch
    return torch.cuda.current_stream().cuda_stream


def _bf16_2d(t, name: str):
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D torch.bfloat16 tensor")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous CUDA/HIP tensor")
    return t


def _logical(t, order: int):
    """(rows, cols) of the logical matrix whose storage is tensor t."""
    r, c = t.shape
    return (r, c) if order == ROW else (c, r)


def _out(out, rows: int, cols: int, out_dtype: int, like, name: str, stream=None):
    """The output tensor: `out` checked, or a new one allocated on the stream that
    writes it (so torch's caching allocator does not hand its memory to other
    work on another stream while the kernels still write it)."""
    import torch
    dt = torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32
    if out is None:
        if out_dtype == OUT_F32_ACC:
            raise ValueError(f"{name}: accumulating needs the existing output tensor (out=)")
        if stream is None or _stream(stream) == torch.cuda.current_stream().cuda_stream:
            return torch.empty((rows, cols), dtype=dt, device=like.device)
        ts = stream if isinstance(stream, torch.cuda.Stream) else \
            torch.cuda.ExternalStream(_stream(stream), device=like.device)
        with torch.cuda.stream(ts):
            return torch.empty((rows, cols), dtype=dt, device=like.device)
    if out.dtype != dt or tuple(out.shape) != (rows, cols) or not out.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dt} tensor of shape {(rows, cols)}")
    if not out.is_cuda:
        raise ValueError(f"{name} must be a CUDA/HIP tensor")
    return out


def _one_device(*ts) -> None:
    """The library runs on the current device: every tensor must live there."""
    import torch
    cur = torch.cuda.current_device()
    for t in ts:
        if t.device.index != cur:
            raise ValueError(f"a tensor is on {t.device}, but the current device is cuda:{cur}")


def fc_fwd(X, W, x_order: int = ROW, w_order: int = ROW, out=None, out_dtype: int = OUT_BF16, stream=None):
    """Y = X . W on the GPU; returns Y (M x N, row-major)."""
    _bf16_2d(X, "X"), _bf16_2d(W, "W")
    M, K = _logical(X, x_order)
    K2, N = _logical(W, w_order)
    if K2 != K:
        raise ValueError(f"inner dimensions differ: X is {M}x{K}, W is {K2}x{N}")
    Y = _out(out, M, N, out_dtype, X, "out", stream)
    _one_device(X, W, Y)
    _check(lib().fc_fwd(X.data_ptr(), x_order, W.data_ptr(), w_order, Y.data_ptr(), out_dtype, M, K, N,
                        _stream(stream)), "fc_fwd")
    return Y


def fc_bwd_data(dY, W, w_order: int = ROW, out=None, out_dtype: int = OUT_BF16, stream=None):
    """dX = dY . W^T on the GPU; returns dX (M x K, row-major)."""
    _bf16_2d(dY, "dY"), _bf16_2d(W, "W")
    M, N = dY.shape
    K, N2 = _logical(W, w_order)
    if N2 != N:
        raise ValueError(f"dY is {M}x{N} but W is {K}x{N2}")
    dX = _out(out, M, K, out_dtype, dY, "out", stream)
    _one_device(dY, W, dX)
    _check(lib().fc_bwd_data(dY.data_ptr(), W.data_ptr(), w_order, dX.data_ptr(), out_dtype, M, K, N,
                             _stream(stream)), "fc_bwd_data")
    return dX


def fc_bwd_weight(X, dY, x_order: int = ROW, out=None, out_dtype: int = OUT_BF16, stream=None):
    """dW = X^T . dY on the GPU; returns dW (K x N, row-major)."""
    _bf16_2d(X, "X"), _bf16_2d(dY, "dY")
    M, K = _logical(X, x_order)
    M2, N = dY.shape
    if M2 != M:
        raise ValueError(f"X is {M}x{K} but dY is {M2}x{N}")
    dW = _out(out, K, N, out_dtype, X, "out", stream)
    _one_device(X, dY, dW)
    _check(lib().fc_bwd_weight(X.data_ptr(), x_order, dY.data_ptr(), dW.data_ptr(), out_dtype, M, K, N,
                               _stream(stream)), "fc_bwd_weight")
    return dW


def fc_bwd_weight_noalloc(X, dY, x_order: int = ROW, out=None, out_dtype: int = OUT_BF16, stream=None):
    """dW = X^T . dY as fc_bwd_weight, with the plan's staging in the library's
    static device scratch instead of its workspace (the library allocates
    nothing; pass out= for a call that allocates nothing at all)."""
    _bf16_2d(X, "X"), _bf16_2d(dY, "dY")
    M, K = _logical(X, x_order)
    M2, N = dY.shape
    if M2 != M:
        raise ValueError(f"X is {M}x{K} but dY is {M2}x{N}")
    dW = _out(out, K, N, out_dtype, X, "out", stream)
    _one_device(X, dY, dW)
    _check(lib().fc_bwd_weight_noalloc(X.data_ptr(), x_order, dY.data_ptr(), dW.data_ptr(), out_dtype, M, K, N,
                                       _stream(stream)), "fc_bwd_weight_noalloc")
    return dW


STAMP_SLOTS = 8  # values per block written by fc_stamped_call


def fc_stamped(op: int, A, B, a_order: int = ROW, b_order: int = ROW, out=None, stamps=None, stream=None):
    """One product with cycle stamps (fc_stamped_call, a measurement aid): the
    same plan and result as the hot call of `op`, with the ring kernel writing
    STAMP_SLOTS counter readings per block.

    op = OP_FWD: A = X (a_order), B = W (b_order); OP_BWD_DATA: A = dY, B = W
    (b_order); OP_BWD_WEIGHT: A = X (a_order), B = dY. The output is bf16.
    Returns (out, stamps): stamps an int64 CUDA tensor (blocks, STAMP_SLOTS),
    laid out as fcshard.h describes. Raises FcError with FC_E_UNSUPPORTED when
    the op's plan has no stamped form (nothing is enqueued then)."""
    import torch
    _bf16_2d(A, "A"), _bf16_2d(B, "B")
    if op == OP_FWD:
        M, K = _logical(A, a_order)
        K2, N = _logical(B, b_order)
        if K2 != K:
            raise ValueError(f"inner dimensions differ: X is {M}x{K}, W is {K2}x{N}")
        rows, cols = M, N
    elif op == OP_BWD_DATA:
        M, N = A.shape
        K, N2 = _logical(B, b_order)
        if N2 != N:
            raise ValueError(f"dY is {M}x{N} but W is {K}x{N2}")
        rows, cols = M, K
    elif op == OP_BWD_WEIGHT:
        M, K = _logical(A, a_order)
        M2, N = B.shape
        if M2 != M:
            raise ValueError(f"X is {M}x{K} but dY is {M2}x{N}")
        rows, cols = K, N
    else:
        raise ValueError(f"unknown op {op}")
    C = _out(out, rows, cols, OUT_BF16, A, "out", stream)
    nb = ((rows + 255) // 256) * ((cols + 255) // 256)
    if stamps is None:
        stamps = torch.zeros((nb, STAMP_SLOTS), dtype=torch.int64, device=A.device)
    if not isinstance(stamps, torch.Tensor) or stamps.dtype != torch.int64 or not stamps.is_cuda \
            or not stamps.is_contiguous() or stamps.dim() != 2 or stamps.shape[1] != STAMP_SLOTS:
        raise ValueError(f"stamps must be a contiguous int64 CUDA tensor of shape (blocks, {STAMP_SLOTS})")
    _one_device(A, B, C, stamps)
    blocks = ctypes.c_int64(0)
    _check(lib().fc_stamped_call(op, A.data_ptr(), a_order, B.data_ptr(), b_order, C.data_ptr(), OUT_BF16,
                                 M, K, N, stamps.data_ptr(), stamps.numel() * 8, ctypes.byref(blocks),
                                 _stream(stream)), "fc_stamped_call")
    return C, stamps[:blocks.value]


def summarize_stamps(stamps, wall_clock_mhz: float, compute_units: Optional[int] = None) -> dict:
    """Per-launch figures from fc_stamped_call's stamps (an integer array of
    shape (blocks, STAMP_SLOTS), on the host): the engine clock while the
    blocks ran (shader-clock ticks over constant-rate ticks), and the mean
    cycles of each block's set-up, prologue (the first stage landing),
    main loop per reduction stage, and epilogue (the output store).

    With compute_units (the stamps of ONE launch), also the launch's span from
    its first block's entry to its last block's exit, in microseconds of the
    constant-rate counter, and the CUs' occupancy: the blocks' summed lifetimes
    over compute_units x that span (one block per CU at a time)."""
    import numpy as np
    s = np.asarray(stamps, dtype=np.float64)
    if s.ndim != 2 or s.shape[1] != STAMP_SLOTS or s.shape[0] == 0:
        raise ValueError(f"stamps must have shape (blocks, {STAMP_SLOTS}), blocks >= 1")
    real = s[:, 6] - s[:, 1]
    if np.any(real <= 0) or np.any(s[:, 7] <= 0):
        raise ValueError("stamps without elapsed time or stages")
    ticks = s[:, 5] - s[:, 0]
    out = {
        "blocks": int(s.shape[0]),
        "clock_GHz": float(ticks.sum() / real.sum() * wall_clock_mhz / 1e3),
        "setup_cycles": float((s[:, 2] - s[:, 0]).mean()),
        "prologue_cycles": float((s[:, 3] - s[:, 2]).mean()),
        "loop_cycles_per_stage": float(((s[:, 4] - s[:, 3]) / s[:, 7]).mean()),
        "epilogue_cycles": float((s[:, 5] - s[:, 4]).mean()),
        "block_cycles": float(ticks.mean()),
        "stages": float(s[:, 7].mean()),
    }
    if compute_units:
        span = float(s[:, 6].max() - s[:, 1].min())
        out["launch_span_us"] = span / wall_clock_mhz
        out["cu_occupancy"] = float(real.sum() / (compute_units * span))
    return out


def fc_noalloc_scratch_bytes() -> int:
    """Size of fc_bwd_weight_noalloc's static device scratch."""
    return int(lib().fc_noalloc_scratch_bytes())


def fc_tune(M: int, K: int, N: int, x_order: int = ROW, w_order: int = ROW, out_dtype: int = OUT_BF16,
            exhaustive: bool = False, warm_caches: bool = False, stream=None) -> None:
    """Time candidate plans of the three products at this shape and cache the fastest
    (with caches flushed before each timed launch unless warm_caches)."""
    flags = (1 if exhaustive else 0) | (2 if warm_caches else 0)
    _check(lib().fc_tune(M, K, N, x_order, w_order, out_dtype, flags, _stream(stream)), "fc_tune")


def fc_plan_count() -> int:
    return int(lib().fc_plan_count())


def fc_set_plan(op: int, M: int, K: int, N: int, x_order: int, w_order: int, out_dtype: int, plan_id: int) -> int:
    """Force a plan (or -1 to clear); returns the status (no raise, for sweeps)."""
    return int(lib().fc_set_plan(op, M, K, N, x_order, w_order, out_dtype, plan_id))


def fc_plan_describe(op: int, M: int, K: int, N: int, x_order: int = ROW, w_order: int = ROW,
                     out_dtype: int = OUT_BF16) -> dict:
    """The plan a hot call would run at this key, parsed into a dict."""
    buf = ctypes.create_string_buffer(512)
    _check(lib().fc_plan_describe(op, M, K, N, x_order, w_order, out_dtype, buf, 512), "fc_plan_describe")
    text = buf.value.decode()
    d = dict(re.findall(r"(\w+)=(gemm_\w+_kernel<[^>]*>|\S+)", text))
    for k in ("plan", "split", "copy", "pad", "ktail", "ws"):
        d[k] = int(d[k])
    if "tuned_ms" in d:
        d["tuned_ms"] = float(d["tuned_ms"])
    return d


def fc_plans_save(path: str) -> None:
    """Write the current device's cached plans to a text file."""
    _check(lib().fc_plans_save(os.fsencode(path)), "fc_plans_save")


def fc_plans_load(path: str) -> None:
    """Load plans saved by fc_plans_save (entries for this device's arch)."""
    _check(lib().fc_plans_load(os.fsencode(path)), "fc_plans_load")


def fc_release() -> None:
    _check(lib().fc_release(), "fc_release")


def fc_mfma_probe(iters: int = 100000, stream=None) -> dict:
    """The MFMA-only stream of the GEMM kernels on every compute unit (measurement
    aid): launch time, flops, compute units and the shader-clock counter ratio."""
    r = MfmaProbeResult()
    _check(lib().fc_mfma_probe(int(iters), ctypes.byref(r), _stream(stream)), "fc_mfma_probe")
    return {"ms": r.ms, "flops": r.flops, "compute_units": r.compute_units, "counter_ratio": r.counter_ratio,
            "wall_clock_mhz": r.wall_clock_mhz}


def fc_mfma_probe_launch(clocks, iters: int = 16, blocks: int = 0, stream=None) -> None:
    """Enqueue the MFMA-only kernel without waiting; block b writes its four
    counter readings to clocks[b] (an int64 CUDA tensor of shape (blocks, 4))."""
    import torch
    if not isinstance(clocks, torch.Tensor) or clocks.dtype != torch.int64 or not clocks.is_cuda \
            or not clocks.is_contiguous() or clocks.dim() != 2 or clocks.shape[1] != 4:
        raise ValueError("clocks must be a contiguous int64 CUDA tensor of shape (blocks, 4)")
    n = clocks.shape[0]
    blocks = int(blocks) or n  # one block per row of clocks by default
    if blocks > n:
        raise ValueError(f"clocks holds {n} blocks, {blocks} requested")
    _one_device(clocks)
    _check(lib().fc_mfma_probe_launch(int(iters), blocks, clocks.data_ptr(), _stream(stream)),
           "fc_mfma_probe_launch")
