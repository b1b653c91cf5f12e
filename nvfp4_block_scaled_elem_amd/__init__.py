"""Python binding of the gfx950 NVFP4 weight quantizer (``libnvfp4.so``; C ABI in ``include/nvfp4.h``).

Argument marshalling only: tensors are torch CUDA (HIP) tensors, every step of the computation runs in
the HIP kernels behind the C ABI, and there is no CPU fallback. A missing library raises at first use.

    codes, scales, alpha = quantize(W, "4o6")          # W: [rows, cols] bf16 or fp32, cols % 16 == 0
    W_hat = dequantize(codes, scales, alpha, torch.bfloat16)

Modes: "max" (max rule), "4o6" (FourOverSix), "cjso" (closed-form joint scale optimisation, ``iters``
rounds), "soar" (CJSO then the decoupled quantise/dequantise scale search).
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("NVFP4_LIB", os.path.join(HERE, "libnvfp4.so"))

MODES = {"max": 0, "4o6": 1, "cjso": 2, "soar": 3}
DTYPES = {torch.bfloat16: 0, torch.float32: 1}
FLAG_FULL_SEARCH = 1  # NVFP4_FLAG_FULL_SEARCH
FLAG_INIT_4O6 = 2  # NVFP4_FLAG_INIT_4O6
INITS = {"max": 0, "4o6": FLAG_INIT_4O6}
DD_RULES = {"cjso": 0, "quant": 1, "lsq": 2}  # enum nvfp4_dd_rule
SEARCH_MAX_COUNT = 1024
STATUS_NONFINITE = 1


class NVFP4Error(RuntimeError):
    pass


class _Args(ctypes.Structure):
    _fields_ = [
        ("W", ctypes.c_void_p), ("dtype", ctypes.c_int), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
        ("mode", ctypes.c_int), ("iters", ctypes.c_int), ("codes_out", ctypes.c_void_p),
        ("scales_out", ctypes.c_void_p), ("alpha_out", ctypes.c_void_p), ("mchoice_out", ctypes.c_void_p),
        ("stats_out", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p), ("stage_events", ctypes.c_void_p), ("n_stage_events", ctypes.c_int),
        ("flags", ctypes.c_uint), ("search_num0", ctypes.c_int), ("search_den", ctypes.c_int),
        ("search_count", ctypes.c_int), ("dd_rule", ctypes.c_int),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise NVFP4Error(f"{LIB_PATH} is missing: build it with `python nvfp4_block_scaled_elem_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.nvfp4_error_stats.argtypes = [vp, i32, i64, i64, vp, vp, vp, vp, vp, vp]
        L.nvfp4_error_stats.restype = i32
        L.nvfp4_matmul.argtypes = [vp, i64, i64, vp, vp, vp, i64, vp, i32, vp]
        L.nvfp4_matmul.restype = i32
        L.nvfp4_matmul_ex.argtypes = [vp, i64, i64, vp, vp, vp, i64, vp, i32, vp, ctypes.c_size_t, vp]
        L.nvfp4_matmul_ex.restype = i32
        L.nvfp4_matmul_workspace_bytes.argtypes = [i64, i64, i64]
        L.nvfp4_matmul_workspace_bytes.restype = ctypes.c_size_t
        L.nvfp4_matmul_plan.argtypes = [i64, i64, i64, vp]
        L.nvfp4_matmul_plan.restype = i32
        L.nvfp4_quantize_ex.argtypes = [ctypes.POINTER(_Args)]
        L.nvfp4_quantize_ex.restype = i32
        L.nvfp4_quantize.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, vp]
        L.nvfp4_quantize.restype = i32
        L.nvfp4_quantize_f32.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, vp]
        L.nvfp4_quantize_f32.restype = i32
        L.nvfp4_workspace_bytes.argtypes = [i64, i64, i32]
        L.nvfp4_workspace_bytes.restype = ctypes.c_size_t
        L.nvfp4_kernel_count.argtypes = [i32, i32]
        L.nvfp4_kernel_count.restype = i32
        L.nvfp4_encode_e2m1.argtypes = [vp, i64, vp, vp]
        L.nvfp4_encode_e2m1.restype = i32
        L.nvfp4_reciprocal_f32.argtypes = [vp, i64, vp, vp]
        L.nvfp4_reciprocal_f32.restype = i32
        L.nvfp4_dequantize.argtypes = [vp, vp, vp, i64, i64, vp, i32, vp]
        L.nvfp4_dequantize.restype = i32
        L.nvfp4_gptq.argtypes = [vp, i32, i64, i64, vp, ctypes.c_double, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.nvfp4_gptq.restype = i32
        L.nvfp4_gptq_workspace_bytes.argtypes = [i64, i64]
        L.nvfp4_gptq_workspace_bytes.restype = ctypes.c_size_t
        L.nvfp4_status_string.argtypes = [i32]
        L.nvfp4_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().nvfp4_status_string(status).decode()


def _check(status: int) -> None:
    if status != 0:
        raise NVFP4Error(f"nvfp4: {status_string(status)} ({status})")


def workspace_bytes(rows: int, cols: int, mode: str) -> int:
    return int(lib().nvfp4_workspace_bytes(rows, cols, MODES[mode]))


def kernel_count(mode: str, iters: int = 0) -> int:
    return int(lib().nvfp4_kernel_count(MODES[mode], iters))


STATS_BYTES = 16  # sizeof(nvfp4_stats_t)


def _check_buffer(t, name: str, nbytes: int, dev, dtype=None) -> None:
    """A caller-supplied buffer must be a contiguous tensor on `dev`, of `dtype` when one is given, holding
    at least `nbytes` bytes: the kernels write through its pointer without knowing its size."""
    if not t.is_cuda or t.device != dev or not t.is_contiguous():
        raise NVFP4Error(f"{name} must be a contiguous tensor on {dev}")
    if dtype is not None and t.dtype != dtype:
        raise NVFP4Error(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() * t.element_size() < nbytes:
        raise NVFP4Error(f"{name} holds {t.numel() * t.element_size()} bytes, {nbytes} needed")


def _scratch(nbytes: int, dev, stream) -> torch.Tensor:
    """A uint8 scratch tensor for one call on `stream` (the current stream when None). Torch's allocator
    may hand the memory out again once the tensor is dropped; recording the call's stream keeps it from
    doing so before the work enqueued on that stream has run."""
    t = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if stream is not None:
        t.record_stream(stream)
    return t


def _stream_ptr(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def quantize(W: torch.Tensor, mode: str, iters: int = 0, *, codes=None, scales=None, alpha=None,
             mchoice=None, stats=None, workspace=None, stream=None, stage_events=None, full_search=False,
             init="max", grid=None, dd_rule="cjso"):
    """Quantise ``W`` ([rows, cols] bf16/fp32 CUDA tensor). Returns (codes [rows, cols//2] uint8,
    scales [rows, cols//16] uint8 E4M3 bits, alpha [1] float32), all on W's device. Optional
    preallocated outputs, an ``mchoice`` uint8 [rows, cols//16] tensor (FourOverSix), a ``stats``
    int32 [4] tensor, a uint8 ``workspace`` tensor, a ``stream`` and a list of
    ``torch.cuda.Event(enable_timing=True)`` stage events (None entries are skipped) may be passed. ``full_search`` makes the
    SOAR search visit all 202 candidates of every block (same outputs; NVFP4_FLAG_FULL_SEARCH); ``init``
    is CJSO's starting point, "max" or "4o6" (NVFP4_FLAG_INIT_4O6; modes cjso and soar). For mode soar,
    ``grid`` = (num0, den, count) sets the search multipliers (nearest binary32 of (num0 + k)/den,
    k < count; None for the page's 50, 100, 101) and ``dd_rule`` ("cjso", "quant" or "lsq") the rule
    for each candidate's reconstruct scales."""
    if W.dim() != 2 or not W.is_cuda or not W.is_contiguous() or W.dtype not in DTYPES:
        raise NVFP4Error("W must be a contiguous 2-D bf16 or fp32 CUDA tensor")
    rows, cols = W.shape
    dev = W.device
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    if alpha is None:
        alpha = torch.empty(1, dtype=torch.float32, device=dev)
    if mode not in MODES:
        raise NVFP4Error(f"unknown mode {mode!r}")
    nel = rows * cols
    _check_buffer(codes, "codes", nel // 2, dev, torch.uint8)
    _check_buffer(scales, "scales", nel // 16, dev, torch.uint8)
    _check_buffer(alpha, "alpha", 4, dev, torch.float32)
    if mchoice is not None:
        _check_buffer(mchoice, "mchoice", nel // 16, dev, torch.uint8)
    if stats is not None:
        _check_buffer(stats, "stats", STATS_BYTES, dev)
    if workspace is not None:
        _check_buffer(workspace, "workspace", 0, dev)
    need = workspace_bytes(rows, cols, mode) if cols % 16 == 0 and rows > 0 else 0
    if workspace is None and need:
        workspace = _scratch(need, dev, stream)
    a = _Args()
    a.W = W.data_ptr()
    a.dtype = DTYPES[W.dtype]
    a.rows, a.cols = rows, cols
    a.mode = MODES[mode]
    a.iters = iters
    a.codes_out = codes.data_ptr()
    a.scales_out = scales.data_ptr()
    a.alpha_out = alpha.data_ptr()
    a.mchoice_out = mchoice.data_ptr() if mchoice is not None else None
    a.stats_out = stats.data_ptr() if stats is not None else None
    a.workspace = workspace.data_ptr() if workspace is not None else None
    a.workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    a.stream = _stream_ptr(stream, dev)
    if init not in INITS:
        raise NVFP4Error(f"unknown init {init!r}")
    a.flags = (FLAG_FULL_SEARCH if full_search else 0) | INITS[init]
    if dd_rule not in DD_RULES:
        raise NVFP4Error(f"unknown dd_rule {dd_rule!r}")
    a.dd_rule = DD_RULES[dd_rule]
    if grid is not None:
        a.search_num0, a.search_den, a.search_count = (int(v) for v in grid)
    ev_arr = None
    if stage_events is not None:
        for e in stage_events:  # torch creates the HIP event at its first record
            if e is not None and not e.cuda_event:
                e.record(stream if stream is not None else torch.cuda.current_stream(dev))
        ev_arr = (ctypes.c_void_p * len(stage_events))(
            *[e.cuda_event if e is not None else None for e in stage_events])
        a.stage_events = ctypes.cast(ev_arr, ctypes.c_void_p)
        a.n_stage_events = len(stage_events)
    with torch.cuda.device(dev):
        _check(lib().nvfp4_quantize_ex(ctypes.byref(a)))
    return codes, scales, alpha


def gptq_workspace_bytes(rows: int, cols: int) -> int:
    return int(lib().nvfp4_gptq_workspace_bytes(rows, cols))


def gptq(W: torch.Tensor, H: torch.Tensor, percdamp: float = 0.01, *, codes=None, scales=None, alpha=None,
         workspace=None, stream=None):
    """GPTQ codes for ``W`` ([rows, cols] bf16/fp32 CUDA tensor) inside the FourOverSix frame (block
    scales and alpha fixed first), with ``H`` the [cols, cols] float64 second moment of the layer's
    inputs (symmetric; its upper triangle is read) and GPTQ's damping fraction ``percdamp``. Returns
    (codes, scales, alpha) laid out as ``quantize`` returns them; alpha is NaN if the damped H is not
    positive definite. Optional preallocated outputs, a uint8 ``workspace`` tensor and a ``stream``."""
    if W.dim() != 2 or not W.is_cuda or not W.is_contiguous() or W.dtype not in DTYPES:
        raise NVFP4Error("W must be a contiguous 2-D bf16 or fp32 CUDA tensor")
    rows, cols = W.shape
    dev = W.device
    if H.dim() != 2 or tuple(H.shape) != (cols, cols):
        raise NVFP4Error("H must be [cols, cols]")
    _check_buffer(H, "H", cols * cols * 8, dev, torch.float64)
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    if alpha is None:
        alpha = torch.empty(1, dtype=torch.float32, device=dev)
    nel = rows * cols
    _check_buffer(codes, "codes", nel // 2, dev, torch.uint8)
    _check_buffer(scales, "scales", nel // 16, dev, torch.uint8)
    _check_buffer(alpha, "alpha", 4, dev, torch.float32)
    if workspace is not None:
        _check_buffer(workspace, "workspace", 0, dev)
    need = gptq_workspace_bytes(rows, cols)
    if workspace is None and need:
        workspace = _scratch(need, dev, stream)
    with torch.cuda.device(dev):
        _check(lib().nvfp4_gptq(W.data_ptr(), DTYPES[W.dtype], rows, cols, H.data_ptr(), float(percdamp),
                                codes.data_ptr(), scales.data_ptr(), alpha.data_ptr(),
                                workspace.data_ptr() if workspace is not None else None,
                                workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                _stream_ptr(stream, dev)))
    return codes, scales, alpha


def encode_e2m1(x: torch.Tensor, stream=None) -> torch.Tensor:
    """E2M1 codes (one per byte) of a contiguous fp32 CUDA tensor."""
    if not x.is_cuda or x.dtype != torch.float32 or not x.is_contiguous():
        raise NVFP4Error("x must be a contiguous fp32 CUDA tensor")
    out = torch.empty(x.numel(), dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib().nvfp4_encode_e2m1(x.data_ptr(), x.numel(), out.data_ptr(), _stream_ptr(stream, x.device)))
    return out.view(x.shape)


def reciprocal_f32(s: torch.Tensor, stream=None) -> torch.Tensor:
    """fl(1/s) element-wise by the reciprocal the search kernel uses (contiguous fp32 CUDA tensor)."""
    if not s.is_cuda or s.dtype != torch.float32 or not s.is_contiguous():
        raise NVFP4Error("s must be a contiguous fp32 CUDA tensor")
    out = torch.empty_like(s)
    with torch.cuda.device(s.device):
        _check(lib().nvfp4_reciprocal_f32(s.data_ptr(), s.numel(), out.data_ptr(), _stream_ptr(stream, s.device)))
    return out


def dequantize(codes: torch.Tensor, scales: torch.Tensor, alpha: torch.Tensor, dtype=torch.bfloat16,
               stream=None) -> torch.Tensor:
    """W_hat = e2m1(code) * e4m3(scale) * alpha as a [rows, cols] bf16 or fp32 tensor."""
    if codes.dim() != 2:
        raise NVFP4Error("codes must be [rows, cols/2]")
    if dtype not in DTYPES:
        raise NVFP4Error("dtype must be bf16 or fp32")
    rows, half = codes.shape
    cols = 2 * half
    dev = codes.device
    _check_buffer(codes, "codes", rows * half, dev, torch.uint8)
    _check_buffer(scales, "scales", rows * cols // 16, dev, torch.uint8)
    _check_buffer(alpha, "alpha", 4, dev, torch.float32)
    out = torch.empty((rows, cols), dtype=dtype, device=dev)
    with torch.cuda.device(dev):
        _check(lib().nvfp4_dequantize(codes.data_ptr(), scales.data_ptr(), alpha.data_ptr(), rows, cols,
                                      out.data_ptr(), DTYPES[dtype], _stream_ptr(stream, dev)))
    return out


def error_stats(W: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, alpha: torch.Tensor, stream=None):
    """Reconstruction statistics of an encoding of ``W`` (all CUDA tensors, as quantize returns them):
    returns (sse float64 tensor [1], hist int64 tensor [16]) on W's device, where sse is the sum of squared
    differences between W and e2m1(code) * e4m3(scale) * alpha and hist[c] counts the elements with code c."""
    if W.dim() != 2 or not W.is_cuda or not W.is_contiguous() or W.dtype not in DTYPES:
        raise NVFP4Error("W must be a contiguous 2-D bf16 or fp32 CUDA tensor")
    rows, cols = W.shape
    dev = W.device
    _check_buffer(codes, "codes", rows * cols // 2, dev, torch.uint8)
    _check_buffer(scales, "scales", rows * cols // 16, dev, torch.uint8)
    _check_buffer(alpha, "alpha", 4, dev, torch.float32)
    sse = torch.empty(1, dtype=torch.float64, device=dev)
    hist = torch.empty(16, dtype=torch.int64, device=dev)
    with torch.cuda.device(dev):
        _check(lib().nvfp4_error_stats(W.data_ptr(), DTYPES[W.dtype], rows, cols, codes.data_ptr(),
                                       scales.data_ptr(), alpha.data_ptr(), sse.data_ptr(), hist.data_ptr(),
                                       _stream_ptr(stream, dev)))
    return sse, hist


def matmul_workspace_bytes(M: int, K: int, N: int) -> int:
    return int(lib().nvfp4_matmul_workspace_bytes(M, K, N))


PLAN_FIELDS = ("kind", "tm", "tn", "tiles_n", "tiles", "slices", "kslice", "grid", "reduce_grid", "part_bytes")


def matmul_plan(M: int, K: int, N: int) -> dict:
    """The launch nvfp4_matmul takes for these shapes (host only): kernel kind (0 GEMV, 1 skinny, 2 tiled),
    tile shape, K split and grid sizes."""
    out = (ctypes.c_int64 * len(PLAN_FIELDS))()
    _check(lib().nvfp4_matmul_plan(M, K, N, ctypes.cast(out, ctypes.c_void_p)))
    return dict(zip(PLAN_FIELDS, (int(v) for v in out)))


def matmul(X: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, alpha: torch.Tensor,
           out_dtype=torch.bfloat16, stream=None, out: torch.Tensor = None, workspace=None) -> torch.Tensor:
    """W4A16 product Y = X @ What.T with NVFP4 weights (codes [N, K/2], scales [N, K/16], alpha [1] as
    quantize returns them for an [N, K] matrix) and bf16 activations X [M, K]; Y is [M, N] bf16 or fp32,
    written into `out` when one is given (contiguous, on X's device, of that shape and out_dtype). The
    K-split scratch (matmul_workspace_bytes) is a torch tensor: the caller's uint8 `workspace`, or one
    allocated here, so the library itself never allocates (a graph capture records kernels only)."""
    if X.dim() != 2 or not X.is_cuda or not X.is_contiguous() or X.dtype != torch.bfloat16:
        raise NVFP4Error("X must be a contiguous 2-D bf16 CUDA tensor")
    M, K = X.shape
    dev = X.device
    if codes.dim() != 2 or codes.shape[1] * 2 != K:
        raise NVFP4Error("codes must be [N, K/2]")
    N = codes.shape[0]
    _check_buffer(codes, "codes", N * K // 2, dev, torch.uint8)
    _check_buffer(scales, "scales", N * K // 16, dev, torch.uint8)
    _check_buffer(alpha, "alpha", 4, dev, torch.float32)
    if out_dtype not in DTYPES:
        raise NVFP4Error("out_dtype must be bf16 or fp32")
    if out is None:
        Y = torch.empty((M, N), dtype=out_dtype, device=dev)
    else:
        if (out.shape != (M, N) or out.dtype != out_dtype or not out.is_cuda or out.device != dev
                or not out.is_contiguous()):
            raise NVFP4Error("out must be a contiguous [M, N] tensor of out_dtype on X's device")
        Y = out
    need = matmul_workspace_bytes(M, K, N)
    if workspace is not None:
        _check_buffer(workspace, "workspace", need, dev)
    elif need:
        workspace = _scratch(need, dev, stream)
    with torch.cuda.device(dev):
        _check(lib().nvfp4_matmul_ex(X.data_ptr(), M, K, codes.data_ptr(), scales.data_ptr(), alpha.data_ptr(), N,
                                     Y.data_ptr(), DTYPES[out_dtype],
                                     workspace.data_ptr() if workspace is not None else None,
                                     workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                     _stream_ptr(stream, dev)))
    return Y
