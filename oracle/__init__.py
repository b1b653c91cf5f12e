"""ctypes binding of the NVFP4 quantizer oracle (``oracle/nvfp4_oracle.c``).

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this module. The product package never imports it.

Inputs are numpy arrays on the host: bf16 matrices are passed as ``uint16`` arrays holding the bf16
bit patterns, fp32 matrices as ``float32`` arrays. Outputs are numpy arrays in the product layout:
codes ``[rows, cols//2]`` uint8 (even column in the low nibble), scales ``[rows, cols//16]`` uint8
E4M3 bytes, alpha a Python float.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

MODES = {"max": 0, "4o6": 1, "cjso": 2, "soar": 3}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: -O2, no FMA contraction, no fast-math."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
               "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
        subprocess.run(cmd, check=True, cwd=HERE)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=True)
        L = ctypes.CDLL(LIB)
        vp, i64, i32, u8p = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.nvfp4_ref_quantize.argtypes = [vp, i32, i64, i64, i32, i32, u8p, u8p, vp, u8p, vp, vp]
        L.nvfp4_ref_quantize.restype = i32
        L.nvfp4_ref_quantize_ex.argtypes = [vp, i32, i64, i64, i32, i32, i32, u8p, u8p, vp, u8p, vp, vp]
        L.nvfp4_ref_quantize_ex.restype = i32
        L.nvfp4_ref_matmul.argtypes = [vp, i32, i64, i64, u8p, u8p, ctypes.c_float, i64, vp]
        L.nvfp4_ref_matmul.restype = i32
        L.nvfp4_ref_soar_blocks.argtypes = [vp, i32, i64, i64, ctypes.c_float, u8p, vp, vp, i64, u8p, u8p]
        L.nvfp4_ref_soar_blocks.restype = i32
        L.nvfp4_ref_soar_blocks_search.argtypes = [vp, i32, i64, i64, ctypes.c_float, u8p, vp, vp, i64,
                                                   i32, i32, i32, i32, u8p, u8p]
        L.nvfp4_ref_soar_blocks_search.restype = i32
        L.nvfp4_ref_quantize_search.argtypes = [vp, i32, i64, i64, i32, i32, i32, i32, i32, i32, u8p, u8p, vp, vp]
        L.nvfp4_ref_quantize_search.restype = i32
        L.nvfp4_ref_grid_multiplier.argtypes = [i32, i32, i32]
        L.nvfp4_ref_grid_multiplier.restype = ctypes.c_float
        L.nvfp4_ref_mse.argtypes = [vp, i32, i64, i64, u8p, u8p, ctypes.c_float]
        L.nvfp4_ref_mse.restype = ctypes.c_double
        L.nvfp4_ref_dequantize.argtypes = [u8p, u8p, ctypes.c_float, i64, i64, vp]
        L.nvfp4_ref_dequantize.restype = None
        L.nvfp4_ref_e2m1_code.argtypes = [ctypes.c_float]
        L.nvfp4_ref_e2m1_code.restype = ctypes.c_uint
        L.nvfp4_ref_e2m1_value.argtypes = [ctypes.c_uint]
        L.nvfp4_ref_e2m1_value.restype = ctypes.c_float
        L.nvfp4_ref_e4m3_value.argtypes = [ctypes.c_uint]
        L.nvfp4_ref_e4m3_value.restype = ctypes.c_double
        L.nvfp4_ref_e4m3_rne.argtypes = [ctypes.c_double]
        L.nvfp4_ref_e4m3_rne.restype = ctypes.c_uint
        L.nvfp4_ref_e4m3_bracket.argtypes = [ctypes.c_double, ctypes.POINTER(ctypes.c_uint),
                                             ctypes.POINTER(ctypes.c_uint)]
        L.nvfp4_ref_e4m3_bracket.restype = None
        L.nvfp4_ref_e2m1_codes.argtypes = [vp, i64, u8p]
        L.nvfp4_ref_e2m1_codes.restype = None
        L.nvfp4_ref_e4m3_rne_many.argtypes = [vp, i64, u8p]
        L.nvfp4_ref_e4m3_rne_many.restype = None
        L.nvfp4_ref_search_multiplier.argtypes = [ctypes.c_int]
        L.nvfp4_ref_search_multiplier.restype = ctypes.c_float
        L.nvfp4_ref_quantize_block.argtypes = [vp, ctypes.c_float, ctypes.c_float, u8p]
        L.nvfp4_ref_quantize_block.restype = None
        L.nvfp4_ref_block_err.argtypes = [vp, u8p, ctypes.c_float, ctypes.c_double]
        L.nvfp4_ref_block_err.restype = ctypes.c_double
        L.nvfp4_ref_alpha_step.argtypes = [vp, i64, u8p, u8p, ctypes.POINTER(ctypes.c_float),
                                           ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
        L.nvfp4_ref_alpha_step.restype = i32
        L.nvfp4_ref_delta_step.argtypes = [vp, u8p, ctypes.c_float, ctypes.POINTER(ctypes.c_double)]
        L.nvfp4_ref_delta_step.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(W: np.ndarray) -> int:
    if W.dtype == np.uint16:
        return 0
    if W.dtype == np.float32:
        return 1
    raise TypeError("W must be uint16 (bf16 bits) or float32")


INITS = {"max": 0, "4o6": 1}
DD_RULES = {"cjso": 0, "quant": 1, "lsq": 2}  # NVFP4_REF_DD_*
PAGES_GRID = (50, 100, 101)  # f_k = (50 + k) / 100, k = 0..100


def quantize(W: np.ndarray, mode: str, iters: int = 0, *, trace: bool = False, init: str = "max"):
    """Run the oracle on a whole matrix. Returns a dict with codes, scales, alpha, status and, by
    mode, mchoice (4o6), dstar (cjso/soar) and alpha_trace (when asked). `init` is CJSO's starting
    point ("max" or "4o6"; cjso/soar only)."""
    W = np.ascontiguousarray(W)
    rows, cols = W.shape
    nblk = rows * cols // 16
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    mch = np.zeros((rows, cols // 16), np.uint8)
    dstar = np.zeros((rows, cols // 16), np.float64)
    alpha = ctypes.c_float(0.0)
    tr = np.zeros(iters + 1, np.float32)
    st = lib().nvfp4_ref_quantize_ex(_ptr(W), _dtype_code(W), rows, cols, MODES[mode], iters, INITS[init],
                                     _ptr(codes), _ptr(scales), ctypes.byref(alpha), _ptr(mch), _ptr(dstar),
                                     _ptr(tr) if trace else None)
    if st < 0:
        raise ValueError(f"oracle rejected the arguments (status {st})")
    out = {"codes": codes, "scales": scales, "alpha": alpha.value, "status": st}
    if mode == "4o6":
        out["mchoice"] = mch
    if mode in ("cjso", "soar"):
        out["dstar"] = dstar
    if trace:
        out["alpha_trace"] = tr
    assert nblk == scales.size
    return out


def quantize_search(W: np.ndarray, iters: int, *, grid=PAGES_GRID, dd_rule: str = "cjso", init: str = "max"):
    """SOAR with a configurable search: grid = (num0, den, count) gives f_k = nearest binary32 of
    (num0 + k) / den for k < count; dd_rule picks each candidate's reconstruct pair ("cjso": around the
    unrounded CJSO scale, the pages' rule; "quant": around Delta_q; "lsq": around the least-squares
    scale of the candidate's codes). Returns a dict with codes, scales, alpha, status and dstar."""
    W = np.ascontiguousarray(W)
    rows, cols = W.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    dstar = np.zeros((rows, cols // 16), np.float64)
    alpha = ctypes.c_float(0.0)
    num0, den, count = grid
    st = lib().nvfp4_ref_quantize_search(_ptr(W), _dtype_code(W), rows, cols, iters, INITS[init], num0, den, count,
                                         DD_RULES[dd_rule], _ptr(codes), _ptr(scales), ctypes.byref(alpha),
                                         _ptr(dstar))
    if st < 0:
        raise ValueError(f"oracle rejected the arguments (status {st})")
    return {"codes": codes, "scales": scales, "alpha": alpha.value, "status": st, "dstar": dstar}


def grid_multiplier(num0: int, den: int, k: int) -> float:
    return lib().nvfp4_ref_grid_multiplier(num0, den, k)


def soar_blocks(W: np.ndarray, alpha: float, dcode: np.ndarray, dstar: np.ndarray, blocks: np.ndarray, *,
                grid=PAGES_GRID, dd_rule: str = "cjso"):
    """Decoupled search on the listed blocks, given the CJSO state (and optionally a search of
    quantize_search). Returns (codes[nsel, 8], scales[nsel])."""
    W = np.ascontiguousarray(W)
    rows, cols = W.shape
    dcode = np.ascontiguousarray(dcode, np.uint8).reshape(-1)
    dstar = np.ascontiguousarray(dstar, np.float64).reshape(-1)
    blocks = np.ascontiguousarray(blocks, np.int64)
    codes = np.zeros((blocks.size, 8), np.uint8)
    scales = np.zeros(blocks.size, np.uint8)
    st = lib().nvfp4_ref_soar_blocks_search(_ptr(W), _dtype_code(W), rows, cols, alpha, _ptr(dcode), _ptr(dstar),
                                            _ptr(blocks), blocks.size, *grid, DD_RULES[dd_rule], _ptr(codes),
                                            _ptr(scales))
    if st < 0:
        raise ValueError("oracle rejected the arguments")
    return codes, scales


def matmul(X: np.ndarray, codes: np.ndarray, scales: np.ndarray, alpha: float, N: int) -> np.ndarray:
    """Y = X @ What.T for an NVFP4 [N][K] weight matrix (codes [N][K/2], scales [N][K/16], alpha):
    exact products summed in binary128, returned as float64 [M][N]."""
    X = np.ascontiguousarray(X)
    M, K = X.shape
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    if K % 16 != 0 or codes.size != N * K // 2 or scales.size != N * K // 16:
        raise ValueError("codes and scales do not describe an [N][K] NVFP4 matrix")
    Y = np.zeros((M, N), np.float64)
    st = lib().nvfp4_ref_matmul(_ptr(X), _dtype_code(X), M, K, _ptr(codes), _ptr(scales), alpha, N, _ptr(Y))
    if st < 0:
        raise ValueError("oracle rejected the arguments")
    return Y


def mse(W: np.ndarray, codes: np.ndarray, scales: np.ndarray, alpha: float) -> float:
    W = np.ascontiguousarray(W)
    rows, cols = W.shape
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    return lib().nvfp4_ref_mse(_ptr(W), _dtype_code(W), rows, cols, _ptr(codes), _ptr(scales), alpha)


def dequantize(codes: np.ndarray, scales: np.ndarray, alpha: float, rows: int, cols: int) -> np.ndarray:
    out = np.zeros((rows, cols), np.float64)
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    lib().nvfp4_ref_dequantize(_ptr(codes), _ptr(scales), alpha, rows, cols, _ptr(out))
    return out


def e2m1_code(x: float) -> int:
    return lib().nvfp4_ref_e2m1_code(x)


def e2m1_value(code: int) -> float:
    return lib().nvfp4_ref_e2m1_value(code)


def e2m1_codes(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32).reshape(-1)
    out = np.zeros(x.size, np.uint8)
    lib().nvfp4_ref_e2m1_codes(_ptr(x), x.size, _ptr(out))
    return out


def e4m3_rne_many(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float64).reshape(-1)
    out = np.zeros(v.size, np.uint8)
    lib().nvfp4_ref_e4m3_rne_many(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_value(code: int) -> float:
    return lib().nvfp4_ref_e4m3_value(code)


def e4m3_rne(v: float) -> int:
    return lib().nvfp4_ref_e4m3_rne(v)


def e4m3_bracket(v: float):
    lo, hi = ctypes.c_uint(0), ctypes.c_uint(0)
    lib().nvfp4_ref_e4m3_bracket(v, ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


def search_multiplier(k: int) -> float:
    return lib().nvfp4_ref_search_multiplier(k)


def quantize_block(w16: np.ndarray, alpha: float, delta: float) -> np.ndarray:
    w16 = np.ascontiguousarray(w16, np.float32)
    out = np.zeros(16, np.uint8)
    lib().nvfp4_ref_quantize_block(_ptr(w16), alpha, delta, _ptr(out))
    return out


def block_err(w16: np.ndarray, codes16: np.ndarray, alpha: float, delta_d: float) -> float:
    w16 = np.ascontiguousarray(w16, np.float32)
    codes16 = np.ascontiguousarray(codes16, np.uint8)
    return lib().nvfp4_ref_block_err(_ptr(w16), _ptr(codes16), alpha, delta_d)


def alpha_step(w: np.ndarray, dcode: np.ndarray, codes16: np.ndarray):
    """Returns (ok, alpha, num, den) of one global-scale step on blocks of 16 floats."""
    w = np.ascontiguousarray(w, np.float32).reshape(-1)
    dcode = np.ascontiguousarray(dcode, np.uint8).reshape(-1)
    codes16 = np.ascontiguousarray(codes16, np.uint8).reshape(-1)
    a, n, d = ctypes.c_float(0.0), ctypes.c_double(0.0), ctypes.c_double(0.0)
    ok = lib().nvfp4_ref_alpha_step(_ptr(w), w.size // 16, _ptr(dcode), _ptr(codes16), ctypes.byref(a),
                                    ctypes.byref(n), ctypes.byref(d))
    return bool(ok), a.value, n.value, d.value


def delta_step(w16: np.ndarray, codes16: np.ndarray, alpha: float):
    w16 = np.ascontiguousarray(w16, np.float32)
    codes16 = np.ascontiguousarray(codes16, np.uint8)
    d = ctypes.c_double(0.0)
    ok = lib().nvfp4_ref_delta_step(_ptr(w16), _ptr(codes16), alpha, ctypes.byref(d))
    return bool(ok), d.value


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """[rows, cols//2] packed bytes -> [rows, cols] codes (0..15)."""
    lo = codes & 15
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)
