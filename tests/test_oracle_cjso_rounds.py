"""Pin of the oracle's whole CJSO iteration, not just its two steps (CPU only).

The SOAR page's CJSO paragraph fixes how the rounds are composed: start from the max rule, then
alternate the global-scale (alpha) step and the block-scale (Delta) step, and quantise to FP4 again after
every update. Its two closed forms (the alpha* and Delta_i* equations; alpha* printed with alpha where
Delta_i belongs, the least-squares minimiser is used) give each step. The stored block scale is FP8, so a
Delta-step ends with the E4M3 rounding of Delta_i*.

This file writes those rounds out a second time with nothing from the oracle: exact integer and rational
arithmetic for every sum, quotient and squared error, and the brute-force E2M1 / E4M3 codecs of
tests/indep.py. It compares alpha after every round, the scales, the codes and the last unrounded scales
bit for bit. Two planted mistakes (no re-quantisation after the alpha-step; Delta-step before the
alpha-step) are compiled from the oracle's own source on the CPU and must each be caught.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import indep

E4M3_POS = indep.E4M3_POS  # the 127 non-negative finite values, increasing with the code
E4M3_INT = np.rint(E4M3_POS * 512).astype(np.int64)  # every value is a multiple of 2^-9
assert np.array_equal(E4M3_INT.astype(np.float64) / 512, E4M3_POS)
MIDPOINTS = (E4M3_POS[:-1] + E4M3_POS[1:]) / 2  # exact in binary64


# ------------------------------------------------------------------------------- exact primitives

def exact_ints(w32: np.ndarray) -> np.ndarray:
    """Each binary32 value as the integer w * 2^149 (binary32 values are multiples of 2^-149)."""
    scaled = np.asarray(w32, np.float32).astype(np.float64) * 2.0 ** 149  # exact: a power-of-two scale
    return np.array([int(v) for v in scaled.ravel()], dtype=object).reshape(scaled.shape)


def e4m3_nearest(v: list) -> np.ndarray:
    """E4M3 code nearest each non-negative rational (ties to the even code, 448 for anything above).
    The binary64 image decides unless it lands on a midpoint of two E4M3 values; then the exact
    rational decides."""
    d = np.array([float(x) for x in v], np.float64)
    out = indep.brute_e4m3(d)
    for i in np.nonzero(np.isin(d, MIDPOINTS))[0]:
        lo = int(np.searchsorted(MIDPOINTS, d[i]))
        mid = Fraction(float(MIDPOINTS[lo]))
        if v[i] < mid:
            out[i] = lo
        elif v[i] > mid:
            out[i] = lo + 1
        else:
            out[i] = lo if lo % 2 == 0 else lo + 1
    return out


def quantize_all(w: np.ndarray, alpha: np.float32, dcode: np.ndarray) -> np.ndarray:
    """Codes of every block under (alpha, Delta_i): s = fl(alpha*Delta), r = fl(1/s), x = fl(w*r) in
    binary32, then the nearest E2M1 value (a zero s gives code 0)."""
    s = (np.float32(alpha) * E4M3_POS[dcode].astype(np.float32)).astype(np.float32)
    with np.errstate(divide="ignore"):
        r = (np.float32(1.0) / s).astype(np.float32)
    x = (w * r[:, None]).astype(np.float32)
    codes = indep.brute_e2m1(np.where(s[:, None] == 0, np.float32(0), x)).reshape(w.shape)
    return codes


def q_twice(codes: np.ndarray) -> np.ndarray:
    """2|q| as integers (E2M1 magnitudes are multiples of 1/2)."""
    return np.rint(np.abs(indep.e2m1_decode(codes)) * 2).astype(np.int64)


def block_sums(Wi: np.ndarray, codes: np.ndarray):
    """Exact per-block sums: sum_j w_j q_j as an integer times 2^-150, sum_j q_j^2 as an integer times
    1/4. A code's sign always equals its element's, so w_j q_j = |w_j| |q_j|."""
    q2 = q_twice(codes)
    swq = (np.abs(Wi) * q2).sum(axis=1)
    sqq = (q2 * q2).sum(axis=1)
    return swq, sqq


def exact_errors(Wi: np.ndarray, codes: np.ndarray, alpha: np.float32, dcode: np.ndarray) -> np.ndarray:
    """Per-block squared error sum_j (w_j - q_j alpha Delta_j)^2 as an integer times 2^-318: w is a
    multiple of 2^-149 and q alpha Delta of 2^-1 * 2^-149 * 2^-9."""
    a = int(float(alpha) * 2.0 ** 149)
    qs = np.rint(indep.e2m1_decode(codes) * 2).astype(np.int64).astype(object)  # signed 2q
    rec = qs * (E4M3_INT[dcode].astype(object)[:, None] * a)  # q alpha Delta * 2^159
    diff = Wi * (1 << 10) - rec
    return (diff * diff).sum(axis=1)


def nearest_f32(fr: Fraction) -> np.float32:
    return indep.nearest_f32(fr)


# ------------------------------------------------------------------------------------ CJSO written out

def cjso_rounds(w32: np.ndarray, iters: int, init: str = "max"):
    """CJSO as the SOAR page composes it. w32: [blocks, 16] binary32. Returns alpha after each round
    (index 0 = the starting alpha), the E4M3 scale codes, the codes and the last unrounded scales."""
    w = np.asarray(w32, np.float32)
    Wi = exact_ints(w)
    nblk = w.shape[0]
    # max rule: alpha = fl(max|W| / (6*448)), Delta_i = E4M3(max|W_i| / (6 alpha)) of the real quotient
    A = Fraction(float(np.abs(w).max()))
    alpha = nearest_f32(A / 2688)
    amax = np.abs(w).max(axis=1)
    if alpha == 0:
        quot = [Fraction(0)] * nblk
    else:
        quot = [Fraction(float(a)) / (6 * Fraction(float(alpha))) for a in amax]
    dcode = e4m3_nearest(quot)
    dstar = np.array([float(x) for x in quot])
    codes = quantize_all(w, alpha, dcode)
    if init == "4o6":
        # FourOverSix: Delta4 = E4M3(1.5 Delta6); M=4 iff its block error is strictly smaller
        d4 = e4m3_nearest([Fraction(3, 2) * Fraction(float(E4M3_POS[c])) for c in dcode])
        c4 = quantize_all(w, alpha, d4)
        m4 = exact_errors(Wi, c4, alpha, d4) < exact_errors(Wi, codes, alpha, dcode)
        m4 = np.array(m4, bool)
        dstar = np.where(m4, 1.5 * E4M3_POS[dcode], dstar)
        dcode = np.where(m4, d4, dcode).astype(np.uint8)
        codes = np.where(m4[:, None], c4, codes)
    trace = [alpha]
    for _ in range(iters):
        # alpha-step: alpha* = sum_i Delta_i sum_j W_ij Q_ij / sum_i Delta_i^2 sum_j Q_ij^2, exactly
        swq, sqq = block_sums(Wi, codes)
        dint = E4M3_INT[dcode]
        num = int((dint * swq).sum())  # * 2^-159
        den = int((dint * dint * sqq).sum())  # * 2^-20
        if den > 0:
            alpha = nearest_f32(Fraction(num, den) / 2 ** 139)
        codes = quantize_all(w, alpha, dcode)  # re-quantise after the alpha update
        # Delta-step: Delta_i* = sum_j W_ij Q_ij / (alpha sum_j Q_ij^2), then its E4M3 rounding
        swq, sqq = block_sums(Wi, codes)
        a = Fraction(float(alpha))
        upd = [Fraction(int(n), 2 ** 150) / (a * Fraction(int(d), 4)) if d > 0 else None for n, d in zip(swq, sqq)]
        new = e4m3_nearest([u for u in upd if u is not None])
        it = iter(range(len(new)))
        for i, u in enumerate(upd):
            if u is None:  # no nonzero code: the block keeps its scale
                dstar[i] = E4M3_POS[dcode[i]]
            else:
                k = next(it)
                dstar[i] = float(u)
                dcode[i] = new[k]
        codes = quantize_all(w, alpha, dcode)  # re-quantise after the Delta update
        trace.append(alpha)
    return np.array(trace, np.float32), dcode.astype(np.uint8), codes.astype(np.uint8), dstar


def pack(codes16: np.ndarray) -> np.ndarray:
    c = codes16.reshape(-1, 2)
    return (c[:, 0] | (c[:, 1] << 4)).astype(np.uint8)


def c2_slice() -> np.ndarray:
    return np.ascontiguousarray(synth.c2(0)[:256, :1024])


INPUTS = {
    "c1": lambda: synth.c1(0),
    "c2_slice": c2_slice,
    "c3_rows": lambda: synth.normal_bf16(64, 512, seed=31, std=0.015),
}
_cache: dict = {}


def _input(name):
    if name not in _cache:
        _cache[name] = INPUTS[name]()
    return _cache[name]


def _check(W, r, iters, init="max"):
    w = indep.as_f32(W).reshape(-1, 16)
    trace, dcode, codes, dstar = cjso_rounds(w, iters, init)
    assert np.array_equal(np.asarray(r["alpha_trace"], np.float32).view(np.uint32), trace.view(np.uint32))
    assert np.array_equal(r["scales"].reshape(-1), dcode)
    assert np.array_equal(r["codes"].reshape(-1), pack(codes))
    assert np.array_equal(r["dstar"].reshape(-1), dstar)


@pytest.mark.parametrize("name", list(INPUTS))
@pytest.mark.parametrize("iters", [1, 2, 3])
def test_cjso_rounds_equal_the_pages_composition(name, iters):
    W = _input(name)
    r = oracle.quantize(W, "cjso", iters, trace=True)
    _check(W, r, iters)


@pytest.mark.parametrize("iters", [0, 2])
def test_cjso_from_4o6_rounds(iters):
    W = _input("c2_slice")[:64]
    r = oracle.quantize(W, "cjso", iters, trace=True, init="4o6")
    _check(W, r, iters, init="4o6")


def test_alpha_moves_and_scales_move():
    """The rounds must do something on these inputs, or the pins above would be vacuous."""
    W = _input("c2_slice")
    w = indep.as_f32(W).reshape(-1, 16)
    t3, d3, c3, _ = cjso_rounds(w, 3)
    _, d0, _, _ = cjso_rounds(w, 0)
    assert len(set(t3.tolist())) == 4
    assert np.mean(d3 != d0) > 0.05


# ------------------------------------------------------------------------------------- planted mistakes

SRC = os.path.join(os.path.dirname(oracle.__file__), "nvfp4_oracle.c")
REQUANT = ("for (i = 0; i < nblk; ++i)\n"
           "            nvfp4_ref_quantize_block(w + 16 * i, *alpha, (float)nvfp4_ref_e4m3_value(dcode[i]), "
           "codes16 + 16 * i);\n")
ALPHA_STEP = "nvfp4_ref_alpha_step(w, nblk, dcode, codes16, alpha, NULL, NULL);\n"


def _round_body(src: str):
    """The text of one CJSO round in the oracle: from its alpha-step to the trace update."""
    m = re.search(r"for \(t = 1; t <= iters; \+\+t\) \{\n(.*?)\n        if \(alpha_trace\) alpha_trace\[t\]", src, re.S)
    assert m, "the oracle's CJSO round loop has changed shape; update the planted mistakes"
    return m.group(1)


def _mutant_no_requant_after_alpha(src: str) -> str:
    body = _round_body(src)
    i = body.index(ALPHA_STEP) + len(ALPHA_STEP)
    rest = body[i:].lstrip()
    assert rest.startswith(REQUANT), "expected the re-quantisation right after the alpha-step"
    new = body[:i] + "        " + rest[len(REQUANT):]
    return src.replace(body, new)


def _mutant_delta_first(src: str) -> str:
    body = _round_body(src)
    i = body.index(ALPHA_STEP)
    j = body.index(REQUANT, i) + len(REQUANT)  # the alpha-step and its re-quantisation
    alpha_part = body[i:j]
    rest = body[j:]
    new = body[:i] + rest.lstrip() + "\n        " + alpha_part.rstrip()
    return src.replace(body, new)


def _run_lib(path, W, iters):
    L = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.nvfp4_ref_quantize_ex.argtypes = [vp, i32, i64, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    L.nvfp4_ref_quantize_ex.restype = i32
    rows, cols = W.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    dstar = np.zeros(rows * cols // 16, np.float64)
    tr = np.zeros(iters + 1, np.float32)
    a = ctypes.c_float(0)
    p = lambda x: x.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    st = L.nvfp4_ref_quantize_ex(p(W), 0 if W.dtype == np.uint16 else 1, rows, cols, 2, iters, 0, p(codes),
                                 p(scales), ctypes.byref(a), None, p(dstar), p(tr))
    assert st == 0
    return {"codes": codes, "scales": scales, "alpha": a.value, "dstar": dstar, "alpha_trace": tr}


@pytest.mark.parametrize("mutate", [_mutant_no_requant_after_alpha, _mutant_delta_first])
def test_planted_round_mistakes_are_caught(mutate):
    src = open(SRC).read()
    bad = mutate(src)
    assert bad != src
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "mutant.c")
        so = os.path.join(d, "libmutant.so")
        with open(c, "w") as f:
            f.write(bad)
        subprocess.run(["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-ffp-contract=off", "-I",
                        os.path.dirname(SRC), "-o", so, c, "-lm"], check=True)
        W = _input("c2_slice")
        r = _run_lib(so, W, 2)
    with pytest.raises(AssertionError):
        _check(W, r, 2)
