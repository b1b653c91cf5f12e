"""Pins for the exact-tie case of the decoupled search (SOAR page, decoupled quantise/dequantise scales:
keep the best of all candidates, the CJSO point first, replaced only by a strictly smaller error).

synth.soar_tie_matrix holds fp32 blocks built so that the least error over the quantise grid is the same
number for both reconstruct scales of the pair, and smaller than the incumbent's. Scan order then
decides: the first candidate reaching it is kept. These tests show, with exact rational arithmetic and
the brute-force codecs of tests/indep (not the oracle's routines), that every constructed block really is
such a tie, and that the oracle resolves it as the scan order does."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import indep
from tests.test_oracle_search import E4M3, bracket, brute_search, exact_err

ALPHA = synth.SOAR_TIE_ALPHA


def nearest_codes(w16, scale: Fraction):
    """Nearest E2M1 magnitude of each exact quotient |w| / scale (no binary32 rounding anywhere)."""
    grid = [Fraction(float(g)) for g in indep.GRID]
    out = []
    for w in w16:
        u = abs(Fraction(float(w))) / scale
        d = [abs(u - g) for g in grid]
        out.append(min(range(8), key=lambda i: (d[i], i % 2)))  # ties to the even code
    return np.array(out)


def per_k_errors(w16, dc, d):
    dcv = np.float32(float(E4M3[dc]))
    errs, codes = [], []
    for k in range(101):
        f = indep.nearest_f32(Fraction(50 + k, 100))
        cand = indep.quantize_block_np(w16, ALPHA, np.float32(dcv * f))
        codes.append(cand)
        errs.append(exact_err(w16, cand, ALPHA, E4M3[d]))
    return errs, codes


@pytest.mark.parametrize("kind", ["A", "B"])
def test_constructed_block_is_an_exact_tie(kind):
    w16 = (np.array(synth.SOAR_TIE_BLOCKS[kind], np.float64) * ALPHA).astype(np.float32)
    amax = Fraction(float(np.abs(w16).max()))
    dstar = amax / (6 * Fraction(ALPHA))
    dc = int(indep.brute_e4m3(np.array([float(dstar)]))[0])
    lo, hi = bracket(dstar)
    assert lo != hi and dc in (lo, hi)
    dcv = np.float32(float(E4M3[dc]))
    inc = indep.quantize_block_np(w16, ALPHA, dcv)
    e_inc = exact_err(w16, inc, ALPHA, E4M3[dc])
    # the incumbent's binary32 scaling rounds one element to the far side of a midpoint
    near = nearest_codes(w16, Fraction(ALPHA) * E4M3[dc])
    assert np.sum((inc & 7) != near) == 1
    e_lo, _ = per_k_errors(w16, dc, lo)
    e_hi, _ = per_k_errors(w16, dc, hi)
    assert min(e_lo) == min(e_hi) < e_inc
    k_lo = e_lo.index(min(e_lo))
    k_hi = e_hi.index(min(e_hi))
    assert k_lo <= k_hi  # so the lower reconstruct scale is reached first


def test_oracle_resolves_ties_in_scan_order():
    W, kinds = synth.soar_tie_matrix()
    r = oracle.quantize(W, "soar", 0)
    assert np.float32(r["alpha"]) == np.float32(ALPHA)
    blocks = W.reshape(-1, 16)
    codes = indep.unpack(r["codes"]).reshape(-1, 16)
    scales = r["scales"].reshape(-1)
    seen = {"A": 0, "B": 0}
    for b, kind in enumerate(kinds):
        if not kind:
            continue
        w16 = blocks[b]
        dstar = Fraction(float(np.abs(w16).max())) / (6 * Fraction(ALPHA))
        dc = int(indep.brute_e4m3(np.array([float(dstar)]))[0])
        want_codes, want_scale = brute_search(w16, ALPHA, dc, float(dstar), (50, 100, 101), "cjso")
        assert want_scale == bracket(dstar)[0]
        assert int(scales[b]) == want_scale
        assert np.array_equal(codes[b], want_codes)
        seen[kind] += 1
    assert seen["A"] > 20 and seen["B"] > 20
