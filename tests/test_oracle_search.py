"""Pins of the oracle's configurable decoupled search (SOAR page, decoupled quantise/dequantise scales):
the multiplier grid f_k = binary32 nearest (num0 + k)/den and the three reconstruct-pair rules (the
pages' bracket of the unrounded CJSO scale, the bracket of Delta_q, the bracket of the candidate's own
least-squares scale). Checks use tests/indep (brute-force codecs) and exact rational arithmetic, not
the oracle's own routines."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import indep

E4M3 = [Fraction(float(v)) for v in indep.e4m3_decode(np.arange(127))]  # codes 0..126, increasing


def bracket(v: Fraction):
    """E4M3 codes (lo, hi) around v >= 0: lo the largest value <= v, hi the smallest >= v (448 caps both)."""
    lo = max(c for c in range(127) if E4M3[c] <= v)
    if E4M3[lo] == v or lo == 126:
        return lo, lo
    return lo, lo + 1


def exact_err(w16, codes16, alpha, delta_d: Fraction) -> Fraction:
    q = indep.e2m1_decode(np.asarray(codes16))
    a = Fraction(float(alpha))
    return sum((Fraction(float(w)) - Fraction(float(qq)) * a * delta_d) ** 2 for w, qq in zip(w16, q))


def brute_search(w16, alpha, dc, dstar, grid, rule):
    """The search written out from the page's description with independent primitives."""
    num0, den, count = grid
    dcv = np.float32(float(E4M3[dc]))
    best_codes = indep.quantize_block_np(w16, alpha, dcv)
    best = exact_err(w16, best_codes, alpha, E4M3[dc])
    best_scale = dc
    pair = bracket(Fraction(float(dstar)))
    for k in range(count):
        f = indep.nearest_f32(Fraction(num0 + k, den))
        dq = np.float32(dcv * f)
        cand = indep.quantize_block_np(w16, alpha, dq)
        if rule == "quant":
            pair = bracket(Fraction(float(dq)))
        elif rule == "lsq":
            q = indep.e2m1_decode(cand)
            swq = sum(Fraction(float(w)) * Fraction(float(x)) for w, x in zip(w16, q))
            sqq = sum(Fraction(float(x)) ** 2 for x in q)
            if sqq > 0:
                ls = float(swq) / (float(np.float32(alpha)) * float(sqq))  # binary64 quotient
                pair = bracket(Fraction(ls))
            else:
                pair = (dc, dc)
        for d in pair:
            e = exact_err(w16, cand, alpha, E4M3[d])
            if e < best:
                best, best_codes, best_scale = e, cand, d
    return best_codes, best_scale


def cjso_state(rows, cols, seed, iters=2):
    W = synth.normal_bf16(rows, cols, seed)
    r = oracle.quantize(W, "cjso", iters)
    return W, r


@pytest.mark.parametrize("num0,den", [(50, 100), (1, 3), (7, 24), (1 << 24, 1 << 24), (12345, 16777213)])
def test_grid_multiplier_is_nearest_binary32(num0, den):
    for k in (0, 1, 2, 17, 100, 1023):
        if num0 + k > 16 * den:
            continue
        got = np.float32(oracle.grid_multiplier(num0, den, k))
        assert got == indep.nearest_f32(Fraction(num0 + k, den)), (num0, den, k)


def test_pages_grid_and_rule_reproduce_soar():
    W = synth.normal_bf16(16, 128, 3)
    a = oracle.quantize(W, "soar", 3)
    b = oracle.quantize_search(W, 3, grid=oracle.PAGES_GRID, dd_rule="cjso")
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])
    assert a["alpha"] == b["alpha"]


@pytest.mark.parametrize("grid,rule", [((1, 4, 7), "cjso"), ((45, 100, 13), "quant"), ((1, 4, 7), "lsq"),
                                       ((90, 100, 21), "lsq"), ((50, 100, 101), "quant")])
def test_search_matches_brute_force(grid, rule):
    W, r = cjso_state(4, 64, seed=11)
    w = indep.as_f32(W).reshape(-1, 16)
    dcode, dstar = r["scales"].reshape(-1), r["dstar"].reshape(-1)
    blocks = np.arange(w.shape[0])
    codes, scales = oracle.soar_blocks(W, r["alpha"], dcode, dstar, blocks, grid=grid, dd_rule=rule)
    for b in blocks:
        bc, bs = brute_search(w[b], r["alpha"], int(dcode[b]), dstar[b], grid, rule)
        assert int(scales[b]) == bs, (b, grid, rule)
        assert np.array_equal(indep.unpack(codes[b:b + 1])[0] & 7, bc & 7), (b, grid, rule)


def test_lsq_rule_on_the_cjso_codes_reaches_the_best_e4m3_scale():
    """With the single multiplier 1 the candidate keeps the CJSO codes; a quadratic's minimum over the E4M3
    values lies next to its real minimiser, so the rule must reach the least error over all 127 scales."""
    W, r = cjso_state(4, 64, seed=5)
    out = oracle.quantize_search(W, 2, grid=(1, 1, 1), dd_rule="lsq")
    w = indep.as_f32(W).reshape(-1, 16)
    cj_codes = indep.unpack(r["codes"].reshape(-1, 8))
    got_codes = indep.unpack(out["codes"].reshape(-1, 8))
    for b in range(w.shape[0]):
        assert np.array_equal(got_codes[b] & 7, cj_codes[b] & 7) or not np.any(cj_codes[b] & 7)
        best = min(exact_err(w[b], cj_codes[b], r["alpha"], v) for v in E4M3)
        got = exact_err(w[b], got_codes[b], out["alpha"], E4M3[int(out["scales"].reshape(-1)[b])])
        assert got == best, b


def test_quant_rule_with_multiplier_one_keeps_cjso():
    """Delta_q = Delta_c is an E4M3 value, so its bracket is {Delta_c}: nothing can beat the incumbent."""
    W, r = cjso_state(8, 64, seed=9)
    out = oracle.quantize_search(W, 2, grid=(1, 1, 1), dd_rule="quant")
    assert np.array_equal(out["codes"], r["codes"]) and np.array_equal(out["scales"], r["scales"])


def test_finer_grid_is_never_worse():
    """(100 + 2k)/200 holds every (50 + k)/100 with the same nearest binary32, and both searches start from
    the same CJSO point, so the finer grid's error is at most the pages' grid's, block by block."""
    W = synth.normal_bf16(4, 64, 21)
    a = oracle.quantize_search(W, 2, grid=(50, 100, 101))
    b = oracle.quantize_search(W, 2, grid=(100, 200, 201))
    ea = indep.block_errors(W, a["codes"], a["scales"], a["alpha"])
    eb = indep.block_errors(W, b["codes"], b["scales"], b["alpha"])
    w = indep.as_f32(W).reshape(-1, 16)
    ca, cb = indep.unpack(a["codes"].reshape(-1, 8)), indep.unpack(b["codes"].reshape(-1, 8))
    sa, sb = a["scales"].reshape(-1), b["scales"].reshape(-1)
    for i in np.nonzero(eb > ea * (1 - 1e-12))[0]:  # confirm the near-equal cases exactly
        assert exact_err(w[i], cb[i], b["alpha"], E4M3[int(sb[i])]) <= exact_err(w[i], ca[i], a["alpha"],
                                                                                  E4M3[int(sa[i])])


@pytest.mark.parametrize("grid,rule", [((0, 100, 101), "cjso"), ((50, 0, 101), "cjso"), ((50, 100, 0), "cjso"),
                                       ((50, 100, 1025), "cjso"), ((1, 1, 17), "cjso"),
                                       ((50, (1 << 24) + 1, 10), "cjso")])
def test_search_rejects_bad_grids(grid, rule):
    W = synth.normal_bf16(2, 32, 1)
    with pytest.raises(ValueError):
        oracle.quantize_search(W, 1, grid=grid, dd_rule=rule)


def test_search_rejects_unknown_rule():
    W = synth.normal_bf16(2, 32, 1)
    with pytest.raises(KeyError):
        oracle.quantize_search(W, 1, dd_rule="nearest")
