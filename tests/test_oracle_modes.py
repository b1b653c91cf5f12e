"""Pins of the oracle's four modes (CPU only).

MAX: exact round trip of matrices built on the NVFP4 grid, and scale monotonicity.
FourOverSix: per-block error never above MAX's; constructed blocks that must pick M=4, M=6 or tie; the
M=4 scale table against torch's float8; the per-block choice against an independent re-scoring.
CJSO: the alpha and block-scale steps land on the minimisers of the quadratic found by dense scans (the
page's literal alpha* does not); each alpha-step never raises the objective; zero iterations equal MAX;
on-grid input is a fixed point.
SOAR: error never above CJSO's per block; the winner equals an independent re-scoring of all 202
candidates; on-grid input is a fixed point.
Edge cases: non-finite input, all-zero input, zero blocks, tiny magnitudes, bad arguments.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import indep


# ---------------------------------------------------------------------------------------------- MAX

@pytest.mark.parametrize("dtype,alpha_exp", [(np.uint16, -12), (np.float32, -3), (np.uint16, 0)])
def test_max_round_trip_on_grid(dtype, alpha_exp):
    W, alpha0, dcode, q = indep.on_grid_matrix(8, 256, alpha_exp, seed=3, dtype=dtype)
    r = oracle.quantize(W, "max")
    assert r["status"] == 0
    assert r["alpha"] == alpha0
    assert np.array_equal(r["scales"], dcode)
    assert np.array_equal(indep.unpack(r["codes"]), q)
    assert oracle.mse(W, r["codes"], r["scales"], r["alpha"]) == 0.0
    assert r["scales"][0, 0] == 0x7E


def test_max_alpha_and_scale_monotone():
    W = synth.c1(0)
    r = oracle.quantize(W, "max")
    A = np.abs(W).max()
    assert r["alpha"] == np.float32(A) / np.float32(2688.0)
    c = indep.golden_constants()
    assert 2688.0 == c["M_FP4"] * c["M_FP8"]
    amax = np.abs(W.reshape(-1, 16)).max(axis=1)
    d = indep.e4m3_decode(r["scales"].reshape(-1))
    order = np.argsort(amax, kind="stable")
    assert np.all(np.diff(d[order]) >= 0)
    # every block's largest element maps near the top of the grid: |x| in (3.5, 6.x]
    q = indep.e2m1_decode(indep.unpack(r["codes"])).reshape(-1, 16)
    assert np.all(np.abs(q).max(axis=1) >= 4)


# --------------------------------------------------------------------------------------- FourOverSix

def test_4o6_m4_scale_table():
    for c6 in range(0x7F):
        d4 = oracle.e4m3_rne(1.5 * oracle.e4m3_value(c6))
        v = np.float32(1.5 * indep.E4M3_POS[c6])
        if v <= 464:
            assert d4 == indep.torch_e4m3(np.array([v]))[0], c6
        else:  # beyond torch's range: saturation (448)
            assert d4 == 0x7E


def test_4o6_never_worse_than_max_and_choice_matches_rescoring():
    W = synth.c1(0)
    rm = oracle.quantize(W, "max")
    r = oracle.quantize(W, "4o6")
    em = indep.block_errors(W, rm["codes"], rm["scales"], rm["alpha"])
    e = indep.block_errors(W, r["codes"], r["scales"], r["alpha"])
    assert r["alpha"] == rm["alpha"]
    assert np.all(e <= em * (1 + 1e-12))
    mch = r["mchoice"].reshape(-1)
    # where M=6 is kept the output equals MAX's
    keep = mch == 0
    assert np.array_equal(r["scales"].reshape(-1)[keep], rm["scales"].reshape(-1)[keep])
    # independent re-scoring of both candidates for every block
    w = W.reshape(-1, 16)
    d6 = indep.e4m3_decode(rm["scales"].reshape(-1))
    d4 = indep.e4m3_decode(indep.brute_e4m3(1.5 * d6))
    ambiguous = 0
    for b in range(w.shape[0]):
        c6 = indep.quantize_block_np(w[b], r["alpha"], d6[b])
        c4 = indep.quantize_block_np(w[b], r["alpha"], d4[b])
        e6 = indep.block_err_np(w[b], c6, r["alpha"], d6[b])
        e4 = indep.block_err_np(w[b], c4, r["alpha"], d4[b])
        if abs(e4 - e6) <= 1e-12 * max(e6, 1e-300):
            ambiguous += 1
            continue
        assert mch[b] == int(e4 < e6), b
    assert ambiguous < 5
    frac = mch.mean()
    assert 0.2 < frac < 0.7  # context: the write-up reports about 40-43 % on real weights


def _block_grid_values(qs, scale):
    return np.array(qs, np.float64) * scale


def test_4o6_constructed_choices():
    alpha0 = 2.0 ** -10
    rows = []
    # block 0: pins alpha (Delta = 448, contains 6*448*alpha0)
    b0 = np.zeros(16); b0[0] = 6 * 448 * alpha0; b0[1:4] = np.array([1, 2, 3]) * alpha0
    rows.append(b0)
    # block 1: exact on the M=4 grid of Delta4 = 3 (max |q| = 4, includes 1.5 and 3): Delta6 = 2, M=4 wins
    b1 = _block_grid_values([4, 3, 1.5, 1, 0.5, 2, 0, -4, -3, -1.5, 1, 0.5, 2, 3, 4, 0], 3 * alpha0)
    rows.append(b1)
    # block 2: exact on the M=6 grid with many 0.5 steps: M=6 has zero error, M=4 does not
    b2 = _block_grid_values([6, 0.5, 1, 1.5, 0.5, -0.5, 2, 3, 0.5, 1, 1.5, -6, 0.5, 1, 0, 0.5], 5 * alpha0)
    rows.append(b2)
    # block 3: Delta6 = 448 -> Delta4 saturates to 448: identical candidates, tie keeps M=6
    b3 = _block_grid_values([6, 5, 1, 2, 0, 3.3, 1, 1, 2, 2, 1, 0, 0, 0, 0, 1], 448 * alpha0)
    rows.append(b3)
    W = np.concatenate(rows).reshape(1, 64).astype(np.float32)
    r = oracle.quantize(W, "4o6")
    assert r["alpha"] == alpha0
    m = r["mchoice"].reshape(-1)
    s = r["scales"].reshape(-1)
    assert m[1] == 1 and indep.e4m3_decode([s[1]])[0] == 3.0
    assert indep.block_errors(W, r["codes"], r["scales"], r["alpha"])[1] == 0.0
    assert m[2] == 0 and indep.e4m3_decode([s[2]])[0] == 5.0
    assert m[3] == 0 and s[3] == 0x7E


# ---------------------------------------------------------------------------------------------- CJSO

def _tiny_problem(seed, nblk):
    g = np.random.default_rng(seed)
    w = (g.standard_t(4, size=(nblk, 16)) * 0.02).astype(np.float32)
    dcode = g.integers(40, 100, size=nblk).astype(np.uint8)
    alpha = np.float32(np.abs(w).max() / 2688.0)
    codes = np.stack([indep.quantize_block_np(w[b], alpha, indep.E4M3_POS[dcode[b]]) for b in range(nblk)])
    return w, dcode, codes, alpha


def _objective(w, dcode, codes, alpha, dscale=None):
    q = indep.e2m1_decode(codes)
    d = indep.E4M3_POS[dcode][:, None] if dscale is None else dscale[:, None]
    e = w.astype(np.float64) - alpha * d * q
    return float(np.sum(e * e))


@pytest.mark.parametrize("seed,nblk", [(0, 1), (1, 2), (2, 3), (3, 4), (4, 4)])
def test_cjso_alpha_step_is_the_least_squares_minimiser(seed, nblk):
    w, dcode, codes, alpha = _tiny_problem(seed, nblk)
    ok, a_star, num, den = oracle.alpha_step(w, dcode, codes)
    assert ok
    grid = a_star * (1 + np.linspace(-1e-3, 1e-3, 2001))
    L = np.array([_objective(w, dcode, codes, a) for a in grid])
    assert abs(int(np.argmin(L)) - 1000) <= 1
    # the page's printed fraction (alpha in place of Delta_i) is not the minimiser
    q = indep.e2m1_decode(codes)
    literal = np.sum(w * q * alpha) / np.sum(q * q * alpha * alpha)
    assert abs(literal / a_star - 1) > 1e-2
    # objective does not increase from the starting alpha
    assert _objective(w, dcode, codes, a_star) <= _objective(w, dcode, codes, alpha) * (1 + 1e-15)


@pytest.mark.parametrize("seed", range(6))
def test_cjso_delta_step_is_the_least_squares_minimiser(seed):
    w, dcode, codes, alpha = _tiny_problem(seed, 1)
    ok, dstar = oracle.delta_step(w[0], codes[0], alpha)
    assert ok
    grid = dstar * (1 + np.linspace(-1e-3, 1e-3, 2001))
    L = [_objective(w, dcode, codes, alpha, np.array([d])) for d in grid]
    assert abs(int(np.argmin(L)) - 1000) <= 1


def test_cjso_zero_iterations_equals_max():
    W = synth.normal_bf16(64, 256, seed=5)
    a = oracle.quantize(W, "max")
    b = oracle.quantize(W, "cjso", 0)
    assert a["alpha"] == b["alpha"]
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])


def test_cjso_trace_and_improvement():
    W = synth.c1(0)
    r = oracle.quantize(W, "cjso", 8, trace=True)
    rm = oracle.quantize(W, "max")
    assert r["alpha_trace"][0] == rm["alpha"]
    assert r["alpha_trace"][-1] == r["alpha"]
    assert oracle.mse(W, r["codes"], r["scales"], r["alpha"]) < oracle.mse(W, rm["codes"], rm["scales"], rm["alpha"])
    # stored scales are the E4M3 roundings of the unrounded ones
    assert np.array_equal(oracle.e4m3_rne_many(r["dstar"]), r["scales"].reshape(-1))


@pytest.mark.parametrize("mode", ["cjso", "soar"])
def test_on_grid_is_a_fixed_point(mode):
    W, alpha0, dcode, q = indep.on_grid_matrix(4, 128, -8, seed=9)
    r = oracle.quantize(W, mode, 3)
    assert r["alpha"] == alpha0
    assert np.array_equal(r["scales"], dcode)
    assert np.array_equal(indep.unpack(r["codes"]), q)


# ---------------------------------------------------------------------------------------------- SOAR

def test_soar_never_worse_than_cjso_and_matches_rescoring():
    W = synth.normal_bf16(32, 256, seed=11)
    rc = oracle.quantize(W, "cjso", 4)
    rs = oracle.quantize(W, "soar", 4)
    assert rs["alpha"] == rc["alpha"]
    ec = indep.block_errors(W, rc["codes"], rc["scales"], rc["alpha"])
    es = indep.block_errors(W, rs["codes"], rs["scales"], rs["alpha"])
    assert np.all(es <= ec * (1 + 1e-12))
    assert np.mean(es < ec) > 0.1
    alpha = rc["alpha"]
    w = indep.as_f32(W).reshape(-1, 16)
    fk = [indep.nearest_f32(Fraction(50 + k, 100)) for k in range(101)]
    dc_all = rc["scales"].reshape(-1)
    ds_all = rc["dstar"].reshape(-1)
    got_codes = indep.unpack(rs["codes"]).reshape(-1, 16)
    got_scales = rs["scales"].reshape(-1)
    ambiguous = 0
    for b in range(0, w.shape[0], 3):
        dcv = indep.E4M3_POS[dc_all[b]]
        lo = int(np.searchsorted(indep.E4M3_POS, ds_all[b], side="right") - 1)
        lo = min(lo, 0x7E)
        hi = lo if (indep.E4M3_POS[lo] == ds_all[b] or lo == 0x7E) else lo + 1
        best_c = indep.quantize_block_np(w[b], alpha, dcv)
        best_e = indep.block_err_np(w[b], best_c, alpha, dcv)
        best = (best_c, dc_all[b])
        errs = [best_e]
        for k in range(101):
            dq = np.float32(np.float32(dcv) * fk[k])
            c = indep.quantize_block_np(w[b], alpha, dq)
            for d in (lo, hi):
                e = indep.block_err_np(w[b], c, alpha, indep.E4M3_POS[d])
                errs.append(e)
                if e < best_e:
                    best_e, best = e, (c, d)
        errs = np.array(errs)
        close = np.sum(np.abs(errs - best_e) <= 1e-12 * best_e) - np.sum(errs == best_e)
        if close:
            ambiguous += 1
            continue
        assert np.array_equal(got_codes[b], best[0]) and got_scales[b] == best[1], b
    assert ambiguous < 3


def test_soar_blocks_matches_whole_matrix_run():
    W = synth.normal_bf16(16, 128, seed=12)
    rs = oracle.quantize(W, "soar", 2)
    rc = oracle.quantize(W, "cjso", 2)
    blocks = np.arange(0, 128, 5)
    c, s = oracle.soar_blocks(W, rc["alpha"], rc["scales"], rc["dstar"], blocks)
    assert np.array_equal(c, rs["codes"].reshape(-1, 8)[blocks])
    assert np.array_equal(s, rs["scales"].reshape(-1)[blocks])


def test_soar_zero_iterations_not_worse_than_max():
    W = synth.c1(0)[:64]
    rm = oracle.quantize(W, "max")
    rs = oracle.quantize(W, "soar", 0)
    em = indep.block_errors(W, rm["codes"], rm["scales"], rm["alpha"])
    es = indep.block_errors(W, rs["codes"], rs["scales"], rs["alpha"])
    assert np.all(es <= em * (1 + 1e-12))


# ---------------------------------------------------------------------------------------- edge cases

@pytest.mark.parametrize("mode", ["max", "4o6", "cjso", "soar"])
@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_nonfinite_input(mode, bad):
    W = synth.normal_f32(4, 64, seed=1)
    W[2, 17] = bad
    r = oracle.quantize(W, mode, 2)
    assert r["status"] == 1 and np.isnan(r["alpha"])
    assert not r["codes"].any() and not r["scales"].any()


@pytest.mark.parametrize("mode", ["max", "4o6", "cjso", "soar"])
def test_all_zero_input(mode):
    W = np.zeros((4, 64), np.uint16)
    W[1, 3] = 0x8000  # -0.0
    r = oracle.quantize(W, mode, 2)
    assert r["status"] == 0 and r["alpha"] == 0.0
    assert not r["codes"].any() and not r["scales"].any()


@pytest.mark.parametrize("mode", ["max", "4o6", "cjso", "soar"])
def test_zero_block_and_tiny_blocks(mode):
    W = synth.normal_f32(4, 64, seed=2)
    W[1, 16:32] = 0.0
    W[2, 32:48] *= 1e-6  # scale underflows E4M3: Delta = 0, codes 0
    r = oracle.quantize(W, mode, 2)
    s = r["scales"].reshape(-1)
    c = r["codes"].reshape(-1, 8)
    assert s[5] == 0 and not c[5].any()
    assert s[10] == 0 and not c[10].any()


def test_tiny_magnitude_matrix_is_consistent():
    W = (synth.normal_f32(2, 32, seed=3) * 1e-36).astype(np.float32)
    for mode in ("max", "4o6", "cjso", "soar"):
        r = oracle.quantize(W, mode, 1)
        assert r["status"] == 0 and r["alpha"] > 0
        c = indep.unpack(r["codes"])
        assert np.all((c != 8))


def test_bad_arguments():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((4, 24), np.float32), "max")


# ------------------------------------------------------------------- CJSO / SOAR from FourOverSix

@pytest.mark.parametrize("gen", [lambda: synth.c1(0)[:64], lambda: synth.c2(0, 64, 512),
                                 lambda: indep.on_grid_matrix(16, 128, -6, 2)[0]])
def test_init_4o6_zero_rounds_equals_4o6(gen):
    """With no rounds, CJSO started from FourOverSix is FourOverSix (codes, scales, alpha)."""
    W = gen()
    r4 = oracle.quantize(W, "4o6")
    rc = oracle.quantize(W, "cjso", 0, init="4o6")
    assert rc["alpha"] == r4["alpha"]
    assert np.array_equal(rc["codes"], r4["codes"]) and np.array_equal(rc["scales"], r4["scales"])


def test_init_4o6_unrounded_scales():
    """The unrounded starting scale (what the search brackets at T = 0) is max|w|/(6 alpha) where
    FourOverSix kept M=6 and 1.5 * Delta6 where it took M=4 (Delta6 = the max rule's scale)."""
    W = synth.c2(0, 64, 512)
    rm = oracle.quantize(W, "max")
    r4 = oracle.quantize(W, "4o6")
    rc = oracle.quantize(W, "cjso", 0, init="4o6")
    alpha = rm["alpha"]
    w = indep.as_f32(W).reshape(-1, 16).astype(np.float64)
    amax = np.abs(w).max(axis=1)
    d6 = indep.E4M3_POS[rm["scales"].reshape(-1)]
    m4 = r4["mchoice"].reshape(-1).astype(bool)
    want = np.where(m4, 1.5 * d6, amax / (6.0 * float(np.float32(alpha))))
    assert m4.any() and (~m4).any()
    assert np.array_equal(rc["dstar"].reshape(-1)[m4], want[m4])
    assert np.allclose(rc["dstar"].reshape(-1)[~m4], want[~m4], rtol=1e-15, atol=0)


def test_soar_from_4o6_never_worse_and_matches_rescoring():
    """SOAR from FourOverSix: per block no worse than its CJSO point, and its choice equals an
    independent scoring of the 202 candidates plus the incumbent."""
    W = synth.normal_bf16(16, 256, seed=21)
    rc = oracle.quantize(W, "cjso", 3, init="4o6")
    rs = oracle.quantize(W, "soar", 3, init="4o6")
    assert rs["alpha"] == rc["alpha"]
    ec = indep.block_errors(W, rc["codes"], rc["scales"], rc["alpha"])
    es = indep.block_errors(W, rs["codes"], rs["scales"], rs["alpha"])
    assert np.all(es <= ec * (1 + 1e-12))
    alpha = rc["alpha"]
    w = indep.as_f32(W).reshape(-1, 16)
    fk = [indep.nearest_f32(Fraction(50 + k, 100)) for k in range(101)]
    dc_all, ds_all = rc["scales"].reshape(-1), rc["dstar"].reshape(-1)
    got_codes, got_scales = indep.unpack(rs["codes"]).reshape(-1, 16), rs["scales"].reshape(-1)
    ambiguous = 0
    for b in range(0, w.shape[0], 7):
        dcv = indep.E4M3_POS[dc_all[b]]
        lo = min(int(np.searchsorted(indep.E4M3_POS, ds_all[b], side="right") - 1), 0x7E)
        hi = lo if (indep.E4M3_POS[lo] == ds_all[b] or lo == 0x7E) else lo + 1
        best_c = indep.quantize_block_np(w[b], alpha, dcv)
        best_e, best_s = indep.block_err_np(w[b], best_c, alpha, dcv), dc_all[b]
        errs = [best_e]
        for k in range(101):
            c = indep.quantize_block_np(w[b], alpha, np.float32(np.float32(dcv) * fk[k]))
            for d in (lo, hi):
                e = indep.block_err_np(w[b], c, alpha, indep.E4M3_POS[d])
                errs.append(e)
                if e < best_e:
                    best_c, best_e, best_s = c, e, d
        errs = np.array(errs)
        # binary64 scoring cannot order errors closer than its rounding: such blocks are skipped
        if np.sum(np.abs(errs - best_e) <= 1e-12 * best_e) > np.sum(errs == best_e):
            ambiguous += 1
            continue
        assert got_scales[b] == best_s and np.array_equal(got_codes[b], best_c), b
    assert ambiguous < 3


def test_init_4o6_rejected_for_max_and_4o6():
    W = synth.c1(0)[:4]
    for mode in ("max", "4o6"):
        with pytest.raises(ValueError):
            oracle.quantize(W, mode, 0, init="4o6")
