"""Pins of the oracle's number formats (CPU only).

E2M1 is checked against an exhaustive nearest-value search over every bf16 pattern, dense neighbourhoods
of every grid value and midpoint, and millions of random binary32 patterns; E4M3 against torch's
float8_e4m3fn and an exhaustive nearest-value search; the search multipliers against exact rational
rounding.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import indep


def test_e2m1_value_table_matches_pages():
    got = np.array([oracle.e2m1_value(c) for c in range(16)], np.float64)
    assert np.array_equal(got, indep.E2M1_VALUES)
    assert np.array_equal(np.signbit(got), np.signbit(indep.E2M1_VALUES))
    assert indep.GRID.max() == indep.golden_constants()["M_FP4"]


def _neighbourhood(vals, width=512):
    out = []
    for v in vals:
        c = np.float32(v)
        up, dn = c, c
        seq = [c]
        for _ in range(width):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(-np.inf))
            seq += [up, dn]
        out.append(np.array(seq, np.float32))
    a = np.concatenate(out)
    return np.concatenate([a, -a])


def test_e2m1_exhaustive_bf16_patterns():
    x = (np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)).view(np.float32)
    assert np.array_equal(oracle.e2m1_codes(x), indep.brute_e2m1(x))


def test_e2m1_grid_points_and_midpoints():
    special = list(indep.GRID) + [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.0, 8.0]
    x = _neighbourhood(special)
    assert np.array_equal(oracle.e2m1_codes(x), indep.brute_e2m1(x))


def test_e2m1_random_patterns():
    g = np.random.default_rng(1)
    bits = g.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([bits.view(np.float32), g.uniform(-8, 8, 2_000_000).astype(np.float32)])
    assert np.array_equal(oracle.e2m1_codes(x), indep.brute_e2m1(x))


def test_e2m1_fixed_cases():
    # ties go to the even code; above 6 saturates; a negative value rounding to zero has code 0
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 6.5: 7, 1e30: 7,
             float("inf"): 7, -float("inf"): 15, -0.2: 0, -0.0: 0, float("nan"): 0, -5.5: 15, 0.26: 1}
    for x, c in cases.items():
        assert oracle.e2m1_code(x) == c, x


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    got = np.array([oracle.e4m3_value(int(c)) for c in codes])
    assert np.array_equal(got, indep.e4m3_decode(codes))
    assert oracle.e4m3_value(0x7E) == indep.golden_constants()["M_FP8"]


def _e4m3_samples():
    g = np.random.default_rng(2)
    pos = indep.E4M3_POS
    mids = (pos[1:] + pos[:-1]) / 2
    bf = (np.arange(0x4400, dtype=np.uint32) << np.uint32(16)).view(np.float32)  # 0 .. 512 in bf16
    bf = bf[bf <= 464]
    return np.concatenate([bf, _neighbourhood(mids, 64), _neighbourhood(pos, 8),
                           g.uniform(0, 464, 400_000).astype(np.float32),
                           (2.0 ** g.uniform(-12, 9, 400_000)).astype(np.float32)])


def test_e4m3_rne_matches_torch_and_brute_force():
    v = _e4m3_samples()
    v = v[~np.signbit(v) & (v <= 464)]
    got = oracle.e4m3_rne_many(v.astype(np.float64))
    assert np.array_equal(got, indep.torch_e4m3(v))
    assert np.array_equal(got, indep.brute_e4m3(v))


def test_e4m3_fixed_cases_and_saturation():
    assert oracle.e4m3_rne(1.6875) == 62   # tie -> 1.75 (even mantissa)
    assert oracle.e4m3_rne(2.0625) == 64   # tie -> 2
    assert oracle.e4m3_rne(2.0 ** -10) == 0
    assert oracle.e4m3_rne(1.5 * 2.0 ** -9) == 2
    for v in (448.0, 463.9, 464.0, 470.0, 1e6, 1e300, float("inf")):
        assert oracle.e4m3_rne(v) == 0x7E


def test_e4m3_bracket():
    v = _e4m3_samples().astype(np.float64)
    v = np.concatenate([v[~np.signbit(v)], [0.0, 448.0, 500.0, 1e9]])
    for x in v[::97]:
        lo, hi = oracle.e4m3_bracket(float(x))
        vl, vh = oracle.e4m3_value(lo), oracle.e4m3_value(hi)
        if x >= 448:
            assert lo == hi == 0x7E
            continue
        assert vl <= x <= vh
        assert hi - lo in (0, 1)
        assert (lo == hi) == (vl == x)
        assert oracle.e4m3_rne(float(x)) in (lo, hi)


def test_search_multipliers_are_nearest_binary32():
    c = indep.golden_constants()
    n = int(round((c["SEARCH_HI"] - c["SEARCH_LO"]) / c["SEARCH_STEP"])) + 1
    assert n == 101 and n * int(c["DELTA_D_CANDIDATES"]) == 202
    for k in range(n):
        fr = Fraction(50 + k, 100)
        assert np.float32(oracle.search_multiplier(k)) == indep.nearest_f32(fr), k
    assert oracle.search_multiplier(0) == 0.5 and oracle.search_multiplier(50) == 1.0
    assert oracle.search_multiplier(100) == 1.5


def test_torch_float8_is_the_expected_format():
    # guards the library pin itself: OCP E4M3 "fn" (bias 7, max 448, no infinities)
    assert torch.finfo(torch.float8_e4m3fn).max == 448.0
    assert torch.tensor([2.0 ** -9]).to(torch.float8_e4m3fn).view(torch.uint8).item() == 1
