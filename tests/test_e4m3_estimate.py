"""The binary32 shortcuts the quantiser kernels take for E4M3 roundings and E2M1 certificates, checked on the CPU.

Two shortcuts replace a binary64 division and rounding in the common case:

* e4m3_quotient_est (codec.hpp): the E4M3 code of x / y (the max rule's max|w| / (6 alpha), the CJSO
  block-scale step's S_wq / (alpha S_qq)) from q = fl(x) * rcp(fl(y)). It claims the code only when q is in
  [2^-6, 2^10) and more than 32 binary32 ulps from every E4M3 midpoint, and otherwise leaves the block to
  the binary64 quotient.
* e4m3_rne_normal (codec.hpp): the E4M3 rounding (ties to even) of an exact binary32 value in E4M3's
  normal range by integer arithmetic on its bits (FourOverSix's E4M3(1.5 Delta6)).

A third one decides, in the decoupled search (soar_kernel.hip, eval_r_far), that a block's codes are the
nearest E2M1 values of the exact quotients |w| / (alpha Delta): every computed x = fl(w fl(1/fl(alpha Delta)))
(within 3 * 2^-24 of its quotient) must lie more than 8 binary32 ulps from every value whose low 21
significand bits are zero, which every E2M1 decision point is. The search's band candidates (window_best)
use the same test with a 32-ulp margin, for quotients within 2^-20 + 2^-23 + 2^-40 of x.

Two exact rewrites are checked as well: the branch-free E4M3 decode (e4m3_value) over every code, and the
search's test that every reciprocal is finite, !(0 < s <= 2^-128), against binary32 division.

The device instructions are modelled here in numpy binary32 arithmetic, v_rcp_f32 as the correctly rounded
reciprocal and one ulp either side of it. The reference is the E4M3 rule itself (nearest value, ties to
the even code, saturation at 448) applied to the binary64 quotient, as the kernels' general path does.
Whenever a shortcut claims a code, the code must be the reference's. The GPU parity tests check the
kernels themselves against the oracle, including every block of the full-size matrices, where some dozens
of blocks per pass fall back from the estimate.
"""
import numpy as np
import pytest

E4M3_MAX_CODE = 0x7E


def e4m3_rne(v):
    """Nearest E4M3 code to v >= 0 (ties to even, values >= 448 saturate), exact for binary64 v."""
    v = np.asarray(v, dtype=np.float64)
    pos = (v > 0) & (v < 448.0)
    w = np.where(pos, v, 1.0)
    _, e = np.frexp(w)  # w = f * 2^e with f in [0.5, 1)
    e = np.maximum(e - 1, -6)
    m = np.rint(np.ldexp(w, 3 - e)).astype(np.int64)  # rint: half to even
    c = np.minimum(8 * (e + 6) + m, E4M3_MAX_CODE)
    return np.where(pos, c, np.where(v >= 448.0, E4M3_MAX_CODE, 0))


def quotient_est(x32, y32, rcp_ulps):
    """Model of e4m3_quotient_est: (claimed, code)."""
    r = (np.float32(1.0) / y32).astype(np.float32)
    if rcp_ulps:
        r = np.nextafter(r, np.float32(np.inf if rcp_ulps > 0 else 0.0), dtype=np.float32)
    q = (x32 * r).astype(np.float32)
    u = q.view(np.uint32).astype(np.int64)
    far = ((u + 0x80000 + 32) & 0xFFFFF) >= 64
    code = np.minimum(((u + 0x80000) >> 20) - 960, E4M3_MAX_CODE)
    return far & (q >= np.float32(2.0 ** -6)) & (q < np.float32(2.0 ** 10)), code


def rne_normal(v32):
    """Model of e4m3_rne_normal: (claimed, code)."""
    u = v32.view(np.uint32).astype(np.int64)
    code = np.minimum(((u + 0x7FFFF + ((u >> 20) & 1)) >> 20) - 960, E4M3_MAX_CODE)
    return v32 >= np.float32(2.0 ** -6), code


def test_reference_rule_on_known_values():
    # E4M3 values and midpoints: 1.0 = code 56, 1.125 = 57, midpoint 1.0625 goes to the even code 56,
    # 1.1875 (between 57 and 58) to 58; 448 = 126; 2^-9 = code 1; half of it rounds to 0 (even).
    got = e4m3_rne([1.0, 1.125, 1.0625, 1.1875, 448.0, 1e9, 2.0 ** -9, 2.0 ** -10, 0.0, 464.0])
    assert list(got) == [56, 57, 56, 58, 126, 126, 1, 0, 0, 126]


@pytest.mark.parametrize("case", ["random", "near_midpoints", "range_ends"])
def test_quotient_estimate_claims_only_exact_codes(case):
    rng = np.random.default_rng({"random": 1, "near_midpoints": 2, "range_ends": 3}[case])
    n = 400_000
    claimed_total = 0
    for trial in range(6):
        alpha = np.float32(2.0 ** rng.uniform(-30, 5))
        sq = rng.integers(1, 2305, n) / 4.0  # S_qq: a multiple of 1/4 up to 16 * 36
        if case == "random":
            target = np.exp2(rng.uniform(-10, 10, n))
        elif case == "near_midpoints":
            codes = rng.integers(8, 126, n)
            mid = np.ldexp(1 + (codes % 8 + 0.5) / 8, codes // 8 - 7)
            target = mid * (1 + rng.integers(-80, 81, n) * 2.0 ** -24)
        else:
            ends = np.array([2.0 ** -6, 448.0, 464.0, 2.0 ** 10, 0.9375 * 2.0 ** -6])
            target = ends[rng.integers(0, len(ends), n)] * (1 + rng.integers(-80, 81, n) * 2.0 ** -24)
        sw = target * (np.float64(alpha) * sq)
        if trial % 2:
            sw = sw.astype(np.float32).astype(np.float64)  # numerators exact in binary32 (bf16 sums)
        ref = e4m3_rne(sw / (np.float64(alpha) * sq))
        x32 = sw.astype(np.float32)
        y32 = (alpha * sq.astype(np.float32)).astype(np.float32)
        for ulps in (-1, 0, 1):
            claimed, code = quotient_est(x32, y32, ulps)
            assert np.array_equal(code[claimed], ref[claimed])
            claimed_total += int(claimed.sum())
    if case == "random":
        assert claimed_total > 0.6 * 6 * 3 * n  # the estimate decides the common case


def test_max_rule_estimate_claims_only_exact_codes():
    # max|w| (a bf16 value) over fl(6 alpha), against E4M3(max|w| / (6 alpha)) in binary64
    rng = np.random.default_rng(4)
    for _ in range(6):
        alpha = np.float32(2.0 ** rng.uniform(-20, 0))
        a = (np.exp2(rng.uniform(-12, 12, 500_000)) * np.float64(alpha)).astype(np.float32)
        a = (a.view(np.uint32) & 0xFFFF0000).view(np.float32)  # bf16 values
        ref = e4m3_rne(a.astype(np.float64) / (6.0 * np.float64(alpha)))
        for ulps in (-1, 0, 1):
            claimed, code = quotient_est(a, np.float32(6.0) * alpha, ulps)
            assert np.array_equal(code[claimed], ref[claimed])


def test_rne_normal_on_every_five_bit_value_and_more():
    # 1.5 * Delta6 (at most 5 significant bits) for every E4M3 value Delta6, and every binary32 value with 8
    # significant bits from 2^-8 to 2^11, ties included; claimed exactly from 2^-6 up
    e4m3_values = [m * 2.0 ** -9 for m in range(1, 8)] + [
        (1 + m / 8.0) * 2.0 ** e for e in range(-6, 9) for m in range(8) if (1 + m / 8.0) * 2.0 ** e <= 448.0]
    mant = np.arange(128, 256) / 128.0
    v = np.concatenate([1.5 * np.array(e4m3_values)] +
                       [mant * 2.0 ** e for e in range(-8, 12)]).astype(np.float32)
    claimed, code = rne_normal(v)
    assert np.array_equal(claimed, v >= np.float32(2.0 ** -6))
    assert np.array_equal(code[claimed], e4m3_rne(v.astype(np.float64))[claimed])


def e2m1_magnitude_code(a):
    """E2M1 magnitude code of |a|: nearest of 0, .5, 1, 1.5, 2, 3, 4, 6, ties to the even code, saturating."""
    a = np.abs(np.asarray(a, dtype=np.float64))
    return ((a > 0.25).astype(int) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5.0))


def certificate_far(x32, margin=8):
    """Model of eval_r_far's test: ((bits + margin) << 11) mod 2^32 >= (2 margin + 1) << 11."""
    u = x32.view(np.uint32).astype(np.uint64)
    return (((u + margin) << 11) & 0xFFFFFFFF) >= ((2 * margin + 1) << 11)


def test_e2m1_certificate_keeps_codes_within_the_rounding_bound():
    # every binary32 value within 4096 ulps of each decision point, both signs, and random magnitudes up to 8
    vals = [np.arange(int(np.float32(t).view(np.uint32)) - 4096, int(np.float32(t).view(np.uint32)) + 4097,
                      dtype=np.int64).astype(np.uint32).view(np.float32)
            for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)]
    vals.append(np.random.default_rng(5).uniform(0, 8, 1_000_000).astype(np.float32))
    x = np.concatenate(vals)
    x = np.concatenate([x, -x])
    far = certificate_far(x)
    for rel in (3 * 2.0 ** -24, -3 * 2.0 ** -24):  # the exact quotient u with |u - x| <= 3 * 2^-24 |u|
        u = x.astype(np.float64) / (1 - rel)
        assert np.array_equal(e2m1_magnitude_code(u)[far], e2m1_magnitude_code(x)[far])
    assert not certificate_far(np.array([0.25, -0.75, 5.0, 0.0], dtype=np.float32)).any()
    assert far.mean() > 0.99  # values near a decision point are the rare ones


def test_e2m1_certificate_with_the_band_margin():
    # the search's band candidate: its scale s_k lies within 2^-20 of the reconstruct scale s_d, so x = fl(w fl(1/s_k))
    # is within (1 + 2^-20)(1 + 2^-24)^2 - 1 < 2^-20 + 2^-23 + 2^-40 of u = |w| / s_d; a 32-ulp margin (at least 2^-19
    # relative) must keep x's code for every such u, and an 8-ulp one must not
    vals = [np.arange(int(np.float32(t).view(np.uint32)) - 8192, int(np.float32(t).view(np.uint32)) + 8193,
                      dtype=np.int64).astype(np.uint32).view(np.float32)
            for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)]
    vals.append(np.random.default_rng(6).uniform(0, 8, 1_000_000).astype(np.float32))
    x = np.concatenate(vals)
    x = np.concatenate([x, -x])
    bound = 2.0 ** -20 + 2.0 ** -23 + 2.0 ** -40
    far = certificate_far(x, margin=32)
    for rel in (bound, -bound):
        u = x.astype(np.float64) / (1 - rel)
        assert np.array_equal(e2m1_magnitude_code(u)[far], e2m1_magnitude_code(x)[far])
    narrow = certificate_far(x, margin=8)
    u = x.astype(np.float64) / (1 - bound)
    assert not np.array_equal(e2m1_magnitude_code(u)[narrow], e2m1_magnitude_code(x)[narrow])
    assert far.mean() > 0.99


def test_e4m3_decode_without_a_branch():
    # e4m3_value (codec.hpp): a normal code c >= 8 is the binary32 pattern (c << 20) + 0x3C000000, a subnormal
    # one c * 2^-9; against the format's definition for every code 0..126
    c = np.arange(127, dtype=np.uint32)
    normal = ((c << 20) + np.uint32(0x3C000000)).view(np.float32)
    sub = c.astype(np.float32) * np.float32(2.0 ** -9)
    got = np.where(c >= 8, normal, sub).astype(np.float64)
    e, m = c // 8, c % 8
    want = np.where(e > 0, (1 + m / 8.0) * 2.0 ** (e.astype(np.int64) - 7), m * 2.0 ** -9)
    assert np.array_equal(got, want)
    assert got[126] == 448.0 and got[8] == 2.0 ** -6 and got[1] == 2.0 ** -9


def test_reciprocal_finite_exactly_above_two_to_minus_128():
    # the search's "every reciprocal is finite" test, !(0 < s <= 2^-128), against fl(1/s) in binary32 over every
    # binary32 value from 2^-131 to 2^-125 (and zero, whose reciprocal the search takes as 0)
    lo, hi = np.float32(2.0 ** -131).view(np.uint32), np.float32(2.0 ** -125).view(np.uint32)
    s = np.arange(int(lo), int(hi) + 1, dtype=np.uint32).view(np.float32)
    with np.errstate(over="ignore", divide="ignore"):
        finite = np.isfinite(np.float32(1) / s)
        assert not np.isfinite(np.float32(1) / np.float32(2.0 ** -128))
    assert np.array_equal(finite, ~((s > 0) & (s <= np.float32(2.0 ** -128))))
