// Device-side number formats and exact comparison helpers for the gfx950 NVFP4 quantizer.
//
// Formats (SOAR page, quantisation definitions; FourOverSix write-up, section 01):
//   E2M1: sign | 2 exponent bits | 1 mantissa bit, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.
//   E4M3 (the "FN" variant): sign | 4 exponent bits (bias 7) | 3 mantissa bits, subnormals m*2^-9, no
//   infinities, largest finite value 448 (code 0x7E).
//
// E2M1 rounding uses gfx950's v_cvt_scalef32_pk_fp4_f32 with a scale of 1.0. On every binary32 input
// it returns the nearest E2M1 value with ties to the even code and saturates to +-6 (infinities
// included); the two differences from the rule the quantiser follows are repaired where it matters:
// a negative value that rounds to zero comes back as code 0x8 (cleared by e2m1_clear_negzero) and
// NaN maps to a nonzero code (the callers never feed NaN to it). Decoding uses
// v_cvt_scalef32_pk_bf16_fp4 / _pk_f32_fp4 (exact for all 16 codes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t d) { return __builtin_bit_cast(bf16x2, d); }

// ---------------------------------------------------------------------------------------- E4M3

// Value of a non-negative finite E4M3 code (0x00..0x7E). A normal code c = 8e + m (e >= 1) is the binary32
// pattern with exponent field e + 120 and m in the top three significand bits, i.e. (c + 960) << 20; a
// subnormal one is m * 2^-9. Both are formed and one is selected (no branch).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    const float nor = __uint_as_float((c << 20) + 0x3C000000u);
    const float sub = (float)c * 0x1p-9f;
    return c >= 8u ? nor : sub;
}

// Nearest E4M3 value to v >= 0 (ties to the even code), values >= 448 saturate to 448. Exact for any
// binary64 v: v is scaled by a power of two so that the E4M3 spacing around it becomes 1, and the
// integer rounding is done by rint (round half to even).
__device__ __forceinline__ uint32_t e4m3_rne(double v) {
    if (!(v > 0.0)) return 0u;
    if (v >= 448.0) return 0x7Eu;
    int e = ilogb(v);
    e = e < -6 ? -6 : e;
    double m = rint(ldexp(v, 3 - e));
    uint32_t c = (uint32_t)(8 * (e + 6)) + (uint32_t)m;
    return c > 0x7Eu ? 0x7Eu : c;
}

// e4m3_rne(x / y) for x >= 0, y > 0 whose binary32 roundings are within 2^-24 of them, decided from the
// binary32 estimate q = fl(x) * rcp(fl(y)) where that is safe; returns false (code unset) otherwise. The
// estimate is within 5 binary32 ulps of x / y (two roundings of the operands, v_rcp_f32's 1 ulp, the
// product's rounding), and every E4M3 midpoint in the normal range has the binary32 pattern ...m m m 1
// followed by 19 zero bits. So when q lies in [2^-6, 2^10) and more than 32 ulps from such a pattern,
// x / y lies on the same side of every midpoint as q, and rounding q's significand to 3 bits (add half an
// E4M3 step, truncate; no tie is possible) gives the code of x / y, clamped to 448.
__device__ __forceinline__ bool e4m3_quotient_est(float x, float y, uint32_t &code) {
    const float q = x * __builtin_amdgcn_rcpf(y);
    const uint32_t u = __float_as_uint(q);
    const bool far = ((u + 0x80000u + 32u) & 0xFFFFFu) >= 64u;
    const uint32_t c = ((u + 0x80000u) >> 20) - 960u;  // (biased exponent, 3 bits) minus E4M3's bias
    code = c < 0x7Eu ? c : 0x7Eu;
    return far && q >= 0x1p-6f && q < 0x1p10f;
}

// e4m3_rne(v) for a binary32 v in E4M3's normal range (v >= 2^-6; false, code unset, below it): the
// significand rounded to 3 bits with ties to even (add 2^19 - 1 plus the kept last bit, truncate), clamped
// to 448.
__device__ __forceinline__ bool e4m3_rne_normal(float v, uint32_t &code) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t c = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - 960u;
    code = c < 0x7Eu ? c : 0x7Eu;
    return v >= 0x1p-6f;
}

// The E4M3 codes around v >= 0: lo = largest value <= v, hi = smallest value >= v (both 448 when
// v >= 448, both 0 when v <= 0).
__device__ __forceinline__ void e4m3_bracket(double v, uint32_t &lo, uint32_t &hi) {
    if (!(v > 0.0)) {
        lo = hi = 0u;
        return;
    }
    if (v >= 448.0) {
        lo = hi = 0x7Eu;
        return;
    }
    int e = ilogb(v);
    e = e < -6 ? -6 : e;
    double t = ldexp(v, 3 - e);
    uint32_t base = (uint32_t)(8 * (e + 6));
    lo = base + (uint32_t)floor(t);
    hi = base + (uint32_t)ceil(t);
    if (hi > 0x7Eu) hi = 0x7Eu;
}

// ---------------------------------------------------------------------------------------- E2M1

// Eight binary32 values -> eight E2M1 codes packed in a dword (value 2k in the low nibble of byte k).
__device__ __forceinline__ uint32_t e2m1_pack8(float x0, float x1, float x2, float x3, float x4, float x5,
                                               float x6, float x7) {
    uint32_t v = 0u;
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, x0, x1, 1.0f, 0);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, x2, x3, 1.0f, 1);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, x4, x5, 1.0f, 2);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, x6, x7, 1.0f, 3);
    return v;
}

// Code 0x8 (negative zero) -> 0x0 in every nibble; other codes unchanged.
__device__ __forceinline__ uint32_t e2m1_clear_negzero(uint32_t c) {
    uint32_t mag = c & 0x77777777u;
    uint32_t nz = (mag + 0x77777777u) & 0x88888888u;  // bit 3 of a nibble set iff its magnitude != 0
    return mag | (c & nz);
}

// Software E2M1 of one binary32 value (the rule spelled out: nearest magnitude, ties to the even
// code, saturate above 6, NaN -> 0, sign only on nonzero codes). Used on rare blocks whose scale
// reciprocal overflows, where w * r can be NaN.
__device__ __forceinline__ uint32_t e2m1_soft(float x) {
    float a = fabsf(x);
    uint32_t i = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
                 (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
    return (i != 0u && __builtin_signbit(x)) ? (i | 8u) : i;
}

// ------------------------------------------------------------------------------- reciprocal

// fl(1/s), the correctly rounded binary32 reciprocal, for any s. For 2^-125 <= s < 2^125 it is formed
// as y = v_rcp_f32(s) (about 1 ulp) plus one correction by the exact residual, y + y*(1 - s*y) with both
// steps fused; that equals the IEEE quotient 1/s for every binary32 s in the range (checked on the
// device for every binary32 value in [2^-125, 2^126), and by a GPU test through nvfp4_reciprocal_f32
// over every mantissa at several exponents). Outside the range it is the IEEE division.
// The range test is taken per wave (a ballot), so the common case is straight-line code.
__device__ __forceinline__ float recip_rn(float s) {
    const float y = __builtin_amdgcn_rcpf(s);
    const float r = __builtin_fmaf(__builtin_fmaf(-s, y, 1.0f), y, y);
    const bool fast = s >= 0x1p-125f && s < 0x1p125f;
    if (__builtin_amdgcn_ballot_w64(!fast) != 0) return fast ? r : 1.0f / s;
    return r;
}

// ------------------------------------------------------------------------ exact double-double

struct dd {
    double hi, lo;
};

// a*b exactly, as an unevaluated sum hi + lo with hi = fl(a*b).
__device__ __forceinline__ dd two_prod(double a, double b) {
    double p = a * b;
    return {p, fma(a, b, -p)};
}

// Exact order of two values held as (fl(x), x - fl(x)).
__device__ __forceinline__ bool dd_less(dd a, dd b) { return a.hi < b.hi || (a.hi == b.hi && a.lo < b.lo); }
__device__ __forceinline__ bool dd_equal(dd a, dd b) { return a.hi == b.hi && a.lo == b.lo; }

// Sum of two non-negative double-doubles (relative error about 2^-104).
__device__ __forceinline__ dd dd_add(dd a, dd b) {
    double s = a.hi + b.hi;
    double bb = s - a.hi;
    double err = (a.hi - (s - bb)) + (b.hi - bb);
    double lo = err + a.lo + b.lo;
    double hi = s + lo;
    return {hi, lo - (hi - s)};
}

}  // namespace nvfp4
