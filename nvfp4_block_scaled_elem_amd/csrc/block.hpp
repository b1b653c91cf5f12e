// One NVFP4 block (16 consecutive elements of a row) held in registers by one lane, and the two
// per-block operations every mode is built from:
//   encode: codes of x_j = w_j * r in binary32, r = fl(1/s), s = fl(alpha * Delta)
//   sums:   S_wq = sum_j w_j q_j and S_qq = sum_j q_j^2 of the decoded codes, exactly.
//
// Exactness of the sums. For bf16 input every product w*q has at most 10 significant bits and, when
// q != 0, |w| >= 2^(E-3) where 2^E <= s < 2^(E+1) (x = w*r must exceed 0.25), so every partial sum is
// a multiple of 2^(E-11); while max|w| <= 32*s their magnitude stays below 2^(E+13), i.e. within 24
// bits, and the v_dot2_f32_bf16 accumulation is exact. Blocks outside that window, fp32 input and
// blocks whose reciprocal overflows use binary64 accumulation of the binary32-decoded values.
#pragma once

#include "codec.hpp"

namespace nvfp4 {

// The raw bytes of a block, loaded ahead of use (bf16: 2 x 16 bytes, fp32: 4 x 16 bytes).
template <bool F32>
struct Raw {
    uint4 v[F32 ? 4 : 2];
    __device__ __forceinline__ void load(const void *W, int64_t b) {
        const uint4 *s = reinterpret_cast<const uint4 *>(W) + (F32 ? 4 : 2) * b;
#pragma unroll
        for (int k = 0; k < (F32 ? 4 : 2); ++k) v[k] = s[k];
    }
};

template <bool F32>
struct Blk;

template <>
struct Blk<false> {  // bf16 input: 32 bytes
    float w[16];
    uint32_t p[8];  // the raw bf16 pairs (element 2k low, 2k+1 high)
    __device__ __forceinline__ void set(const Raw<false> &r) {
        p[0] = r.v[0].x; p[1] = r.v[0].y; p[2] = r.v[0].z; p[3] = r.v[0].w;
        p[4] = r.v[1].x; p[5] = r.v[1].y; p[6] = r.v[1].z; p[7] = r.v[1].w;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            w[2 * k] = bf16_lo(p[k]);
            w[2 * k + 1] = bf16_hi(p[k]);
        }
    }
    __device__ __forceinline__ void load(const void *W, int64_t b) {
        Raw<false> r;
        r.load(W, b);
        set(r);
    }
    __device__ __forceinline__ float amax() const {
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(w[j]));
        return a;
    }
};

template <>
struct Blk<true> {  // fp32 input: 64 bytes
    float w[16];
    __device__ __forceinline__ void set(const Raw<true> &r) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            w[4 * k] = __uint_as_float(r.v[k].x);
            w[4 * k + 1] = __uint_as_float(r.v[k].y);
            w[4 * k + 2] = __uint_as_float(r.v[k].z);
            w[4 * k + 3] = __uint_as_float(r.v[k].w);
        }
    }
    __device__ __forceinline__ void load(const void *W, int64_t b) {
        Raw<true> r;
        r.load(W, b);
        set(r);
    }
    __device__ __forceinline__ float amax() const {
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(w[j]));
        return a;
    }
};

// ------------------------------------------------------------------------------------- encode

__device__ __forceinline__ void encode16(const float *w, float r, uint32_t &c0, uint32_t &c1) {
    c0 = e2m1_pack8(w[0] * r, w[1] * r, w[2] * r, w[3] * r, w[4] * r, w[5] * r, w[6] * r, w[7] * r);
    c1 = e2m1_pack8(w[8] * r, w[9] * r, w[10] * r, w[11] * r, w[12] * r, w[13] * r, w[14] * r, w[15] * r);
}

__device__ __forceinline__ void encode16_soft(const float *w, float r, uint32_t &c0, uint32_t &c1) {
    c0 = 0u;
    c1 = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        c0 |= e2m1_soft(w[j] * r) << (4 * j);
        c1 |= e2m1_soft(w[8 + j] * r) << (4 * j);
    }
}

__device__ __forceinline__ bool finite_pos(float r) { return r <= 3.40282347e38f; }

// Codes of a block for the scale s (zero scale -> all codes 0). Negative zeros are not yet cleared.
__device__ __forceinline__ void encode_scale(const float *w, float s, uint32_t &c0, uint32_t &c1) {
    if (s == 0.0f) {
        c0 = c1 = 0u;
        return;
    }
    const float r = 1.0f / s;
    if (finite_pos(r))
        encode16(w, r, c0, c1);
    else
        encode16_soft(w, r, c0, c1);
}

// ------------------------------------------------------------------------------------------ sums

template <int SEL>
__device__ __forceinline__ void acc_bf16(uint32_t c, uint32_t wpair, float &sw, float &sq) {
    const bf16x2 q = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, SEL);
    sw = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wpair), q, sw, false);
    sq = __builtin_amdgcn_fdot2_f32_bf16(q, q, sq, false);
}

__device__ __forceinline__ void sums_bf16(uint32_t c0, uint32_t c1, const uint32_t *p, float &sw, float &sq) {
    sw = 0.0f;
    sq = 0.0f;
    acc_bf16<0>(c0, p[0], sw, sq);
    acc_bf16<1>(c0, p[1], sw, sq);
    acc_bf16<2>(c0, p[2], sw, sq);
    acc_bf16<3>(c0, p[3], sw, sq);
    acc_bf16<0>(c1, p[4], sw, sq);
    acc_bf16<1>(c1, p[5], sw, sq);
    acc_bf16<2>(c1, p[6], sw, sq);
    acc_bf16<3>(c1, p[7], sw, sq);
}

// The value itself, opaque to the optimiser: keeps the widening of w for the rare binary64 path inside
// that path (the compiler otherwise hoists it in front of the branch, onto every block).
__device__ __forceinline__ float opaque(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

template <int SEL>
__device__ __forceinline__ void acc_f64(uint32_t c, float w0, float w1, double &sw, double &sq) {
    const f32x2 q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, SEL);
    const double q0 = (double)q.x, q1 = (double)q.y;
    sw = fma((double)opaque(w0), q0, sw);
    sw = fma((double)opaque(w1), q1, sw);
    sq = fma(q0, q0, sq);
    sq = fma(q1, q1, sq);
}

__device__ __forceinline__ void sums_f64(uint32_t c0, uint32_t c1, const float *w, double &sw, double &sq) {
    sw = 0.0;
    sq = 0.0;
    acc_f64<0>(c0, w[0], w[1], sw, sq);
    acc_f64<1>(c0, w[2], w[3], sw, sq);
    acc_f64<2>(c0, w[4], w[5], sw, sq);
    acc_f64<3>(c0, w[6], w[7], sw, sq);
    acc_f64<0>(c1, w[8], w[9], sw, sq);
    acc_f64<1>(c1, w[10], w[11], sw, sq);
    acc_f64<2>(c1, w[12], w[13], sw, sq);
    acc_f64<3>(c1, w[14], w[15], sw, sq);
}

// Work-group barrier for data exchanged through LDS only. The fences cover the local address space, so
// global loads and stores still in flight (a block prefetched before a kernel's prologue, a partial
// result written for the next kernel) are not waited for, unlike __syncthreads.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s = fl(alpha * Delta) and r = fl(1/s) (0 for s = 0) for every E4M3 code, built once per work-group.
struct ScaleTab {
    float s[128];
    float r[128];
};

template <int THREADS>
__device__ __forceinline__ void build_scale_tab(ScaleTab &T, float alpha) {
    for (int c = threadIdx.x; c < 128; c += THREADS) {
        const float s = c < 0x7F ? alpha * e4m3_value((uint32_t)c) : 0.0f;
        T.s[c] = s;
        T.r[c] = s == 0.0f ? 0.0f : 1.0f / s;
    }
    lds_barrier();
}

// Codes for the scale s (reciprocal r = fl(1/s), or 0 when s = 0: every code is then 0) and the exact
// sums of the block.
template <bool F32>
__device__ __forceinline__ void quant_sums_r(const Blk<F32> &B, float amax, float s, float r, uint32_t &c0,
                                             uint32_t &c1, double &sw, double &sq) {
    const bool rfin = finite_pos(r);
    if (rfin)
        encode16(B.w, r, c0, c1);
    else
        encode16_soft(B.w, r, c0, c1);
    if constexpr (!F32) {
        if (rfin && amax <= 32.0f * s && amax <= 0x1p100f) {
            float a, q;
            sums_bf16(c0, c1, B.p, a, q);
            sw = a;
            sq = q;
            return;
        }
    }
    sums_f64(c0, c1, B.w, sw, sq);
}

template <bool F32>
__device__ __forceinline__ void quant_sums(const Blk<F32> &B, float amax, float s, uint32_t &c0, uint32_t &c1,
                                           double &sw, double &sq) {
    quant_sums_r(B, amax, s, s == 0.0f ? 0.0f : 1.0f / s, c0, c1, sw, sq);
}

// Running sum hi + lo of exact binary64 terms: TwoSum into hi, errors gathered in lo (renormalised by
// dd_add when partial sums are combined).
__device__ __forceinline__ void acc2(dd &A, double x_hi, double x_lo) {
    const double s = A.hi + x_hi;
    const double bb = s - A.hi;
    const double e = (A.hi - (s - bb)) + (x_hi - bb);
    A.hi = s;
    A.lo += e + x_lo;
}

}  // namespace nvfp4
