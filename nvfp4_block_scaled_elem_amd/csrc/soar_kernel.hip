// gfx950 kernel for the decoupled quantise/dequantise block-scale search of the SOAR page ("SOAR:
// Scale Optimization for Accurate Reconstruction in NVFP4 Quantization", decoupled search).
//
// Per block: the CJSO scale Delta_c (E4M3) and the E4M3 pair {lo, hi} around its unrounded value are
// given. Candidates are Delta_q = fl(Delta_c * f_k), f_k the binary32 value nearest (50+k)/100,
// k = 0..100 (quantise), times Delta_d in {lo, hi} (reconstruct): 202 candidates. The CJSO point
// (k = 50, Delta_d = Delta_c) is the incumbent; candidates are visited k = 0..100, lo before hi, and
// replace it only when their squared error is strictly smaller.
//
// Mapping: one lane per block. The block stays in registers (16 binary32 values and the 8 raw bf16
// pairs); the reciprocals 1/fl(alpha*Delta_q) of all (k, Delta_c) pairs are a 101 x 128 table in LDS
// built once per work-group (alpha is global). For each k the lane encodes 16 values with the hardware
// E2M1 converter, decodes them to bf16 pairs and forms S_wq and S_qq with v_dot2_f32_bf16 (exact, see
// block.hpp). The error of candidate (k, d) minus sum w^2 is s_d * A_d(k) with
// A_d(k) = s_d*S_qq - 2*S_wq, exact in binary64 (s_d = alpha*Delta_d exactly). For a fixed d the
// argmin over k is the argmin of A_d (s_d > 0), so the loop tracks the first minimum of A_lo and A_hi;
// the final choice compares the two minima and the incumbent exactly as double-doubles.
#include <float.h>

#include "block.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int kSoarThreads = 1024;
constexpr int kSoarK = 101;
constexpr int kTabStride = 128;

template <bool F32, bool FAST>
__device__ __forceinline__ void block_sums_k(const Blk<F32> &B, float r, bool rfin, double &sw, double &sq) {
    uint32_t c0, c1;
    if (FAST) {
        encode16(B.w, r, c0, c1);
        if constexpr (!F32) {
            float a, q;
            sums_bf16(c0, c1, B.p, a, q);
            sw = a;
            sq = q;
        }
    } else {
        if (rfin)
            encode16(B.w, r, c0, c1);
        else
            encode16_soft(B.w, r, c0, c1);
        sums_f64(c0, c1, B.w, sw, sq);
    }
}

// First minimum over k of A'_d(k) = (s_d/2)*S_qq(k) - S_wq(k) (= A_d(k)/2, exact in binary64) for
// d = lo and hi. The reciprocal of the next k is read from LDS one step ahead.
template <bool F32, bool FAST>
__device__ __forceinline__ void scan(const Blk<F32> &B, const float *__restrict__ rtab, uint32_t dc, bool rfin,
                                     double hlo, double hhi, double &best_lo, int &k_lo, double &best_hi,
                                     int &k_hi) {
    best_lo = INFINITY;
    best_hi = INFINITY;
    k_lo = 0;
    k_hi = 0;
    float r = rtab[dc];
    for (int k = 0; k < kSoarK; ++k) {
        const float rn = rtab[(k + 1 < kSoarK ? k + 1 : k) * kTabStride + dc];
        double sw = 0.0, sq = 0.0;
        block_sums_k<F32, FAST>(B, r, rfin, sw, sq);
        const double alo = fma(hlo, sq, -sw);
        const double ahi = fma(hhi, sq, -sw);
        if (alo < best_lo) {
            best_lo = alo;
            k_lo = k;
        }
        if (ahi < best_hi) {
            best_hi = ahi;
            k_hi = k;
        }
        r = rn;
    }
}

// Same minimum through packed keys: key_d(k) = A'_d(k) + C + k*u. A' lies on the lattice 2^L Z with
// |A'| < 2^M = C, and u = 2^(L-7), so every key is a non-negative multiple of u below 2^(M+2): exact in
// binary64 when M - L <= 44 (checked per block by the caller), ordered like (A', k), and the running
// minimum is one v_min_f64 per reconstruct scale.
template <bool F32>
__device__ __forceinline__ void scan_keys(const Blk<F32> &B, const float *__restrict__ rtab, uint32_t dc, double hlo,
                                          double hhi, double C, double u, double &key_lo, double &key_hi) {
    key_lo = INFINITY;
    key_hi = INFINITY;
    double kc = C;
    float r = rtab[dc];
    for (int k = 0; k < kSoarK; ++k) {
        const float rn = rtab[(k + 1 < kSoarK ? k + 1 : k) * kTabStride + dc];
        double sw = 0.0, sq = 0.0;
        block_sums_k<F32, true>(B, r, true, sw, sq);
        const double t = kc - sw;
        key_lo = fmin(key_lo, fma(hlo, sq, t));
        key_hi = fmin(key_hi, fma(hhi, sq, t));
        kc += u;
        r = rn;
    }
}

// (A', k) of a packed key (see scan_keys).
__device__ __forceinline__ void unpack_key(double key, int L, double C, double &a, int &k) {
    const double K = ldexp(key, 7 - L);
    const double kk = K - 128.0 * floor(K * (1.0 / 128.0));
    k = (int)kk;
    a = ldexp(K - kk, L - 7) - C;
}

template <bool F32>
__global__ __launch_bounds__(kSoarThreads) void k_soar(const void *__restrict__ W, int64_t nblk,
                                                       const float *__restrict__ alpha_p, uint8_t *__restrict__ codes,
                                                       uint8_t *__restrict__ scales,
                                                       const uint16_t *__restrict__ brackets) {
    __shared__ float rtab[kSoarK * kTabStride];
    const float alpha = *alpha_p;
    if (alpha != alpha) return;  // non-finite input: outputs already zero
    // reciprocal table: r = fl(1/s), s = fl(alpha * fl(Delta_c * f_k)); a zero scale quantises to 0
    for (int i = threadIdx.x; i < kSoarK * kTabStride; i += blockDim.x) {
        const int k = i / kTabStride, c = i % kTabStride;
        float r = 0.0f;
        if (c < 0x7F) {
            const float f = (float)((double)(50 + k) / 100.0);
            const float s = alpha * (e4m3_value((uint32_t)c) * f);
            r = s == 0.0f ? 0.0f : 1.0f / s;
        }
        rtab[i] = r;
    }
    __syncthreads();

    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblk) return;
    const uint32_t dc = scales[b];
    if (dc == 0u) return;  // Delta_c = 0: every candidate quantises to 0 and ties; codes and scale stay 0
    const uint32_t br = brackets[b];
    const uint32_t lo = br & 0xFFu, hi = br >> 8;
    Blk<F32> B;
    B.load(W, b);
    const float a = B.amax();
    const float r0 = rtab[dc];
    const bool rfin = finite_pos(r0);  // s grows with k, so r_0 bounds every reciprocal
    const float smin = alpha * (e4m3_value(dc) * 0.5f);
    // s_d = alpha * Delta_d exactly; errors are compared through s_d * A'_d with A'_d = A_d / 2
    const double slo = (double)alpha * (double)e4m3_value(lo);
    const double shi = (double)alpha * (double)e4m3_value(hi);
    const double hlo = 0.5 * slo, hhi = 0.5 * shi;
    const bool c_is_lo = dc == lo;
    double best_lo, best_hi, a_c, sw50, sq50;
    int k_lo, k_hi;
    if constexpr (!F32) {
        // lattice 2^L and bound 2^M of A' = h*S_qq - S_wq (see block.hpp and scan_keys)
        const int L = min(ilogb(hlo) - 29, ilogbf(smin) - 11);
        const int M = max(ilogb(hhi) + 11, ilogbf(a) + 8);
        const bool fast = rfin && a <= 32.0f * smin && a <= 0x1p100f;
        if (fast && hlo > 0.0 && smin > 0.0f && M - L <= 44) {
            const double C = ldexp(1.0, M), u = ldexp(1.0, L - 7);
            double key_lo, key_hi;
            scan_keys<F32>(B, rtab, dc, hlo, hhi, C, u, key_lo, key_hi);
            unpack_key(key_lo, L, C, best_lo, k_lo);
            unpack_key(key_hi, L, C, best_hi, k_hi);
            block_sums_k<F32, true>(B, rtab[50 * kTabStride + dc], rfin, sw50, sq50);
        } else if (fast) {
            scan<F32, true>(B, rtab, dc, rfin, hlo, hhi, best_lo, k_lo, best_hi, k_hi);
            block_sums_k<F32, true>(B, rtab[50 * kTabStride + dc], rfin, sw50, sq50);
        } else {
            scan<F32, false>(B, rtab, dc, rfin, hlo, hhi, best_lo, k_lo, best_hi, k_hi);
            block_sums_k<F32, false>(B, rtab[50 * kTabStride + dc], rfin, sw50, sq50);
        }
    } else {
        scan<F32, false>(B, rtab, dc, rfin, hlo, hhi, best_lo, k_lo, best_hi, k_hi);
        block_sums_k<F32, false>(B, rtab[50 * kTabStride + dc], rfin, sw50, sq50);
    }
    // the incumbent: Delta_q = Delta_c * f_50 = Delta_c, Delta_d = Delta_c
    a_c = fma(c_is_lo ? hlo : hhi, sq50, -sw50);
    // a zero reconstruction scale makes every candidate's error sum w^2: the first one (k = 0) stands
    if (slo == 0.0) {
        best_lo = 0.0;
        k_lo = 0;
    }
    if (shi == 0.0) {
        best_hi = 0.0;
        k_hi = 0;
    }
    const dd jc = two_prod(c_is_lo ? slo : shi, a_c);
    const dd jlo = two_prod(slo, best_lo);
    const dd jhi = two_prod(shi, best_hi);
    const dd jmin = dd_less(jhi, jlo) ? jhi : jlo;
    int kb;
    uint32_t db;
    if (dd_equal(jc, jmin)) {
        kb = 50;
        db = dc;
    } else if (dd_less(jlo, jhi)) {
        kb = k_lo;
        db = lo;
    } else if (dd_less(jhi, jlo)) {
        kb = k_hi;
        db = hi;
    } else if (k_lo <= k_hi) {
        kb = k_lo;
        db = lo;
    } else {
        kb = k_hi;
        db = hi;
    }
    const float r = rtab[kb * kTabStride + dc];
    uint32_t c0, c1;
    if (rfin)
        encode16(B.w, r, c0, c1);
    else
        encode16_soft(B.w, r, c0, c1);
    *reinterpret_cast<uint2 *>(codes + 8 * b) = make_uint2(e2m1_clear_negzero(c0), e2m1_clear_negzero(c1));
    scales[b] = (uint8_t)db;
}

hipError_t launch_soar(const void *W, bool f32, int64_t nblk, const float *alpha, uint8_t *codes, uint8_t *scales,
                       const uint16_t *brackets, hipStream_t stream) {
    const dim3 grid((unsigned)((nblk + kSoarThreads - 1) / kSoarThreads)), block(kSoarThreads);
    if (f32)
        hipLaunchKernelGGL(k_soar<true>, grid, block, 0, stream, W, nblk, alpha, codes, scales, brackets);
    else
        hipLaunchKernelGGL(k_soar<false>, grid, block, 0, stream, W, nblk, alpha, codes, scales, brackets);
    return hipGetLastError();
}

}  // namespace nvfp4
