// gfx950 kernel for the decoupled quantise/dequantise block-scale search of the SOAR page ("SOAR:
// Scale Optimization for Accurate Reconstruction in NVFP4 Quantization", decoupled search).
//
// Per block: the CJSO scale Delta_c (E4M3) and the E4M3 pair {lo, hi} around its unrounded value are
// given. Candidates are Delta_q = fl(Delta_c * f_k), f_k the binary32 value nearest (50+k)/100,
// k = 0..100 (quantise), times Delta_d in {lo, hi} (reconstruct): 202 candidates. The CJSO point
// (k = 50, Delta_d = Delta_c) is the incumbent; candidates are visited k = 0..100, lo before hi, and
// replace it only when their squared error is strictly smaller.
//
// Error of candidate (k, d): sum w^2 + 2 s_d A_d(k), A_d(k) = (s_d/2) S_qq(k) - S_wq(k), with
// s_d = alpha * Delta_d and S_qq, S_wq the sums of q^2 and |w| q over the block's code magnitudes q at
// quantisation scale s_k = fl(alpha * Delta_q(k)).
//
// Exact search on a window. A_d(k) = sum_j psi_j(q_j(k)) with psi_j(m) = (s_d/2) m^2 - |w_j| m, a convex
// function of m whose minimisers over the E2M1 grid are the grid points nearest |w_j| / s_d. Each
// magnitude q_j(k) is non-increasing in k (s_k grows with k, so fl(w_j * fl(1/s_k)) shrinks, and E2M1
// rounding is monotone). Hence, for every j:
//   * while s_k < s_d (1 - 2^-20) the computed |x_j| = fl(|w_j| / s_k) exceeds |w_j| / s_d, so q_j(k)
//     is at or above every nearest grid point and psi_j(q_j(k)) does not increase with k;
//   * while s_k > s_d (1 + 2^-20) q_j(k) is at or below every nearest grid point and psi_j(q_j(k))
//     does not decrease with k.
// (The margin covers the two binary32 roundings of r = fl(1/s_k) and x = fl(w r), 2^-24 each.) With
// K1 the last k of the first kind and K2 the first of the second, A_d does not increase on [0, K1]
// and does not decrease on [K2, 100], so its minimum lies in [K1, K2], which holds two or three k
// (s_k moves by about 1 % per step). The first minimiser in k order is the window's first minimiser,
// unless that is K1 itself: then every k < K1 with A_d(k) = A_d(K1) has exactly the same codes (a
// larger magnitude strictly raises psi_j there), so it only matters when the two reconstruct scales
// tie exactly, and that rare case walks down to the first k with the codes of K1.
// The full 101-step scan remains for blocks outside the exactness window of the binary32 sums or of
// binary64 A_d, and for fp32 input.
#include <float.h>

#include "block.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int kSoarThreads = 256;
constexpr int kSoarK = 101;

// s_k = fl(alpha * fl(Delta_c * f_k)) and its reciprocal (0 for a zero scale: every code is then 0).
__device__ __forceinline__ float quant_scale(float alpha, float vc, const float *ftab, int k) {
    return alpha * (vc * ftab[k]);
}
__device__ __forceinline__ float recip(float s) { return s == 0.0f ? 0.0f : 1.0f / s; }

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

// Full scan: first minimum over k of A_d(k) for d = lo and hi.
template <bool F32, bool FAST>
__device__ __forceinline__ void scan(const Blk<F32> &B, const float *__restrict__ ftab, float alpha, float vc,
                                     bool rfin, double hlo, double hhi, double &best_lo, int &k_lo, double &best_hi,
                                     int &k_hi) {
    best_lo = INFINITY;
    best_hi = INFINITY;
    k_lo = 0;
    k_hi = 0;
    for (int k = 0; k < kSoarK; ++k) {
        double sw = 0.0, sq = 0.0;
        block_sums_k<F32, FAST>(B, recip(quant_scale(alpha, vc, ftab, k)), rfin, sw, sq);
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
    }
}

// A_d at quantisation scale index k (bf16 block inside the exactness window), with its codes.
__device__ __forceinline__ double eval_k(const Blk<false> &B, float alpha, float vc, const float *ftab, int k,
                                         double h, uint32_t &c0, uint32_t &c1) {
    encode16(B.w, 1.0f / quant_scale(alpha, vc, ftab, k), c0, c1);
    float sw, sq;
    sums_bf16(c0, c1, B.p, sw, sq);
    return fma(h, (double)sq, -(double)sw);
}

// The window [kA, kB] for reconstruct scale s_d (exact in binary64): kA = max(K1, 0), kB = min(K2, 100)
// with K1 the last k with s_d > s_k (1 + 2^-20) (-1 if none) and K2 the first k with
// s_d < s_k (1 - 2^-20) (101 if none). Both products are exact in binary64. The search starts from the
// k where s_k would equal s_d and walks to the exact bounds.
__device__ __forceinline__ void window(float alpha, float vc, float vd, double sd, const float *ftab, int &kA,
                                       int &kB) {
    const double up = 1.0 + 0x1p-20, dn = 1.0 - 0x1p-20;
    auto below = [&](int k) { return sd > (double)quant_scale(alpha, vc, ftab, k) * up; };
    auto above = [&](int k) { return sd < (double)quant_scale(alpha, vc, ftab, k) * dn; };
    int k1 = (int)floorf(100.0f * (vd * __builtin_amdgcn_rcpf(vc))) - 50;
    k1 = k1 < -1 ? -1 : (k1 > 100 ? 100 : k1);
    while (k1 < 100 && below(k1 + 1)) ++k1;
    while (k1 >= 0 && !below(k1)) --k1;
    int k2 = k1 + 1;
    while (k2 <= 100 && !above(k2)) ++k2;
    kA = k1 > 0 ? k1 : 0;
    kB = k2 < 100 ? k2 : 100;
}

// First k <= kA whose codes equal those at kA (the start of A_d's plateau ending at kA).
__device__ __forceinline__ int plateau_start(const Blk<false> &B, float alpha, float vc, const float *ftab, int kA,
                                             uint32_t c0, uint32_t c1) {
    int k = kA;
    while (k > 0) {
        uint32_t d0, d1;
        encode16(B.w, 1.0f / quant_scale(alpha, vc, ftab, k - 1), d0, d1);
        if (d0 != c0 || d1 != c1) break;
        --k;
    }
    return k;
}

struct Pick {
    double a;     // min A_d over the window
    int k;        // its first minimiser in the window
    int kA;       // the window's first k
    uint32_t c0, c1;
};

template <bool F32>
__global__ __launch_bounds__(kSoarThreads) void k_soar(const void *__restrict__ W, int64_t nblk,
                                                       const float *__restrict__ alpha_p, uint8_t *__restrict__ codes,
                                                       uint8_t *__restrict__ scales,
                                                       const uint16_t *__restrict__ brackets, bool full_search) {
    __shared__ float ftab[kSoarK];
    const float alpha = *alpha_p;
    if (alpha != alpha) return;  // non-finite input: outputs already zero
    if (threadIdx.x < kSoarK) ftab[threadIdx.x] = (float)((double)(50 + threadIdx.x) / 100.0);
    __syncthreads();

    const int64_t b = (int64_t)blockIdx.x * kSoarThreads + threadIdx.x;
    if (b >= nblk) return;
    const uint32_t dc = scales[b];
    if (dc == 0u) return;  // Delta_c = 0: every candidate quantises to 0 and ties; codes and scale stay 0
    const uint32_t br = brackets[b];
    const uint32_t lo = br & 0xFFu, hi = br >> 8;
    Blk<F32> B;
    B.load(W, b);
    const float a = B.amax();
    const float vc = e4m3_value(dc);
    const float r0 = recip(quant_scale(alpha, vc, ftab, 0));
    const bool rfin = finite_pos(r0);  // s grows with k, so r_0 bounds every reciprocal
    const float smin = quant_scale(alpha, vc, ftab, 0);
    // s_d = alpha * Delta_d exactly; errors are compared through s_d * A_d
    const float vlo = e4m3_value(lo), vhi = e4m3_value(hi);
    const double slo = (double)alpha * (double)vlo;
    const double shi = (double)alpha * (double)vhi;
    const double hlo = 0.5 * slo, hhi = 0.5 * shi;
    const bool c_is_lo = dc == lo;
    double best_lo, best_hi, a_c;
    int k_lo, k_hi;
    uint32_t c0, c1;  // codes of the chosen candidate
    int kb;
    uint32_t db;

    bool windowed = false;
    if constexpr (!F32) {
        // A_d lies on the lattice 2^L with |A_d| < 2^M (see block.hpp): exact in binary64 when M - L <= 53
        const int L = min(ilogb(hlo) - 29, ilogbf(smin) - 11);
        const int M = max(ilogb(hhi) + 11, ilogbf(a) + 8);
        windowed = !full_search && rfin && a <= 32.0f * smin && a <= 0x1p100f && hlo > 0.0 && smin > 0.0f &&
                   M - L <= 53;
    }
    if constexpr (!F32) {
        if (windowed) {
            // own window (d = Delta_c) always holds k = 50, the incumbent; the other scale's window is
            // evaluated in full
            const double sd_c = c_is_lo ? slo : shi, h_c = c_is_lo ? hlo : hhi;
            const float vo = c_is_lo ? vhi : vlo;
            const double sd_o = c_is_lo ? shi : slo, h_o = c_is_lo ? hhi : hlo;
            uint32_t i0, i1;
            a_c = eval_k(B, alpha, vc, ftab, 50, h_c, i0, i1);
            Pick pc, po;
            int kA, kB;
            window(alpha, vc, vc, sd_c, ftab, kA, kB);
            pc.a = a_c;
            pc.k = 50;
            pc.kA = kA;
            pc.c0 = i0;
            pc.c1 = i1;
            for (int k = kA; k <= kB; ++k) {
                if (k == 50) continue;
                uint32_t d0, d1;
                const double v = eval_k(B, alpha, vc, ftab, k, h_c, d0, d1);
                if (v < pc.a || (v == pc.a && k < pc.k)) {
                    pc.a = v;
                    pc.k = k;
                    pc.c0 = d0;
                    pc.c1 = d1;
                }
            }
            window(alpha, vc, vo, sd_o, ftab, kA, kB);
            po.a = INFINITY;
            po.k = kA;
            po.kA = kA;
            po.c0 = po.c1 = 0u;
            for (int k = kA; k <= kB; ++k) {
                uint32_t d0, d1;
                const double v = eval_k(B, alpha, vc, ftab, k, h_o, d0, d1);
                if (v < po.a) {
                    po.a = v;
                    po.k = k;
                    po.c0 = d0;
                    po.c1 = d1;
                }
            }
            const Pick &pl = c_is_lo ? pc : po;
            const Pick &ph = c_is_lo ? po : pc;
            const dd jc = two_prod(sd_c, a_c);
            const dd jlo = two_prod(slo, pl.a);
            const dd jhi = two_prod(shi, ph.a);
            const dd jmin = dd_less(jhi, jlo) ? jhi : jlo;
            if (dd_equal(jc, jmin)) {
                db = dc;
                c0 = i0;
                c1 = i1;
            } else if (dd_less(jlo, jhi)) {
                db = lo;
                c0 = pl.c0;
                c1 = pl.c1;
            } else if (dd_less(jhi, jlo)) {
                db = hi;
                c0 = ph.c0;
                c1 = ph.c1;
            } else {
                // equal errors: the earlier first minimiser wins, lo on equal k
                const int kl = pl.k == pl.kA ? plateau_start(B, alpha, vc, ftab, pl.kA, pl.c0, pl.c1) : pl.k;
                const int kh = ph.k == ph.kA ? plateau_start(B, alpha, vc, ftab, ph.kA, ph.c0, ph.c1) : ph.k;
                const bool take_lo = kl <= kh;
                db = take_lo ? lo : hi;
                c0 = take_lo ? pl.c0 : ph.c0;
                c1 = take_lo ? pl.c1 : ph.c1;
            }
            *reinterpret_cast<uint2 *>(codes + 8 * b) =
                make_uint2(e2m1_clear_negzero(c0), e2m1_clear_negzero(c1));
            scales[b] = (uint8_t)db;
            return;
        }
    }

    // full scan
    double sw50, sq50;
    const float r50 = recip(quant_scale(alpha, vc, ftab, 50));
    const bool fast = !F32 && rfin && a <= 32.0f * smin && a <= 0x1p100f;
    if (fast) {
        scan<F32, true>(B, ftab, alpha, vc, rfin, hlo, hhi, best_lo, k_lo, best_hi, k_hi);
        block_sums_k<F32, true>(B, r50, rfin, sw50, sq50);
    } else {
        scan<F32, false>(B, ftab, alpha, vc, rfin, hlo, hhi, best_lo, k_lo, best_hi, k_hi);
        block_sums_k<F32, false>(B, r50, rfin, sw50, sq50);
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
    const float r = recip(quant_scale(alpha, vc, ftab, kb));
    if (rfin)
        encode16(B.w, r, c0, c1);
    else
        encode16_soft(B.w, r, c0, c1);
    *reinterpret_cast<uint2 *>(codes + 8 * b) = make_uint2(e2m1_clear_negzero(c0), e2m1_clear_negzero(c1));
    scales[b] = (uint8_t)db;
}

hipError_t launch_soar(const void *W, bool f32, int64_t nblk, const float *alpha, uint8_t *codes, uint8_t *scales,
                       const uint16_t *brackets, bool full_search, hipStream_t stream) {
    const dim3 grid((unsigned)((nblk + kSoarThreads - 1) / kSoarThreads)), block(kSoarThreads);
    if (f32)
        hipLaunchKernelGGL(k_soar<true>, grid, block, 0, stream, W, nblk, alpha, codes, scales, brackets,
                           full_search);
    else
        hipLaunchKernelGGL(k_soar<false>, grid, block, 0, stream, W, nblk, alpha, codes, scales, brackets,
                           full_search);
    return hipGetLastError();
}

}  // namespace nvfp4
