// gfx950 kernels for the global max, the max rule, FourOverSix, the CJSO rounds, E2M1 encoding and
// dequantisation. All are bandwidth-bound passes over W: one lane owns one 16-element block (two 16-byte
// loads for bf16), so the block max, the candidate codes and the block sums never leave registers.
//
// Device-wide dependencies (alpha needs all of W; each CJSO round needs the previous round's
// least-squares sums) are kernel boundaries. Each producer writes one small partial per work-group and
// every work-group of the consumer reduces those partials in a fixed order, so results are
// deterministic and no atomics, counters or memsets are needed.
#include <float.h>

#include "block.hpp"
#include "launch.hpp"

namespace nvfp4 {

// ------------------------------------------------------------------------------- reductions

// Wave-wide reductions on the VALU through DPP (no LDS round trips): swaps within quads (xor 1, xor 2),
// the half-row and row mirrors (which pair the two quads of each half-row, then the two half-rows of
// each row), then the row broadcasts of lane 15 to rows 1 and 3 and of lane 31 to rows 2 and 3. Rows
// left out by a step's row mask receive `old` = 0, the identity, so lane 63 ends with the total.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint64_t lo = dpp_u32<CTRL, ROWS>((uint32_t)u), hi = dpp_u32<CTRL, ROWS>((uint32_t)(u >> 32));
    return __longlong_as_double((long long)((hi << 32) | lo));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140,
              kDppBcast15 = 0x142, kDppBcast31 = 0x143;

template <int CTRL, int ROWS>
__device__ __forceinline__ void dd2_step(dd &N, dd &D) {
    const dd n2 = {dpp_f64<CTRL, ROWS>(N.hi), dpp_f64<CTRL, ROWS>(N.lo)};
    const dd d2 = {dpp_f64<CTRL, ROWS>(D.hi), dpp_f64<CTRL, ROWS>(D.lo)};
    N = dd_add(N, n2);
    D = dd_add(D, d2);
}

// Sum of two double-doubles over the wave (fixed order); valid in lane 63.
__device__ __forceinline__ void wave_sum_dd2(dd &N, dd &D) {
    dd2_step<kDppXor1, 0xF>(N, D);
    dd2_step<kDppXor2, 0xF>(N, D);
    dd2_step<kDppHalfMirror, 0xF>(N, D);
    dd2_step<kDppMirror, 0xF>(N, D);
    dd2_step<kDppBcast15, 0xA>(N, D);
    dd2_step<kDppBcast31, 0xC>(N, D);
}

// Max over the wave; valid in lane 63.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
    uint32_t t;
    t = dpp_u32<kDppXor1, 0xF>(m); m = t > m ? t : m;
    t = dpp_u32<kDppXor2, 0xF>(m); m = t > m ? t : m;
    t = dpp_u32<kDppHalfMirror, 0xF>(m); m = t > m ? t : m;
    t = dpp_u32<kDppMirror, 0xF>(m); m = t > m ? t : m;
    t = dpp_u32<kDppBcast15, 0xA>(m); m = t > m ? t : m;
    t = dpp_u32<kDppBcast31, 0xC>(m); m = t > m ? t : m;
    return m;
}

// Max over the work-group (T threads) of one value per thread; every thread gets the result.
template <int T>
__device__ __forceinline__ uint32_t wg_max(uint32_t m) {
    __shared__ uint32_t red[T / 64];
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 63) red[threadIdx.x >> 6] = m;
    lds_barrier();
    m = 0u;
#pragma unroll
    for (int i = 0; i < T / 64; ++i) m = red[i] > m ? red[i] : m;
    return m;
}

// Work-group sum (T threads) of two double-doubles in a fixed order, over the values of the first TA
// threads (a multiple of 64; the other threads only take part in the barriers). The result is valid
// in thread kSumLane. Schemes for combining the waves (NVFP4_WG_SUM): 0, waves 1.. hand their lanes'
// values to wave 0 through LDS and wave 0 adds them lane by lane; 1, every wave reduces its own lanes
// and wave 0 reduces their totals; 2, a tree across waves through LDS (the upper half of the remaining
// waves hands its values to the lower half, once per level). Wave 0 then reduces across its lanes.
constexpr int kSumLane = 63;
template <int T, int TA = T>
__device__ __forceinline__ void wg_sum_dd2(dd &N, dd &D) {
    constexpr int NW = TA / 64;
    static_assert(T % 64 == 0 && TA % 64 == 0 && NW >= 1 && TA <= T, "whole waves");
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    if constexpr (NW > 1 && NVFP4_WG_SUM == 1) {
        __shared__ double tot[4][NW];  // [N.hi, N.lo, D.hi, D.lo][wave]
        if (w < NW) {
            wave_sum_dd2(N, D);
            if (l == 63) {
                tot[0][w] = N.hi;
                tot[1][w] = N.lo;
                tot[2][w] = D.hi;
                tot[3][w] = D.lo;
            }
        }
        lds_barrier();
        if (w == 0) {
            N = l < NW ? dd{tot[0][l], tot[1][l]} : dd{0.0, 0.0};
            D = l < NW ? dd{tot[2][l], tot[3][l]} : dd{0.0, 0.0};
            wave_sum_dd2(N, D);
        }
        return;
    } else if constexpr (NW > 1 && NVFP4_WG_SUM == 2) {
        static_assert((NW & (NW - 1)) == 0, "a power of two of waves");
        __shared__ double buf[NW - 1][4][64];  // level with h waves receiving: rows h - 1 .. 2h - 2
#pragma unroll
        for (int h = NW / 2; h >= 1; h >>= 1) {
            if (w >= h && w < 2 * h) {
                double *r = &buf[h - 1 + (w - h)][0][0];
                r[l] = N.hi;
                r[64 + l] = N.lo;
                r[128 + l] = D.hi;
                r[192 + l] = D.lo;
            }
            lds_barrier();
            if (w < h) {
                const double *r = &buf[h - 1 + w][0][0];
                N = dd_add(N, dd{r[l], r[64 + l]});
                D = dd_add(D, dd{r[128 + l], r[192 + l]});
            }
        }
    } else if constexpr (NW > 1) {
        __shared__ double buf[NW - 1][4][64];  // [wave - 1][N.hi, N.lo, D.hi, D.lo][lane]
        if (w > 0 && w < NW) {
            buf[w - 1][0][l] = N.hi;
            buf[w - 1][1][l] = N.lo;
            buf[w - 1][2][l] = D.hi;
            buf[w - 1][3][l] = D.lo;
        }
        lds_barrier();
        if (w == 0) {
#pragma unroll
            for (int i = 0; i < NW - 1; ++i) {
                N = dd_add(N, dd{buf[i][0][l], buf[i][1][l]});
                D = dd_add(D, dd{buf[i][2][l], buf[i][3][l]});
            }
        }
    }
    if (w == 0) wave_sum_dd2(N, D);
}

// A kernel's prologue reads the previous kernel's per-work-group partials. Each thread loads its share
// first (before the block prefetch, so that waiting for these loads does not wait for the prefetch)
// and reduces it afterwards. T = threads of the reading kernel, G = most partials.
template <int T>
struct AmaxShare {
    static constexpr int K = (kAmaxMaxGroups + T - 1) / T;
    uint32_t v[K];
    __device__ __forceinline__ void load(const uint32_t *part, int n) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int i = (int)threadIdx.x + k * T;
            v[k] = i < n ? part[i] : 0u;
        }
    }
    // max of part[0..n) over the work-group (every thread gets it)
    __device__ __forceinline__ uint32_t reduce() const {
        uint32_t m = 0u;
#pragma unroll
        for (int k = 0; k < K; ++k) m = v[k] > m ? v[k] : m;
        return wg_max<T>(m);
    }
};

template <int T, int G>
struct CjsoShare {
    static constexpr int K = (G + T - 1) / T;
    double v[K][4];
    __device__ __forceinline__ void load(const double *part, int n) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int i = (int)threadIdx.x + k * T;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[k][j] = i < n ? part[4 * i + j] : 0.0;
        }
    }
    // sum of the partials (fixed order); every thread gets it
    __device__ __forceinline__ void reduce(dd &N, dd &D) const {
        __shared__ double tot[4];
        N = {0.0, 0.0};
        D = {0.0, 0.0};
#pragma unroll
        for (int k = 0; k < K; ++k) {
            N = dd_add(N, dd{v[k][0], v[k][1]});
            D = dd_add(D, dd{v[k][2], v[k][3]});
        }
        // only the first min(T, G) threads hold partials
        wg_sum_dd2<T, (G < T ? (G + 63) / 64 * 64 : T)>(N, D);
        if (threadIdx.x == kSumLane) {
            tot[0] = N.hi;
            tot[1] = N.lo;
            tot[2] = D.hi;
            tot[3] = D.lo;
        }
        lds_barrier();
        N = {tot[0], tot[1]};
        D = {tot[2], tot[3]};
    }
};

// SOAR page, global-scale step: alpha* = N / D (the least-squares minimiser over alpha), rounded once
// to binary32. D = 0 (every code zero) keeps the previous alpha.
__device__ __forceinline__ float alpha_from(dd N, dd D, float prev) {
    if (!(D.hi > 0.0)) return prev;
    double q = N.hi / D.hi;
    const double rem = fma(-q, D.hi, N.hi) + N.lo - q * D.lo;
    q = q + rem / D.hi;
    return (float)q;
}

// SOAR page, max rule: alpha = max|W| / (M_FP4 * M_FP8) = max|W| / 2688, binary32.
__device__ __forceinline__ float max_rule_alpha(uint32_t amax_bits) { return __uint_as_float(amax_bits) / 2688.0f; }

// SOAR page, max rule: the argument max|W_i| / (alpha * M_FP4) of the block scale, in binary64 (both
// operands carry at most 26 significant bits, so its E4M3 rounding is that of the real quotient).
__device__ __forceinline__ double max_rule_quotient(float a, float alpha) {
    return a == 0.0f ? 0.0 : (double)a / (6.0 * (double)alpha);
}

__device__ __forceinline__ void store_codes(uint8_t *codes, int64_t b, uint32_t c0, uint32_t c1) {
    *reinterpret_cast<uint2 *>(codes + 8 * b) = make_uint2(e2m1_clear_negzero(c0), e2m1_clear_negzero(c1));
}

// Visit this thread's blocks b = gid, gid + S, gid + 2S, ... (S = all T * gridDim threads), in that order
// or, with `reverse`, from the last one down, through a ring of DEPTH blocks in registers: the loads of
// block i + DEPTH are issued as soon as block i has been unpacked, so DEPTH blocks are in flight while one
// is processed (a prefetch past the thread's last block re-reads its first one, a cached read). The ring is
// unrolled, so no register copy waits on a load. `pre` issues the prologue's own loads, then the first DEPTH
// blocks are requested, then `post` (run by every thread of the work-group) finishes the prologue; it
// returns false to skip the blocks (the function then returns false). f(b, B, sc) gets the block and, when
// `sc_in` is given, its scale byte.
//
// A work-group runs on the XCD blockIdx.x % 8, and every pass over W with the same grid hands the same
// blocks to the same work-group, so a pass that visits them in the opposite order to the pass before it
// starts on the blocks that pass read last, which its XCD's L2 still holds.
template <int T, int DEPTH, bool F32, class Pre, class Post, class F>
__device__ __forceinline__ bool for_my_blocks(const void *__restrict__ W, const uint8_t *__restrict__ sc_in,
                                              int64_t nblk, bool reverse, Pre &&pre, Post &&post, F &&f) {
    constexpr int D = DEPTH;
    const int64_t stride = (int64_t)gridDim.x * T;
    const int64_t first = (int64_t)blockIdx.x * T + threadIdx.x;
    const int64_t n = first < nblk ? (nblk - 1 - first) / stride + 1 : 0;  // blocks of this thread
    const int64_t start = reverse && n > 0 ? first + (n - 1) * stride : first;
    const int64_t step = reverse ? -stride : stride;
    const int64_t safe = n > 0 ? start : nblk - 1;  // a valid block to prefetch past the end
    Raw<F32> r[D];
    uint32_t sc[D];
    pre();
#pragma unroll
    for (int k = 0; k < D; ++k) {
        const int64_t c = k < n ? start + k * step : safe;
        r[k].load(W, c);
        sc[k] = sc_in ? (uint32_t)sc_in[c] : 0u;
    }
    if (!post()) return false;
    int64_t b = start;
    for (int64_t i = 0; i < n;) {
#pragma unroll
        for (int k = 0; k < D; ++k) {
            Blk<F32> B;
            B.set(r[k]);
            const uint32_t s = sc[k];
            const int64_t c = i + D < n ? b + D * step : safe;
            r[k].load(W, c);
            if (sc_in) sc[k] = sc_in[c];
            f(b, B, s);
            b += step;
            if (++i >= n) return true;
        }
    }
    return true;
}

// The same visit, two blocks at a time: f2(b, A, da, b', B, db) gets two consecutive blocks of this thread
// (b' = b + S, or b - S with `reverse`) and their scale bytes (0 without `sc_in`), so that their independent
// arithmetic can be interleaved; an odd last block goes to f1(b, A, da). The next pair's loads are issued
// before a pair is processed.
template <int T, bool F32, class Pre, class Post, class F2, class F1>
__device__ __forceinline__ bool for_my_pairs(const void *__restrict__ W, const uint8_t *__restrict__ sc_in,
                                             int64_t nblk, bool reverse, Pre &&pre, Post &&post, F2 &&f2, F1 &&f1) {
    const int64_t stride = (int64_t)gridDim.x * T;
    const int64_t first = (int64_t)blockIdx.x * T + threadIdx.x;
    const int64_t n = first < nblk ? (nblk - 1 - first) / stride + 1 : 0;  // blocks of this thread
    const int64_t start = reverse && n > 0 ? first + (n - 1) * stride : first;
    const int64_t step = reverse ? -stride : stride;
    const int64_t safe = n > 0 ? start : nblk - 1;  // a valid block to prefetch past the end
    Raw<F32> r0, r1;
    uint32_t s0 = 0u, s1 = 0u;
    pre();
    {
        const int64_t c0 = safe, c1 = n > 1 ? start + step : safe;
        r0.load(W, c0);
        r1.load(W, c1);
        if (sc_in) {
            s0 = sc_in[c0];
            s1 = sc_in[c1];
        }
    }
    if (!post()) return false;
    int64_t b = start, i = 0;
    for (; i + 1 < n; i += 2) {
        Blk<F32> A, B;
        A.set(r0);
        B.set(r1);
        const uint32_t da = s0, db = s1;
        const int64_t c0 = i + 2 < n ? b + 2 * step : safe, c1 = i + 3 < n ? b + 3 * step : safe;
        r0.load(W, c0);
        r1.load(W, c1);
        if (sc_in) {
            s0 = sc_in[c0];
            s1 = sc_in[c1];
        }
        f2(b, A, da, b + step, B, db);
        b += 2 * step;
    }
    if (i < n) {
        Blk<F32> A;
        A.set(r0);
        f1(b, A, s0);
    }
    return true;
}

// ---------------------------------------------------------------------------------- global max

// Per work-group max of |w| as binary32 bits (bf16 bits are widened), plus the non-finite test
// (any NaN or infinity makes the max >= 0x7F800000). Zeroes the stats for this call. The work-groups
// and threads are laid out exactly as in the pass that consumes the max (T threads, the same grid, thread
// b of the grid visiting blocks b, b + S, ...), so each block is read twice by the same work-group on
// the same XCD; the consumer visits its blocks in the opposite order and starts on those still in L2.
template <bool F32, int T>
__global__ __launch_bounds__(T) void k_amax(const void *__restrict__ W, int64_t nblk, uint32_t *__restrict__ part,
                                            nvfp4_stats_t *stats) {
    constexpr int U = 4;  // blocks in flight per thread
    constexpr int NV = F32 ? 4 : 2;
    uint32_t m = 0u;
    auto fold = [&](const Raw<F32> &r) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const uint32_t d[4] = {r.v[v].x, r.v[v].y, r.v[v].z, r.v[v].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (F32) {
                    const uint32_t a = d[k] & 0x7FFFFFFFu;
                    m = a > m ? a : m;
                } else {
                    const uint32_t lo = (d[k] & 0x7FFFu) << 16, hi = d[k] & 0x7FFF0000u;
                    m = lo > m ? lo : m;
                    m = hi > m ? hi : m;
                }
            }
        }
    };
    const int64_t stride = (int64_t)gridDim.x * T;
    int64_t b = (int64_t)blockIdx.x * T + threadIdx.x;
    for (; b + (U - 1) * stride < nblk; b += U * stride) {
        Raw<F32> r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) r[u].load(W, b + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) fold(r[u]);
    }
    for (; b < nblk; b += stride) {
        Raw<F32> r;
        r.load(W, b);
        fold(r);
    }
    __shared__ uint32_t red[T / 64];
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 63) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = red[0];
        for (int k = 1; k < T / 64; ++k) m = red[k] > m ? red[k] : m;
        part[blockIdx.x] = m;
        if (blockIdx.x == 0 && stats) {
            stats->status = 0u;
            stats->m4_blocks = 0u;
        }
    }
}

// ------------------------------------------------------------------------- MAX and FourOverSix

// FourOverSix write-up, section 02, for one block under alpha: scale_m4 = fp8(scale_m6 * 1.5); M=4 is
// kept iff its squared error is strictly smaller. With S_wq, S_qq exact and s_d = alpha*Delta exact in
// binary64, the error minus sum w^2 is s_d*(s_d*S_qq - 2*S_wq): the inner term is exact in binary64 and
// the product is held exactly as a double-double. In: d6 (the max-rule scale). Out: the chosen scale d,
// its codes and sums; returns whether M=4 was taken.
template <bool F32>
__device__ __forceinline__ bool fos_choice(const Blk<F32> &B, float a, const ScaleTab &T, float alpha, uint32_t d6,
                                           uint32_t &d, uint32_t &c0, uint32_t &c1, double &sw, double &sq) {
    const float v6 = e4m3_value(d6);
    double w6, q6, w4, q4;
    uint32_t e0, e1;
    quant_sums_r(B, a, T.s[d6], T.r[d6], c0, c1, w6, q6);
    const uint32_t d4 = e4m3_rne(1.5 * (double)v6);
    const float v4 = e4m3_value(d4);
    quant_sums_r(B, a, T.s[d4], T.r[d4], e0, e1, w4, q4);
    const double sd6 = (double)alpha * (double)v6, sd4 = (double)alpha * (double)v4;
    const dd j6 = two_prod(sd6, fma(sd6, q6, -2.0 * w6));
    const dd j4 = two_prod(sd4, fma(sd4, q4, -2.0 * w4));
    const bool m4 = dd_less(j4, j6);
    d = m4 ? d4 : d6;
    sw = m4 ? w4 : w6;
    sq = m4 ? q4 : q6;
    if (m4) {
        c0 = e0;
        c1 = e1;
    }
    return m4;
}

// The max rule's code E4M3(max|w| / (6 alpha)) of a block (six_alpha = fl(6 alpha)): decided by the binary32
// estimate where it can be, else by the binary64 quotient. Returns whether the estimate decided it; the
// caller then skips the binary64 form (kept out of this function so that two blocks' estimates stay side by
// side).
__device__ __forceinline__ bool max_rule_est(float a, float six_alpha, uint32_t &d) {
    return e4m3_quotient_est(a, six_alpha, d);
}

// One candidate scale of a bf16 block: its codes and exact sums.
struct Cand {
    uint32_t c0, c1;
    double sw, sq;
};

// The common case of quant_sums_r for a bf16 block: hardware codes for the reciprocal r of s and the
// binary32 sums. Returns whether those sums are exact (quant_sums_r's own test); when not, the caller
// redoes the candidate with quant_sums_r.
__device__ __forceinline__ bool cand_fast(const Blk<false> &B, float a, float s, float r, Cand &k) {
    encode16(B.w, r, k.c0, k.c1);
    float fw, fq;
    sums_bf16(k.c0, k.c1, B.p, fw, fq);
    k.sw = fw;
    k.sq = fq;
    return finite_pos(r) && a <= 32.0f * s && a <= 0x1p100f;
}

// fos_choice's comparison: whether M=4 (scale v4, candidate k4) has the strictly smaller squared error.
__device__ __forceinline__ bool fos_m4(float alpha, float v6, float v4, const Cand &k6, const Cand &k4) {
    const double sd6 = (double)alpha * (double)v6, sd4 = (double)alpha * (double)v4;
    const dd j6 = two_prod(sd6, fma(sd6, k6.sq, -2.0 * k6.sw));
    const dd j4 = two_prod(sd4, fma(sd4, k4.sq, -2.0 * k4.sw));
    return dd_less(j4, j6);
}

// fos_choice for two bf16 blocks A and B (max-rule codes dA6, dB6), their four candidates written out side by
// side; the rare cases (M=4 scale below E4M3's normal range, sums outside the binary32 window) take the
// general forms. Out: each block's chosen scale, its candidate, and whether M=4 was taken.
__device__ __forceinline__ void fos_pair(const Blk<false> &A, float aA, uint32_t dA6, const Blk<false> &B, float aB,
                                         uint32_t dB6, const ScaleTab &T, float alpha, uint32_t &dA, Cand &kA,
                                         bool &mA, uint32_t &dB, Cand &kB, bool &mB) {
    const float vA6 = e4m3_value(dA6), vB6 = e4m3_value(dB6);
    uint32_t dA4, dB4;
    const bool nA = e4m3_rne_normal(1.5f * vA6, dA4), nB = e4m3_rne_normal(1.5f * vB6, dB4);  // 1.5 v exact
    if (!nA) dA4 = e4m3_rne(1.5 * (double)vA6);
    if (!nB) dB4 = e4m3_rne(1.5 * (double)vB6);
    const float sA6 = T.s[dA6], rA6 = T.r[dA6], sA4 = T.s[dA4], rA4 = T.r[dA4];
    const float sB6 = T.s[dB6], rB6 = T.r[dB6], sB4 = T.s[dB4], rB4 = T.r[dB4];
    Cand A6, A4, B6, B4;
    const bool fA6 = cand_fast(A, aA, sA6, rA6, A6), fA4 = cand_fast(A, aA, sA4, rA4, A4);
    const bool fB6 = cand_fast(B, aB, sB6, rB6, B6), fB4 = cand_fast(B, aB, sB4, rB4, B4);
    // the reciprocals pass opaquely, so that the compiler keeps these encodings apart from the ones above
    if (!fA6) quant_sums_r(A, aA, sA6, opaque(rA6), A6.c0, A6.c1, A6.sw, A6.sq);
    if (!fA4) quant_sums_r(A, aA, sA4, opaque(rA4), A4.c0, A4.c1, A4.sw, A4.sq);
    if (!fB6) quant_sums_r(B, aB, sB6, opaque(rB6), B6.c0, B6.c1, B6.sw, B6.sq);
    if (!fB4) quant_sums_r(B, aB, sB4, opaque(rB4), B4.c0, B4.c1, B4.sw, B4.sq);
    mA = fos_m4(alpha, vA6, e4m3_value(dA4), A6, A4);
    mB = fos_m4(alpha, vB6, e4m3_value(dB4), B6, B4);
    dA = mA ? dA4 : dA6;
    kA = mA ? A4 : A6;
    dB = mB ? dB4 : dB6;
    kB = mB ? B4 : B6;
}

template <bool F32, bool FOS>
__global__ __launch_bounds__(kQuantThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_quant(const void *__restrict__ W, int64_t nblk,
                                                          const uint32_t *__restrict__ amax_part, int amax_n,
                                                          uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                          float *__restrict__ alpha_out, uint8_t *__restrict__ mchoice,
                                                          nvfp4_stats_t *stats, uint32_t *__restrict__ m4_part) {
    __shared__ ScaleTab T;
    AmaxShare<kQuantThreads> am;
    float alpha = 0.0f, six_alpha = 0.0f;
    uint32_t m4count = 0u;
    auto pre = [&] { am.load(amax_part, amax_n); };
    auto post = [&] {
        const uint32_t abits = am.reduce();
        const bool nonfinite = abits >= 0x7F800000u;
        alpha = max_rule_alpha(abits);
        six_alpha = 6.0f * alpha;
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            *alpha_out = nonfinite ? __builtin_nanf("") : alpha;
            if (stats) stats->status = nonfinite ? NVFP4_STATUS_NONFINITE : 0u;
        }
        if (nonfinite) return false;
        build_scale_tab<kQuantThreads>(T, alpha);
        return true;
    };
    const auto one = [&](int64_t b, const Blk<F32> &B, uint32_t) {
        uint32_t c0, c1, sc;
        bool m4 = false;
        const float a = B.amax();
        const uint32_t d6 = e4m3_rne(max_rule_quotient(a, alpha));
        sc = d6;
        if constexpr (!FOS) {
            const float r = T.r[d6];
            if (finite_pos(r))
                encode16(B.w, r, c0, c1);
            else
                encode16_soft(B.w, r, c0, c1);
        } else {
            double sw, sq;
            m4 = fos_choice(B, a, T, alpha, d6, sc, c0, c1, sw, sq);
            if (mchoice) mchoice[b] = m4 ? 1 : 0;
            m4count += m4 ? 1u : 0u;
        }
        store_codes(codes, b, c0, c1);
        scales[b] = (uint8_t)sc;
    };
    // two bf16 blocks with their common path side by side (see k_cjso_iter), the rare cases per block
    const auto two = [&](int64_t bA, const auto &A, uint32_t, int64_t bB, const auto &B, uint32_t) {
        const float aA = A.amax(), aB = B.amax();
        uint32_t dA, dB;
        const bool eA = max_rule_est(aA, six_alpha, dA), eB = max_rule_est(aB, six_alpha, dB);
        if (!eA) dA = e4m3_rne(max_rule_quotient(aA, alpha));
        if (!eB) dB = e4m3_rne(max_rule_quotient(aB, alpha));
        if constexpr (!FOS) {
            const float rA = T.r[dA], rB = T.r[dB];
            uint32_t cA0, cA1, cB0, cB1;
            encode16(A.w, rA, cA0, cA1);
            encode16(B.w, rB, cB0, cB1);
            if (!finite_pos(rA)) encode16_soft(A.w, opaque(rA), cA0, cA1);
            if (!finite_pos(rB)) encode16_soft(B.w, opaque(rB), cB0, cB1);
            store_codes(codes, bA, cA0, cA1);
            store_codes(codes, bB, cB0, cB1);
            scales[bA] = (uint8_t)dA;
            scales[bB] = (uint8_t)dB;
        } else {
            uint32_t sA, sB;
            Cand kA, kB;
            bool mA, mB;
            fos_pair(A, aA, dA, B, aB, dB, T, alpha, sA, kA, mA, sB, kB, mB);
            if (mchoice) {
                mchoice[bA] = mA ? 1 : 0;
                mchoice[bB] = mB ? 1 : 0;
            }
            m4count += (mA ? 1u : 0u) + (mB ? 1u : 0u);
            store_codes(codes, bA, kA.c0, kA.c1);
            store_codes(codes, bB, kB.c0, kB.c1);
            scales[bA] = (uint8_t)sA;
            scales[bB] = (uint8_t)sB;
        }
    };
    // the opposite order to k_amax, which read the same blocks in the same work-group just before
    bool finite;
    if constexpr (F32)
        finite = for_my_blocks<kQuantThreads, kQuantDepth, F32>(W, nullptr, nblk, true, pre, post, one);
    else
        finite = for_my_pairs<kQuantThreads, F32>(W, nullptr, nblk, true, pre, post, two, one);
    if (!finite) {  // non-finite input: all-zero codes and scales
        const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
        for (int64_t b = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; b < nblk; b += stride) {
            store_codes(codes, b, 0u, 0u);
            scales[b] = 0;
            if (FOS && mchoice) mchoice[b] = 0;
        }
    }
    if (FOS && m4_part) {  // per work-group count of M=4 blocks (summed by k_count only if asked)
        __shared__ uint32_t cnt[kQuantThreads / 64];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m4count += (uint32_t)__shfl_xor((int)m4count, o);
        if ((threadIdx.x & 63) == 0) cnt[threadIdx.x >> 6] = m4count;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t t = 0u;
            for (int i = 0; i < kQuantThreads / 64; ++i) t += cnt[i];
            m4_part[blockIdx.x] = t;
        }
    }
}

// stats->m4_blocks = sum of the per-work-group counts (one work-group, fixed order).
constexpr int kCountThreads = 256;
__global__ __launch_bounds__(kCountThreads) void k_count(const uint32_t *__restrict__ part, int64_t n,
                                                         nvfp4_stats_t *stats) {
    __shared__ uint32_t red[kCountThreads / 64];
    uint32_t c = 0u;
    for (int64_t i = threadIdx.x; i < n; i += kCountThreads) c += part[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c += (uint32_t)__shfl_xor((int)c, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) stats->m4_blocks = red[0] + red[1] + red[2] + red[3];
}

// ----------------------------------------------------------------------------------------- CJSO

// Max rule (or, with FOS, FourOverSix's choice of block scale under the max-rule alpha) plus, when rounds
// follow (ROUNDS), the least-squares sums of the first alpha-step; without rounds these codes (and for
// SOAR the E4M3 bracket of the unrounded block scale: max|w|/(6 alpha), or 1.5*Delta6 where FourOverSix
// took M=4) are final.
template <bool F32, bool SOAR, bool ROUNDS, bool FOS>
__global__ __launch_bounds__(kCjsoThreads) __attribute__((amdgpu_waves_per_eu(NVFP4_CJSO_WAVES))) void k_cjso_init(const void *__restrict__ W, int64_t nblk,
                                                              const uint32_t *__restrict__ amax_part, int amax_n,
                                                              uint8_t *__restrict__ codes,
                                                              uint8_t *__restrict__ scales,
                                                              float *__restrict__ alpha_out,
                                                              float *__restrict__ alpha_state,
                                                              double *__restrict__ part_out,
                                                              uint16_t *__restrict__ brackets, nvfp4_stats_t *stats) {
    __shared__ ScaleTab T;
    AmaxShare<kCjsoThreads> am;
    float alpha = 0.0f, six_alpha = 0.0f;
    dd N = {0.0, 0.0}, D = {0.0, 0.0};
    auto pre = [&] { am.load(amax_part, amax_n); };
    auto post = [&] {
        const uint32_t abits = am.reduce();
        const bool nonfinite = abits >= 0x7F800000u;
        alpha = max_rule_alpha(abits);
        six_alpha = 6.0f * alpha;
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            const float av = nonfinite ? __builtin_nanf("") : alpha;
            alpha_state[0] = av;
            if (!ROUNDS) *alpha_out = av;
            if (stats) stats->status = nonfinite ? NVFP4_STATUS_NONFINITE : 0u;
        }
        if (nonfinite) return false;
        build_scale_tab<kCjsoThreads>(T, alpha);
        return true;
    };
    const auto one = [&](int64_t b, const Blk<F32> &B, uint32_t) {
        const float a = B.amax();
        const double q = max_rule_quotient(a, alpha);
        uint32_t d = e4m3_rne(q);
        double dstar = q;
        uint32_t c0, c1;
        double sw, sq;
        if constexpr (FOS) {
            const uint32_t d6 = d;
            if (fos_choice(B, a, T, alpha, d6, d, c0, c1, sw, sq)) dstar = 1.5 * (double)e4m3_value(d6);
        }
        const float v = e4m3_value(d);
        scales[b] = (uint8_t)d;
        if constexpr (!ROUNDS) {
            if constexpr (!FOS) {
                const float r = T.r[d];
                if (finite_pos(r))
                    encode16(B.w, r, c0, c1);
                else
                    encode16_soft(B.w, r, c0, c1);
            }
            store_codes(codes, b, c0, c1);
            if (SOAR) {
                uint32_t lo, hi;
                e4m3_bracket(dstar, lo, hi);
                brackets[b] = (uint16_t)(lo | (hi << 8));
            }
        } else {
            if constexpr (!FOS) quant_sums_r(B, a, T.s[d], T.r[d], c0, c1, sw, sq);
            const dd t = two_prod((double)v, sw);
            acc2(N, t.hi, t.lo);
            acc2(D, (double)v * (double)v * sq, 0.0);
        }
    };
    // two bf16 blocks with their common path side by side (see k_cjso_iter), the rare cases per block
    const auto two = [&](int64_t bA, const auto &A, uint32_t, int64_t bB, const auto &B, uint32_t) {
        const float aA = A.amax(), aB = B.amax();
        uint32_t dA, dB;
        const bool eA = max_rule_est(aA, six_alpha, dA), eB = max_rule_est(aB, six_alpha, dB);
        if (!eA) dA = e4m3_rne(max_rule_quotient(aA, alpha));
        if (!eB) dB = e4m3_rne(max_rule_quotient(aB, alpha));
        const uint32_t dA6 = dA, dB6 = dB;
        Cand kA, kB;
        bool mA = false, mB = false;
        if constexpr (FOS) {
            fos_pair(A, aA, dA6, B, aB, dB6, T, alpha, dA, kA, mA, dB, kB, mB);
        } else if constexpr (ROUNDS) {
            const float sA = T.s[dA], rA = T.r[dA], sB = T.s[dB], rB = T.r[dB];
            const bool fA = cand_fast(A, aA, sA, rA, kA), fB = cand_fast(B, aB, sB, rB, kB);
            if (!fA) quant_sums_r(A, aA, sA, opaque(rA), kA.c0, kA.c1, kA.sw, kA.sq);
            if (!fB) quant_sums_r(B, aB, sB, opaque(rB), kB.c0, kB.c1, kB.sw, kB.sq);
        } else {
            const float rA = T.r[dA], rB = T.r[dB];
            encode16(A.w, rA, kA.c0, kA.c1);
            encode16(B.w, rB, kB.c0, kB.c1);
            if (!finite_pos(rA)) encode16_soft(A.w, opaque(rA), kA.c0, kA.c1);
            if (!finite_pos(rB)) encode16_soft(B.w, opaque(rB), kB.c0, kB.c1);
        }
        scales[bA] = (uint8_t)dA;
        scales[bB] = (uint8_t)dB;
        if constexpr (!ROUNDS) {
            store_codes(codes, bA, kA.c0, kA.c1);
            store_codes(codes, bB, kB.c0, kB.c1);
            if (SOAR) {
                const double sA = mA ? 1.5 * (double)e4m3_value(dA6) : max_rule_quotient(aA, alpha);
                const double sB = mB ? 1.5 * (double)e4m3_value(dB6) : max_rule_quotient(aB, alpha);
                uint32_t lo, hi;
                e4m3_bracket(sA, lo, hi);
                brackets[bA] = (uint16_t)(lo | (hi << 8));
                e4m3_bracket(sB, lo, hi);
                brackets[bB] = (uint16_t)(lo | (hi << 8));
            }
        } else {
            const float vA = e4m3_value(dA), vB = e4m3_value(dB);
            const dd tA = two_prod((double)vA, kA.sw);
            acc2(N, tA.hi, tA.lo);
            acc2(D, (double)vA * (double)vA * kA.sq, 0.0);
            const dd tB = two_prod((double)vB, kB.sw);
            acc2(N, tB.hi, tB.lo);
            acc2(D, (double)vB * (double)vB * kB.sq, 0.0);
        }
    };
    // the opposite order to k_amax, which read the same blocks in the same work-group just before
    bool finite;
    if constexpr (F32)
        finite = for_my_blocks<kCjsoThreads, kCjsoDepth, F32>(W, nullptr, nblk, true, pre, post, one);
    else
        finite = for_my_pairs<kCjsoThreads, F32>(W, nullptr, nblk, true, pre, post, two, one);
    if (!finite) {  // non-finite input: all-zero outputs; the rounds see alpha = NaN and stop
        const int64_t stride = (int64_t)gridDim.x * kCjsoThreads;
        for (int64_t b = (int64_t)blockIdx.x * kCjsoThreads + threadIdx.x; b < nblk; b += stride) {
            store_codes(codes, b, 0u, 0u);
            scales[b] = 0;
            if (SOAR) brackets[b] = 0;
        }
    }
    if (ROUNDS) {
        wg_sum_dd2<kCjsoThreads>(N, D);
        if (threadIdx.x == kSumLane) {
            part_out[4 * blockIdx.x + 0] = N.hi;
            part_out[4 * blockIdx.x + 1] = N.lo;
            part_out[4 * blockIdx.x + 2] = D.hi;
            part_out[4 * blockIdx.x + 3] = D.lo;
        }
    }
}

// CJSO round t (1..iters): alpha-step from the previous round's sums, re-quantise, Delta-step (SOAR
// page, block-scale closed form, rounded to E4M3), re-quantise; then the sums for round t+1, or, in the
// last round (LAST), the codes (before the SOAR search: the E4M3 bracket of the unrounded block scale
// instead, since the search writes every block's codes).
template <bool F32, bool SOAR, bool LAST>
__global__ __launch_bounds__(kCjsoThreads) __attribute__((amdgpu_waves_per_eu(NVFP4_CJSO_WAVES))) void k_cjso_iter(const void *__restrict__ W, int64_t nblk, int t,
                                                              const double *__restrict__ part_in, int n_part,
                                                              double *__restrict__ part_out, float *alpha_state,
                                                              float *__restrict__ alpha_out,
                                                              uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                              uint16_t *__restrict__ brackets) {
    __shared__ ScaleTab T;
    CjsoShare<kCjsoThreads, kCjsoGroups> sh;
    float alpha = 0.0f;
    dd Nn = {0.0, 0.0}, Dn = {0.0, 0.0};
    auto pre = [&] { sh.load(part_in, n_part); };
    auto post = [&] {
        const float prev = alpha_state[(t - 1) & 1];
        if (prev != prev) {  // non-finite input: the outputs were zeroed by the first pass
            if (blockIdx.x == 0 && threadIdx.x == 0) {
                alpha_state[t & 1] = prev;
                if (LAST) *alpha_out = prev;
            }
            return false;
        }
        dd N, D;
        sh.reduce(N, D);
        alpha = alpha_from(N, D, prev);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            alpha_state[t & 1] = alpha;
            if (LAST) *alpha_out = alpha;
        }
        build_scale_tab<kCjsoThreads>(T, alpha);
        return true;
    };
    // The Delta-step's E4M3 code (and, where the search's bracket needs it, its unrounded quotient); a block
    // whose codes are all zero keeps its scale. Elsewhere the code comes from a binary32 estimate where that
    // decides it, and from the binary64 quotient where it does not.
    const auto delta_step = [&](double sw, double sq, uint32_t d, double &dstar, uint32_t &dn) {
        const bool pos = sq > 0.0;
        if constexpr (LAST && SOAR) {
            const double q = sw / ((double)alpha * sq);  // not used when sq = 0
            dstar = pos ? q : (double)e4m3_value(d);
            dn = pos ? e4m3_rne(q) : d;
        } else {
            uint32_t c;
            const bool ok = e4m3_quotient_est((float)sw, alpha * (float)sq, c);
            dstar = 0.0;  // not used
            dn = pos ? c : d;
            if (pos && !ok) dn = e4m3_rne(sw / ((double)alpha * sq));
        }
    };
    // After the block's last re-quantisation: the sums of the next alpha-step, or the final outputs. Before the
    // search (SOAR) the last round writes only the scale and the bracket: the search writes every block's codes.
    constexpr bool kRequant = !(LAST && SOAR);  // whether the codes and sums after the Delta-step are used
    const auto finish = [&](int64_t b, uint32_t dn, double dstar, uint32_t c0, uint32_t c1, double sw, double sq) {
        if (!LAST) {
            // vn has 4 significant bits, S_wq at most 53 and S_qq at most 12: v*S_wq needs the exact
            // product, v^2*S_qq is exact in binary64
            const float vn = e4m3_value(dn);
            const dd tn = two_prod((double)vn, sw);
            acc2(Nn, tn.hi, tn.lo);
            acc2(Dn, (double)vn * (double)vn * sq, 0.0);
        } else if (SOAR) {
            uint32_t lo, hi;
            e4m3_bracket(dstar, lo, hi);
            brackets[b] = (uint16_t)(lo | (hi << 8));
        } else {
            store_codes(codes, b, c0, c1);
        }
    };
    const auto one = [&](int64_t b, const Blk<F32> &B, uint32_t d) {
        uint32_t c0, c1, dn;
        double sw, sq, dstar;
        const float a = B.amax();
        quant_sums_r(B, a, T.s[d], T.r[d], c0, c1, sw, sq);
        delta_step(sw, sq, d, dstar, dn);
        scales[b] = (uint8_t)dn;
        // an unchanged scale re-quantises to the same codes and sums (the common case once the rounds
        // settle; a wave skips this when none of its blocks changed)
        if (kRequant && dn != d) quant_sums_r(B, a, T.s[dn], T.r[dn], c0, c1, sw, sq);
        finish(b, dn, dstar, c0, c1, sw, sq);
    };
    // Two blocks with their common path written out side by side (hardware codes, binary32 sums, the
    // Delta-step), so that one block's arithmetic fills the other's latencies; a block outside the binary32
    // sums' exactness window redoes its first pass on the general path (its reciprocal passed opaquely, so
    // that the compiler does not merge the two encodings into one branch between the blocks).
    const auto two = [&](int64_t bA, const auto &A, uint32_t dA, int64_t bB, const auto &B, uint32_t dB) {
        const float aA = A.amax(), aB = B.amax();
        const float sA = T.s[dA], rA = T.r[dA], sB = T.s[dB], rB = T.r[dB];
        uint32_t cA0, cA1, cB0, cB1;
        encode16(A.w, rA, cA0, cA1);
        encode16(B.w, rB, cB0, cB1);
        float fwA, fqA, fwB, fqB;
        sums_bf16(cA0, cA1, A.p, fwA, fqA);
        sums_bf16(cB0, cB1, B.p, fwB, fqB);
        double swA = fwA, sqA = fqA, swB = fwB, sqB = fqB;
        if (!(finite_pos(rA) && aA <= 32.0f * sA && aA <= 0x1p100f)) quant_sums_r(A, aA, sA, opaque(rA), cA0, cA1, swA, sqA);
        if (!(finite_pos(rB) && aB <= 32.0f * sB && aB <= 0x1p100f)) quant_sums_r(B, aB, sB, opaque(rB), cB0, cB1, swB, sqB);
        uint32_t dnA, dnB;
        double dsA, dsB;
        delta_step(swA, sqA, dA, dsA, dnA);
        delta_step(swB, sqB, dB, dsB, dnB);
        scales[bA] = (uint8_t)dnA;
        scales[bB] = (uint8_t)dnB;
        if (kRequant && dnA != dA) quant_sums_r(A, aA, T.s[dnA], T.r[dnA], cA0, cA1, swA, sqA);
        if (kRequant && dnB != dB) quant_sums_r(B, aB, T.s[dnB], T.r[dnB], cB0, cB1, swB, sqB);
        finish(bA, dnA, dsA, cA0, cA1, swA, sqA);
        finish(bB, dnB, dsB, cB0, cB1, swB, sqB);
    };
    // forward: round 1 starts on the blocks k_cjso_init (which runs backwards) read last; alternating the
    // order of later rounds as well was timed and gained nothing (their time is spent on arithmetic)
    bool went;
    if constexpr (F32)
        went = for_my_blocks<kCjsoThreads, kCjsoDepth, F32>(W, scales, nblk, false, pre, post, one);
    else
        went = for_my_pairs<kCjsoThreads, F32>(W, scales, nblk, false, pre, post, two, one);
    if (!went) return;
    if (!LAST) {
        wg_sum_dd2<kCjsoThreads>(Nn, Dn);
        if (threadIdx.x == kSumLane) {
            part_out[4 * blockIdx.x + 0] = Nn.hi;
            part_out[4 * blockIdx.x + 1] = Nn.lo;
            part_out[4 * blockIdx.x + 2] = Dn.hi;
            part_out[4 * blockIdx.x + 3] = Dn.lo;
        }
    }
}

// ------------------------------------------------------------------------------ codec kernels

// One code per output byte; 8 values per lane.
__global__ __launch_bounds__(256) void k_encode_e2m1(const float *__restrict__ x, int64_t n,
                                                     uint8_t *__restrict__ out) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t base = 8 * g;
    if (base >= n) return;
    if (base + 8 <= n) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = x[base + j];
        uint32_t c = e2m1_clear_negzero(e2m1_pack8(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]));
        uint32_t lo = 0u, hi = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t a = (v[j] != v[j]) ? 0u : ((c >> (4 * j)) & 15u);
            const uint32_t b = (v[4 + j] != v[4 + j]) ? 0u : ((c >> (4 * (4 + j))) & 15u);
            lo |= a << (8 * j);
            hi |= b << (8 * j);
        }
        *reinterpret_cast<uint2 *>(out + base) = make_uint2(lo, hi);
    } else {
        for (int64_t i = base; i < n; ++i) out[i] = (uint8_t)e2m1_soft(x[i]);
    }
}

// SOAR page, dequantisation: w_hat = Q * (alpha * Delta). q*Delta is exact in binary32 (at most 6
// significant bits); the product with alpha is rounded once to the output type.
template <bool OUTF32>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                                 const float *__restrict__ alpha_p, int64_t nblk, void *__restrict__ out) {
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblk) return;
    const float alpha = *alpha_p;
    const float dv = e4m3_value(scales[b] & 0x7Fu);
    const uint2 c = *reinterpret_cast<const uint2 *>(codes + 8 * b);
    float o[16];
    const uint32_t cw[2] = {c.x, c.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        f32x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[h], 1.0f, 0);
        f32x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[h], 1.0f, 1);
        f32x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[h], 1.0f, 2);
        f32x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[h], 1.0f, 3);
        const float q[8] = {q0.x, q0.y, q1.x, q1.y, q2.x, q2.y, q3.x, q3.y};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float qd = q[j] * dv;  // exact
            if (OUTF32) {
                o[8 * h + j] = qd * alpha;
            } else {
                // round the exact product to bf16 once: p = f + e exactly with f = fl32(p); a bf16
                // midpoint f is resolved by the sign of e.
                const float f = qd * alpha;
                const float e = fmaf(qd, alpha, -f);
                uint32_t u = __float_as_uint(f);
                const uint32_t low = u & 0xFFFFu;
                if (low == 0x8000u && e != 0.0f) {
                    const bool away = (e > 0.0f) == (f > 0.0f);
                    u = away ? u + 0x8000u : u - 0x8000u;
                } else {
                    u = u + 0x7FFFu + ((u >> 16) & 1u);
                }
                o[8 * h + j] = __uint_as_float(u & 0xFFFF0000u);
            }
        }
    }
    if (OUTF32) {
        float4 *dst = reinterpret_cast<float4 *>(out) + 4 * b;
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[k] = make_float4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
    } else {
        uint4 *dst = reinterpret_cast<uint4 *>(out) + 2 * b;
        uint32_t p[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) p[k] = (__float_as_uint(o[2 * k]) >> 16) | (__float_as_uint(o[2 * k + 1]) & 0xFFFF0000u);
        dst[0] = make_uint4(p[0], p[1], p[2], p[3]);
        dst[1] = make_uint4(p[4], p[5], p[6], p[7]);
    }
}

// --------------------------------------------------------------------------- error statistics

// Reconstruction error and code histogram of an encoding (SOAR page, dequantisation: the reconstruction
// of w is Q * alpha * Delta). Per element d = fl64(w - (q*alpha)*Delta) (q*alpha and the product with
// Delta are exact in binary64), and d^2 is summed exactly as a double-double; each work-group writes its
// sum and its 16 code counts, and k_stats_final adds the partials in a fixed order.
constexpr int kStatThreads = 256;
constexpr int kStatMaxGroups = 512;

template <bool F32>
__global__ __launch_bounds__(kStatThreads) void k_stats(const void *__restrict__ W, int64_t nblk,
                                                        const uint8_t *__restrict__ codes,
                                                        const uint8_t *__restrict__ scales,
                                                        const float *__restrict__ alpha_p, double *__restrict__ part,
                                                        uint32_t *__restrict__ part_hist) {
    __shared__ uint32_t hist[16];
    if (threadIdx.x < 16) hist[threadIdx.x] = 0u;
    lds_barrier();
    const double alpha = (double)*alpha_p;
    dd S = {0.0, 0.0}, Z = {0.0, 0.0};
    const int64_t stride = (int64_t)gridDim.x * kStatThreads;
    for (int64_t b = (int64_t)blockIdx.x * kStatThreads + threadIdx.x; b < nblk; b += stride) {
        Blk<F32> B;
        B.load(W, b);
        const uint2 c = *reinterpret_cast<const uint2 *>(codes + 8 * b);
        const double dv = (double)e4m3_value(scales[b] & 0x7Fu);
        const uint32_t cw[2] = {c.x, c.y};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const f32x2 q = p == 0   ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[h], 1.0f, 0)
                                : p == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[h], 1.0f, 1)
                                : p == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[h], 1.0f, 2)
                                         : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[h], 1.0f, 3);
                const int j = 8 * h + 2 * p;
                const double d0 = (double)B.w[j] - (double)q.x * alpha * dv;
                const double d1 = (double)B.w[j + 1] - (double)q.y * alpha * dv;
                const dd e0 = two_prod(d0, d0), e1 = two_prod(d1, d1);
                acc2(S, e0.hi, e0.lo);
                acc2(S, e1.hi, e1.lo);
                atomicAdd(&hist[(cw[h] >> (8 * p)) & 15u], 1u);
                atomicAdd(&hist[(cw[h] >> (8 * p + 4)) & 15u], 1u);
            }
        }
    }
    wg_sum_dd2<kStatThreads>(S, Z);
    lds_barrier();
    if (threadIdx.x == kSumLane) {
        part[2 * blockIdx.x] = S.hi;
        part[2 * blockIdx.x + 1] = S.lo;
    }
    if (threadIdx.x < 16) part_hist[16 * blockIdx.x + threadIdx.x] = hist[threadIdx.x];
}

// sse_out = sum of the partial sums (fixed order), hist_out[i] = sum of the partial counts of code i.
__global__ __launch_bounds__(kStatThreads) void k_stats_final(const double *__restrict__ part,
                                                              const uint32_t *__restrict__ part_hist, int groups,
                                                              double *__restrict__ sse_out,
                                                              unsigned long long *__restrict__ hist_out) {
    // code counts: thread t adds code t % 16 over every 16th work-group (eight independent loads at a
    // time, consecutive threads on consecutive words), then the 16 slices of each code are added
    constexpr int kSlices = kStatThreads / 16;
    __shared__ unsigned long long slice[kStatThreads];
    const int code = threadIdx.x & 15, first = threadIdx.x >> 4;
    unsigned long long n = 0ull;
    for (int g0 = first; g0 < groups; g0 += 8 * kSlices) {
        uint32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int g = g0 + u * kSlices;
            v[u] = g < groups ? part_hist[16 * g + code] : 0u;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) n += v[u];
    }
    slice[threadIdx.x] = n;
    lds_barrier();
    dd S = {0.0, 0.0}, Z = {0.0, 0.0};
    for (int g = threadIdx.x; g < groups; g += kStatThreads) S = dd_add(S, dd{part[2 * g], part[2 * g + 1]});
    wg_sum_dd2<kStatThreads>(S, Z);
    if (threadIdx.x == kSumLane) *sse_out = S.hi + S.lo;
    if (threadIdx.x < 16) {
        unsigned long long t = 0ull;
#pragma unroll
        for (int k = 0; k < kSlices; ++k) t += slice[16 * k + threadIdx.x];
        hist_out[threadIdx.x] = t;
    }
}

// ------------------------------------------------------------------------------------ launchers

static int stream_groups(int64_t nblk, int threads, int max_groups) {
    int64_t g = (nblk + (int64_t)threads * kMinBlocksPerThread - 1) / ((int64_t)threads * kMinBlocksPerThread);
    return (int)(g < 1 ? 1 : (g > max_groups ? max_groups : g));
}
int quant_groups(int64_t nblk) { return stream_groups(nblk, kQuantThreads, kQuantGroups); }
int cjso_groups(int64_t nblk) { return stream_groups(nblk, kCjsoThreads, kCjsoGroups); }

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t workspace_bytes(int64_t nblk, int mode) {
    size_t s = align256(sizeof(uint32_t) * kAmaxMaxGroups) + align256(2 * sizeof(float)) +
               align256(sizeof(double) * 2 * kCjsoGroups * 4);
    if (mode == NVFP4_MODE_FOUR_OVER_SIX) s += align256(sizeof(uint32_t) * kQuantGroups);
    if (mode == NVFP4_MODE_SOAR) s += align256(sizeof(uint16_t) * (size_t)nblk);
    return s;
}

Workspace carve(void *base, int64_t nblk) {
    (void)nblk;
    char *p = static_cast<char *>(base);
    Workspace w;
    w.amax_part = reinterpret_cast<uint32_t *>(p);
    p += align256(sizeof(uint32_t) * kAmaxMaxGroups);
    w.alpha_state = reinterpret_cast<float *>(p);
    p += align256(2 * sizeof(float));
    w.cjso_part = reinterpret_cast<double *>(p);
    p += align256(sizeof(double) * 2 * kCjsoGroups * 4);
    w.brackets = reinterpret_cast<uint16_t *>(p);  // SOAR only
    w.m4_part = reinterpret_cast<uint32_t *>(p);    // FourOverSix only (same offset: the modes differ)
    return w;
}

hipError_t launch_amax(const void *W, bool f32, int64_t nblk, bool for_cjso, uint32_t *amax_part, int &groups,
                       nvfp4_stats_t *stats, hipStream_t stream) {
    if (for_cjso) {
        groups = cjso_groups(nblk);
        if (f32)
            hipLaunchKernelGGL((k_amax<true, kCjsoThreads>), dim3(groups), dim3(kCjsoThreads), 0, stream, W, nblk,
                               amax_part, stats);
        else
            hipLaunchKernelGGL((k_amax<false, kCjsoThreads>), dim3(groups), dim3(kCjsoThreads), 0, stream, W, nblk,
                               amax_part, stats);
    } else {
        groups = quant_groups(nblk);
        if (f32)
            hipLaunchKernelGGL((k_amax<true, kQuantThreads>), dim3(groups), dim3(kQuantThreads), 0, stream, W, nblk,
                               amax_part, stats);
        else
            hipLaunchKernelGGL((k_amax<false, kQuantThreads>), dim3(groups), dim3(kQuantThreads), 0, stream, W,
                               nblk, amax_part, stats);
    }
    return hipGetLastError();
}

hipError_t launch_quant(const void *W, bool f32, bool fos, int64_t nblk, const uint32_t *amax_part, int amax_n,
                        uint8_t *codes, uint8_t *scales, float *alpha_out, uint8_t *mchoice, nvfp4_stats_t *stats,
                        uint32_t *m4_part, hipStream_t stream) {
    const int groups = quant_groups(nblk);
    const dim3 grid(groups), block(kQuantThreads);
    uint32_t *mp = (fos && stats) ? m4_part : nullptr;
    if (f32) {
        if (fos)
            hipLaunchKernelGGL((k_quant<true, true>), grid, block, 0, stream, W, nblk, amax_part, amax_n, codes, scales,
                               alpha_out, mchoice, stats, mp);
        else
            hipLaunchKernelGGL((k_quant<true, false>), grid, block, 0, stream, W, nblk, amax_part, amax_n, codes,
                               scales, alpha_out, mchoice, stats, mp);
    } else {
        if (fos)
            hipLaunchKernelGGL((k_quant<false, true>), grid, block, 0, stream, W, nblk, amax_part, amax_n, codes,
                               scales, alpha_out, mchoice, stats, mp);
        else
            hipLaunchKernelGGL((k_quant<false, false>), grid, block, 0, stream, W, nblk, amax_part, amax_n, codes,
                               scales, alpha_out, mchoice, stats, mp);
    }
    if (mp) hipLaunchKernelGGL(k_count, dim3(1), dim3(kCountThreads), 0, stream, mp, groups, stats);
    return hipGetLastError();
}

hipError_t launch_cjso_init(const void *W, bool f32, bool soar, bool fos, int64_t nblk, const uint32_t *amax_part,
                            int amax_n, int iters, uint8_t *codes, uint8_t *scales, float *alpha_out,
                            const Workspace &ws, int groups, nvfp4_stats_t *stats, hipStream_t stream) {
    const dim3 grid(groups), block(kCjsoThreads);
    double *part = ws.cjso_part;  // round 0 writes buffer 0
#define NVFP4_INIT(F, S, R, O)                                                                                    \
    hipLaunchKernelGGL((k_cjso_init<F, S, R, O>), grid, block, 0, stream, W, nblk, amax_part, amax_n, codes, scales, \
                       alpha_out, ws.alpha_state, part, ws.brackets, stats)
#define NVFP4_INIT_O(F, S, R)                                                                                     \
    do {                                                                                                          \
        if (fos) NVFP4_INIT(F, S, R, true); else NVFP4_INIT(F, S, R, false);                                      \
    } while (0)
#define NVFP4_INIT_R(F, S)                                                                                        \
    do {                                                                                                          \
        if (iters > 0) NVFP4_INIT_O(F, S, true); else NVFP4_INIT_O(F, S, false);                                  \
    } while (0)
    if (f32) {
        if (soar) NVFP4_INIT_R(true, true); else NVFP4_INIT_R(true, false);
    } else {
        if (soar) NVFP4_INIT_R(false, true); else NVFP4_INIT_R(false, false);
    }
#undef NVFP4_INIT_R
#undef NVFP4_INIT_O
#undef NVFP4_INIT
    return hipGetLastError();
}

hipError_t launch_cjso_iter(const void *W, bool f32, bool soar, int64_t nblk, int t, int iters, uint8_t *codes,
                            uint8_t *scales, float *alpha_out, const Workspace &ws, int groups, hipStream_t stream) {
    const dim3 grid(groups), block(kCjsoThreads);
    const double *pin = ws.cjso_part + (size_t)((t - 1) & 1) * kCjsoGroups * 4;
    double *pout = ws.cjso_part + (size_t)(t & 1) * kCjsoGroups * 4;
#define NVFP4_ITER(F, S, L)                                                                                       \
    hipLaunchKernelGGL((k_cjso_iter<F, S, L>), grid, block, 0, stream, W, nblk, t, pin, groups, pout,              \
                       ws.alpha_state, alpha_out, codes, scales, ws.brackets)
#define NVFP4_ITER_L(F, S)                                                                                        \
    do {                                                                                                          \
        if (t == iters) NVFP4_ITER(F, S, true); else NVFP4_ITER(F, S, false);                                     \
    } while (0)
    if (f32) {
        if (soar) NVFP4_ITER_L(true, true); else NVFP4_ITER_L(true, false);
    } else {
        if (soar) NVFP4_ITER_L(false, true); else NVFP4_ITER_L(false, false);
    }
#undef NVFP4_ITER_L
#undef NVFP4_ITER
    return hipGetLastError();
}

hipError_t launch_encode_e2m1(const float *x, int64_t n, uint8_t *codes, hipStream_t stream) {
    const int64_t lanes = (n + 7) / 8;
    hipLaunchKernelGGL(k_encode_e2m1, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, stream, x, n, codes);
    return hipGetLastError();
}

// The reciprocal the search uses (recip_rn), element-wise; for the self-check entry point.
__global__ __launch_bounds__(256) void k_reciprocal(const float *__restrict__ s, int64_t n, float *__restrict__ r) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) r[i] = recip_rn(s[i]);
}

hipError_t launch_reciprocal(const float *s, int64_t n, float *r, hipStream_t stream) {
    hipLaunchKernelGGL(k_reciprocal, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, s, n, r);
    return hipGetLastError();
}

size_t stats_workspace_bytes() {
    return align256(sizeof(double) * 2 * kStatMaxGroups) + align256(sizeof(uint32_t) * 16 * kStatMaxGroups);
}

hipError_t launch_stats(const void *W, bool f32, int64_t nblk, const uint8_t *codes, const uint8_t *scales,
                        const float *alpha, double *sse_out, unsigned long long *hist_out, void *workspace,
                        hipStream_t stream) {
    int64_t g = (nblk + 4 * kStatThreads - 1) / (4 * kStatThreads);
    const int groups = (int)(g < 1 ? 1 : (g > kStatMaxGroups ? kStatMaxGroups : g));
    double *part = static_cast<double *>(workspace);
    uint32_t *part_hist = reinterpret_cast<uint32_t *>(static_cast<char *>(workspace) +
                                                       align256(sizeof(double) * 2 * kStatMaxGroups));
    if (f32)
        hipLaunchKernelGGL(k_stats<true>, dim3(groups), dim3(kStatThreads), 0, stream, W, nblk, codes, scales, alpha,
                           part, part_hist);
    else
        hipLaunchKernelGGL(k_stats<false>, dim3(groups), dim3(kStatThreads), 0, stream, W, nblk, codes, scales, alpha,
                           part, part_hist);
    hipLaunchKernelGGL(k_stats_final, dim3(1), dim3(kStatThreads), 0, stream, part, part_hist, groups, sse_out,
                       hist_out);
    return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t *codes, const uint8_t *scales, const float *alpha, int64_t nblk, void *out,
                          bool out_f32, hipStream_t stream) {
    const dim3 grid((unsigned)((nblk + 255) / 256)), block(256);
    if (out_f32)
        hipLaunchKernelGGL(k_dequant<true>, grid, block, 0, stream, codes, scales, alpha, nblk, out);
    else
        hipLaunchKernelGGL(k_dequant<false>, grid, block, 0, stream, codes, scales, alpha, nblk, out);
    return hipGetLastError();
}

}  // namespace nvfp4
