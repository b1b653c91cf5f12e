// gfx950 W4A16 matrix product with NVFP4 weights: Y[M][N] = X[M][K] * What[N][K]^T, where What is the
// reconstruction the SOAR page defines (dequantisation equation): e2m1(code) * e4m3(scale) * alpha, for
// a weight matrix stored as the quantiser writes it ([N][K] codes, two per byte, one E4M3 scale per 16
// consecutive k). X is bf16.
//
// Arithmetic. q * Delta has at most 6 significant bits and lies in [2^-10, 2688], so every dequantised
// weight without alpha is exactly a bf16: the bf16 MFMA forms exact products and accumulates them in
// fp32, and alpha multiplies the fp32 sum once at the end (y = fl(alpha * acc), then rounded to the
// output type). Only the accumulation order differs from an exact product.
//
// Kernels, by the number M of rows of X:
//   k_w4a16_gemv (M <= 4, X up to 128 KB; decoding one or a few tokens): bound by reading the 0.5625
//     bytes per weight once; each wave requests all codes of its row n up front, X sits in LDS, each
//     lane takes 32 consecutive k per 2048-k chunk, and the row sums are DPP wave reductions.
//   k_w4a16_skinny (M <= 64 otherwise): 16 weight rows per work-group, K split over its 16 waves, the
//     products on v_mfma_f32_16x16x32_bf16 with weights decoded straight into the A operand.
//   k_w4a16_gemm (M > 64): 256 x 128 output tile per work-group (4 waves, 128 x 64 each as 4 x 2 tiles of
//     v_mfma_f32_32x32x16_bf16; 128 x 64 for M <= 512 and 128 x 128 when the 256 x 128 tiles would not
//     fill the GPU), K in steps of 64 through
//     LDS: the X tile is copied, the weight tile is decoded to bf16 (codes -> binary32 q, times Delta,
//     high half) once per work-group as it is stored, and the next step's loads are in flight while the
//     matrix cores work on this one. When the tiles are too few to fill the GPU, K is split and
//     k_w4a16_reduce adds the slices.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "codec.hpp"
#include "launch.hpp"

namespace nvfp4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGemmThreads = 256;
constexpr int kBM = 256, kBN = 128, kBK = 64;

// Tile shapes: TM x TN outputs per work-group: 256 x 128 (large M), 128 x 128 (middle M: more
// work-groups, three per CU) and 128 x 64 (few rows of X: more tiles, so fewer and longer K slices).
// Four waves: 2 x 2 for TN = 128 (128 x 64 or 64 x 64 each), 4 x 1 of 32 x 64 for TN = 64. A K step
// (64 k) of X is TM / 32 16-byte loads per thread; a weight row of it (32 bytes of codes) is loaded by
// 256 / TN threads.
template <int TM, int TN>
struct TileCfg {
    static constexpr int kWavesN = TN == 128 ? 2 : 1, kWavesM = 4 / kWavesN;
    static constexpr int kWaveM = TM / kWavesM, kWaveN = TN / kWavesN;  // the wave's corner of the tile
    static constexpr int kMI = kWaveM / 32, kNJ = kWaveN / 32;            // 32 x 32 MFMA tiles per wave
    static constexpr int kRowThreads = kGemmThreads / TN;                // threads per weight row
    static constexpr int kThreadK = kBK / kRowThreads;                   // k per thread: 32 or 16
};
constexpr int kLdsStride = kBK + 8;  // bf16 per LDS row: the padding spreads the rows a wave reads over the banks

// 8 codes (one dword) and their scale value -> 8 dequantised weights (without alpha) as bf16 pairs.
__device__ __forceinline__ uint4 dequant8(uint32_t c, float dv) {
    const f32x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
    const f32x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
    const f32x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
    const f32x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
    // q*dv is exact and has at most 6 significant bits: its high 16 bits are the bf16 value. The byte
    // permute takes bytes 2, 3 of a*dv (selectors 2, 3: the second operand) and of b*dv (6, 7: the first).
    auto pair = [&](float a, float b) {
        return __builtin_amdgcn_perm(__float_as_uint(b * dv), __float_as_uint(a * dv), 0x07060302u);
    };
    return make_uint4(pair(q0.x, q0.y), pair(q1.x, q1.y), pair(q2.x, q2.y), pair(q3.x, q3.y));
}

// Round binary32 to bf16 (nearest, ties to even; infinities stay, a NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <bool OUTF32>
__device__ __forceinline__ void store_y(void *Y, int64_t idx, float v) {
    if (OUTF32)
        static_cast<float *>(Y)[idx] = v;
    else
        static_cast<uint16_t *>(Y)[idx] = to_bf16(v);
}

// One K step of a work-group's operands, held in registers between the global loads and the LDS stores:
// the X tile (256 rows x 64 k, 8 x 16 bytes per thread) and the weight tile (128 rows n x 64 k: 16 bytes
// of codes = 32 k and their two scale bytes per thread). Rows and k past the matrix read as zeros.
template <int TM>
struct GemmStage {
    uint4 x[TM / 32];
    uint4 c;
    uint32_t sc;
};

// k < kend is loaded (kend = K, or the end of a split-K slice: a multiple of the K step); K is the row
// length.
template <int TM, int TN>
__device__ __forceinline__ void gemm_load(GemmStage<TM> &S, const uint16_t *__restrict__ X, int64_t M, int64_t K,
                                          int64_t kend, const uint8_t *__restrict__ codes,
                                          const uint8_t *__restrict__ scales, int64_t N, int64_t m0, int64_t n0,
                                          int64_t k0, int tid) {
#pragma unroll
    for (int p = 0; p < TM / 32; ++p) {
        const int idx = tid + p * kGemmThreads;  // row idx / 8, 8-element group idx % 8
        const int64_t m = m0 + (idx >> 3), k = k0 + 8 * (idx & 7);
        S.x[p] = make_uint4(0u, 0u, 0u, 0u);
        if (m < M && k < kend) S.x[p] = *reinterpret_cast<const uint4 *>(X + m * K + k);  // K % 16 == 0
    }
    using C = TileCfg<TM, TN>;
    const int64_t n = n0 + tid / C::kRowThreads, k = k0 + C::kThreadK * (tid % C::kRowThreads);
    S.c = make_uint4(0u, 0u, 0u, 0u);
    S.sc = 0u;
    if (n < N && k < kend) {
        const int64_t e = n * K + k;  // element index, a multiple of 16
        if (C::kThreadK == 16) {  // 16 k: 8 bytes of codes, one scale byte (K % 16 == 0)
            const uint2 c2 = *reinterpret_cast<const uint2 *>(codes + e / 2);
            S.c = make_uint4(c2.x, c2.y, 0u, 0u);
            S.sc = (uint32_t)scales[e / 16];
        } else if (k + 32 <= kend) {
            S.c = *reinterpret_cast<const uint4 *>(codes + e / 2);
            S.sc = (uint32_t)scales[e / 16] | ((uint32_t)scales[e / 16 + 1] << 8);
        } else {  // K % 32 == 16: the last 16 k of the row
            const uint2 c2 = *reinterpret_cast<const uint2 *>(codes + e / 2);
            S.c = make_uint4(c2.x, c2.y, 0u, 0u);
            S.sc = (uint32_t)scales[e / 16];
        }
    }
}

// The unmasked form for a work-group whose tile and K slice lie inside the matrices: xp points at X row
// m0 + tid / 8, column k0 + 8 (tid % 8) (row p of the thread adds 32 p K), cp at the codes of weight row
// n0 + tid / R from k0 + kThreadK (tid % R) (R threads per weight row), sp at their scale bytes.
template <int TM, int TN>
__device__ __forceinline__ void gemm_load_full(GemmStage<TM> &S, const uint16_t *__restrict__ xp, int64_t K,
                                               const uint8_t *__restrict__ cp, const uint8_t *__restrict__ sp) {
#pragma unroll
    for (int p = 0; p < TM / 32; ++p) S.x[p] = *reinterpret_cast<const uint4 *>(xp + p * 32 * K);
    if (TileCfg<TM, TN>::kThreadK == 16) {
        const uint2 c2 = *reinterpret_cast<const uint2 *>(cp);
        S.c = make_uint4(c2.x, c2.y, 0u, 0u);
        S.sc = (uint32_t)sp[0];
    } else {
        S.c = *reinterpret_cast<const uint4 *>(cp);
        S.sc = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
    }
}

template <int TM, int TN>
__device__ __forceinline__ void gemm_store(const GemmStage<TM> &S, uint16_t *xs, uint16_t *ws, int tid) {
#pragma unroll
    for (int p = 0; p < TM / 32; ++p) {
        const int idx = tid + p * kGemmThreads;
        *reinterpret_cast<uint4 *>(&xs[(idx >> 3) * kLdsStride + 8 * (idx & 7)]) = S.x[p];
    }
    using C = TileCfg<TM, TN>;
    const float d0 = e4m3_value(S.sc & 0x7Fu);
    uint16_t *dst = &ws[(tid / C::kRowThreads) * kLdsStride + C::kThreadK * (tid % C::kRowThreads)];
    *reinterpret_cast<uint4 *>(dst) = dequant8(S.c.x, d0);
    *reinterpret_cast<uint4 *>(dst + 8) = dequant8(S.c.y, d0);
    if (C::kThreadK == 32) {
        const float d1 = e4m3_value((S.sc >> 8) & 0x7Fu);
        *reinterpret_cast<uint4 *>(dst + 16) = dequant8(S.c.z, d1);
        *reinterpret_cast<uint4 *>(dst + 24) = dequant8(S.c.w, d1);
    }
}

// TM x TN output tile per work-group (TileCfg: 4 waves of 128 x 64, 64 x 64 or 32 x 64, each as tiles of
// v_mfma_f32_32x32x16_bf16). The loads of K step t + 1 are issued into registers before the products of step t, so they are in
// flight while the matrix cores run; one LDS buffer (55 KB for 256 x 128, less for the smaller tiles) leaves room for at least two work-groups
// per CU.
// Waves raise their issue priority for the products, so a SIMD serves the work-group at its matrix
// step before the other one's decode and stores.
// Work-groups go to the 8 XCDs round robin; the tile order is remapped so that each XCD takes a
// contiguous band of tiles and its L2 holds the few X row blocks that band needs.
// Split K (when the tiles alone are too few to fill the chip): work-group b takes tile b % tiles and
// the K slice b / tiles of kslice elements, and writes its fp32 sums without alpha to
// part[slice][M][N]; k_w4a16_reduce adds the slices in order. With one slice it writes Y directly.
template <int TM, int TN, bool OUTF32>
__global__ __launch_bounds__(kGemmThreads, 2) void k_w4a16_gemm(const uint16_t *__restrict__ X, int64_t M, int64_t K,
                                                             const uint8_t *__restrict__ codes,
                                                             const uint8_t *__restrict__ scales,
                                                             const float *__restrict__ alpha_p, int64_t N,
                                                             void *__restrict__ Y, unsigned tiles_n, unsigned tiles,
                                                             int64_t kslice, float *__restrict__ part) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[TM * kLdsStride];
    __shared__ __attribute__((aligned(16))) uint16_t ws[TN * kLdsStride];
    using C = TileCfg<TM, TN>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const unsigned total = gridDim.x;  // 1-D grid: slices * tiles_m * tiles_n, tiles row-major
    unsigned b = blockIdx.x;
    if (total % 8 == 0) b = (b % 8) * (total / 8) + b / 8;
    const unsigned slice = b / tiles, t = b % tiles;
    const int64_t m0 = (int64_t)(t / tiles_n) * TM, n0 = (int64_t)(t % tiles_n) * TN;
    const int64_t kbeg = (int64_t)slice * kslice, kend = min(K, kbeg + kslice);
    const int wm = (wave / C::kWavesN) * C::kWaveM, wn = (wave % C::kWavesN) * C::kWaveN;  // the wave's corner
    f32x16 acc[C::kMI][C::kNJ] = {};
    GemmStage<TM> S;
    // the products of one K step from the staged tiles
    auto mfma_step = [&]() {
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 16) {
            bf16x8 a[C::kMI], bb[C::kNJ];
            // A operand: row (lane % 32) of a 32-row tile, k = 8 * (lane / 32) .. + 7; B: column lane % 32
#pragma unroll
            for (int i = 0; i < C::kMI; ++i)
                a[i] = *reinterpret_cast<const bf16x8 *>(&xs[(wm + 32 * i + (lane & 31)) * kLdsStride + kk + 8 * (lane >> 5)]);
#pragma unroll
            for (int j = 0; j < C::kNJ; ++j)
                bb[j] = *reinterpret_cast<const bf16x8 *>(&ws[(wn + 32 * j + (lane & 31)) * kLdsStride + kk + 8 * (lane >> 5)]);
#pragma unroll
            for (int i = 0; i < C::kMI; ++i)
#pragma unroll
                for (int j = 0; j < C::kNJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
        }
    };
    const bool full = m0 + TM <= M && n0 + TN <= N && (kend - kbeg) % kBK == 0;  // uniform
    if (full) {
        const uint16_t *xp = X + (m0 + (tid >> 3)) * K + kbeg + 8 * (tid & 7);
        // element index, a multiple of 16
        const int64_t e = (n0 + tid / C::kRowThreads) * K + kbeg + C::kThreadK * (tid % C::kRowThreads);
        const uint8_t *cp = codes + e / 2, *sp = scales + e / 16;
        gemm_load_full<TM, TN>(S, xp, K, cp, sp);
        for (int64_t k0 = kbeg; k0 < kend; k0 += kBK) {
            gemm_store<TM, TN>(S, xs, ws, tid);
            __syncthreads();
            xp += kBK;
            cp += kBK / 2;
            sp += kBK / 16;
            if (k0 + kBK < kend) gemm_load_full<TM, TN>(S, xp, K, cp, sp);
            __builtin_amdgcn_s_setprio(1);
            mfma_step();
            __builtin_amdgcn_s_setprio(0);
            __syncthreads();
        }
    } else {
        gemm_load<TM, TN>(S, X, M, K, kend, codes, scales, N, m0, n0, kbeg, tid);
        for (int64_t k0 = kbeg; k0 < kend; k0 += kBK) {
            gemm_store<TM, TN>(S, xs, ws, tid);
            __syncthreads();
            if (k0 + kBK < kend) gemm_load<TM, TN>(S, X, M, K, kend, codes, scales, N, m0, n0, k0 + kBK, tid);
            __builtin_amdgcn_s_setprio(1);
            mfma_step();
            __builtin_amdgcn_s_setprio(0);
            __syncthreads();
        }
    }
    // D layout: element e of lane l is row 8 * (e / 4) + 4 * (l / 32) + e % 4, column l % 32
    const float alpha = *alpha_p;
    float *const dst = part ? part + (int64_t)slice * M * N : nullptr;
    const int64_t mb = m0 + wm + 4 * (lane >> 5), nb = n0 + wn + (lane & 31);  // the lane's first row, column
    const int64_t yb = mb * N + nb;
#pragma unroll
    for (int i = 0; i < C::kMI; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int r = 32 * i + 8 * (e >> 2) + (e & 3);  // row offset from mb
            const int64_t yr = yb + r * N;
#pragma unroll
            for (int j = 0; j < C::kNJ; ++j) {
                if (!full && (mb + r >= M || nb + 32 * j >= N)) continue;
                if (dst)
                    dst[yr + 32 * j] = acc[i][j][e];
                else
                    store_y<OUTF32>(Y, yr + 32 * j, alpha * acc[i][j][e]);
            }
        }
}

constexpr int kReduceThreads = 256;

// Y = alpha * (sum of the split-K slices, added in slice order), rounded once to the output type.
template <bool OUTF32>
__global__ __launch_bounds__(kReduceThreads) void k_w4a16_reduce(const float *__restrict__ part, int slices,
                                                                 int64_t n, const float *__restrict__ alpha_p,
                                                                 void *__restrict__ Y) {
    const float alpha = *alpha_p;
    for (int64_t i = (int64_t)blockIdx.x * kReduceThreads + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kReduceThreads) {
        float acc = part[i];
        for (int sl = 1; sl < slices; ++sl) acc += part[(int64_t)sl * n + i];
        store_y<OUTF32>(Y, i, alpha * acc);
    }
}

// -------------------------------------------------------------------------------------- skinny MFMA

// Few rows of X (M <= 64): a work-group owns 16 weight rows n and its 16 waves split K into chunks of
// 128 k (wave w takes chunks w, w + 16, ...). Products run on v_mfma_f32_16x16x32_bf16 with the weights as
// the A operand (16 rows n) and X^T as the B operand (16 columns m per tile, MT tiles). The MFMA sums
// over its 32 k slots in any order, so each slot is mapped to the k that makes the loads contiguous:
// in chunk c, lane l (row or column l % 16, group g = l / 16) supplies for MFMA i (0..3) the 8 values at
// k = 128 c + 32 g + 8 i .. + 7, for the weights and for X alike. A lane thus loads 16 bytes of codes
// (two 16-blocks, two scale bytes) per chunk and decodes them straight into the A operand, and 64
// contiguous bytes of each of its X rows. Weights are read once; X (at most 64 x K bf16) comes from L2.
// The 16 waves' partial tiles are added through LDS in wave order, and alpha is applied once.
constexpr int kSkinnyThreads = 1024, kSkinnyWaves = kSkinnyThreads / 64, kSkinnyMaxM = 64;

template <int MT, bool OUTF32>
__global__ __launch_bounds__(kSkinnyThreads) void k_w4a16_skinny(const uint16_t *__restrict__ X, int M, int64_t K,
                                                                 const uint8_t *__restrict__ codes,
                                                                 const uint8_t *__restrict__ scales,
                                                                 const float *__restrict__ alpha_p, int64_t N,
                                                                 void *__restrict__ Y) {
    __shared__ float red[kSkinnyWaves][MT][256];  // each wave's 16 x 16 tiles, lane-major
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16, n = n0 + r16;
    const int64_t nch = (K + 127) / 128;
    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // the lane's codes (16 bytes) and scale bytes of chunk c; zeros past the row or past N
    auto load_w = [&](int64_t c, uint4 &cv, uint32_t &sv) {
        const int64_t k = 128 * c + 32 * g;
        cv = make_uint4(0u, 0u, 0u, 0u);
        sv = 0u;
        if (n < N && k < K) {
            const int64_t e = n * K + k;  // element index, a multiple of 16
            if (k + 32 <= K) {
                cv = *reinterpret_cast<const uint4 *>(codes + e / 2);
                sv = (uint32_t)scales[e / 16] | ((uint32_t)scales[e / 16 + 1] << 8);
            } else {  // K % 32 == 16: the row's last 16 k
                const uint2 c2 = *reinterpret_cast<const uint2 *>(codes + e / 2);
                cv = make_uint4(c2.x, c2.y, 0u, 0u);
                sv = scales[e / 16];
            }
        }
    };
    int64_t c = wave;
    uint4 cv;
    uint32_t sv;
    if (c < nch) load_w(c, cv, sv);
    for (; c < nch; c += kSkinnyWaves) {
        const uint4 cur = cv;
        const uint32_t scur = sv;
        if (c + kSkinnyWaves < nch) load_w(c + kSkinnyWaves, cv, sv);  // next chunk's weights in flight
        const int64_t k = 128 * c + 32 * g;
        // X rows m = 16 t + r16 at k .. k + 31 (zeros past M or past K; K % 16 == 0)
        uint4 xv[MT][4];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int m = 16 * t + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xv[t][i] = make_uint4(0u, 0u, 0u, 0u);
                if (m < M && k + 8 * i < K) xv[t][i] = *reinterpret_cast<const uint4 *>(X + (int64_t)m * K + k + 8 * i);
            }
        }
        const float d0 = e4m3_value(scur & 0x7Fu), d1 = e4m3_value((scur >> 8) & 0x7Fu);
        const uint4 w[4] = {dequant8(cur.x, d0), dequant8(cur.y, d0), dequant8(cur.z, d1), dequant8(cur.w, d1)};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < MT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w[i]),
                                                                 __builtin_bit_cast(bf16x8, xv[t][i]), acc[t], 0, 0, 0);
    }
    // D layout: element r of lane l is row n0 + 4 (l / 16) + r, column m = 16 t + l % 16
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][t][lane * 4 + r] = acc[t][r];
    __syncthreads();
    const float alpha = *alpha_p;
    for (int o = tid; o < MT * 256; o += kSkinnyThreads) {  // o = 256 t + 4 lane + r
        const int t = o >> 8, l = (o >> 2) & 63, r = o & 3;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kSkinnyWaves; ++w) sum += red[w][t][o & 255];
        const int64_t nn = n0 + 4 * (l >> 4) + r;
        const int m = 16 * t + (l & 15);
        if (nn < N && m < M) store_y<OUTF32>(Y, (int64_t)m * N + nn, alpha * sum);
    }
}

// ------------------------------------------------------------------------------------------- GEMV

#ifndef NVFP4_GEMV_THREADS
#define NVFP4_GEMV_THREADS 1024
#endif
#ifndef NVFP4_GEMV_ROWS
#define NVFP4_GEMV_ROWS 1
#endif
#ifndef NVFP4_GEMV_MAX_M
#define NVFP4_GEMV_MAX_M 4  // the GEMV serves M up to this; the skinny MFMA kernel the rest up to 64
#endif
constexpr int kGemvThreads = NVFP4_GEMV_THREADS;
constexpr int kGemvMaxM = NVFP4_GEMV_MAX_M;

// Wave sum on the VALU (DPP; the total ends in lane 63).
__device__ __forceinline__ float wave_sum_f32(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xA, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xC, 0xF, false));
    return x;
}

// Each wave owns kGemvRows consecutive rows n (one by default: with 16 waves per work-group the most
// loads are in flight) and, before anything else, requests all of their codes and scales (lane l takes
// k = 32 * (l + 64 c) .. + 31 of chunk c < CH, 16 bytes of codes): the whole weight matrix is in flight
// at once, which is what a read-once product needs. Meanwhile the work-group copies X (M rows, up to
// kGemvMaxLds bytes) to LDS; then each lane decodes its weights once, forms an fp32 dot product with
// packed bf16 dot instructions for each of the M rows of X, and DPP wave reductions give the sums.
// MM >= M is the compiled row count; rows past M are neither computed nor stored.
constexpr int kGemvRows = NVFP4_GEMV_ROWS;

template <int MM, int CH, bool OUTF32>
__global__ __launch_bounds__(kGemvThreads) void k_w4a16_gemv(const uint16_t *__restrict__ X, int M, int64_t K,
                                                             const uint8_t *__restrict__ codes,
                                                             const uint8_t *__restrict__ scales,
                                                             const float *__restrict__ alpha_p, int64_t N,
                                                             void *__restrict__ Y) {
    extern __shared__ __attribute__((aligned(16))) uint16_t xl[];  // [MM][K]
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t n0 = ((int64_t)blockIdx.x * (kGemvThreads / 64) + (tid >> 6)) * kGemvRows;
    uint4 c[kGemvRows][CH];
    uint32_t sc[kGemvRows][CH];  // the chunk's two scale bytes
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) {
            const int64_t n = n0 + r, k = 32 * (lane + 64 * ch);
            c[r][ch] = make_uint4(0u, 0u, 0u, 0u);
            sc[r][ch] = 0u;
            if (n < N && k < K) {
                const int64_t e = n * K + k;
                if (k + 32 <= K) {
                    c[r][ch] = *reinterpret_cast<const uint4 *>(codes + e / 2);
                    sc[r][ch] = (uint32_t)scales[e / 16] | ((uint32_t)scales[e / 16 + 1] << 8);
                } else {  // the row's last 16 k (K % 32 == 16)
                    const uint2 c2 = *reinterpret_cast<const uint2 *>(codes + e / 2);
                    c[r][ch] = make_uint4(c2.x, c2.y, 0u, 0u);
                    sc[r][ch] = (uint32_t)scales[e / 16];
                }
            }
        }
    for (int64_t i = tid; i < M * K / 8; i += kGemvThreads)
        reinterpret_cast<uint4 *>(xl)[i] = reinterpret_cast<const uint4 *>(X)[i];
    __syncthreads();
    const float alpha = *alpha_p;
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
        float s[MM];
#pragma unroll
        for (int m = 0; m < MM; ++m) s[m] = 0.0f;
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) {
            const int64_t k = 32 * (lane + 64 * ch);
            if (k >= K) break;
            const int nq = k + 32 <= K ? 4 : 2;
            const float d0 = e4m3_value(sc[r][ch] & 0x7Fu), d1 = e4m3_value((sc[r][ch] >> 8) & 0x7Fu);
            const uint4 w[4] = {dequant8(c[r][ch].x, d0), dequant8(c[r][ch].y, d0), dequant8(c[r][ch].z, d1),
                                dequant8(c[r][ch].w, d1)};
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                if (m >= M) break;
                const uint4 *xr = reinterpret_cast<const uint4 *>(xl + m * K + k);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (q >= nq) break;
                    const uint4 xv = xr[q];
                    const uint32_t xa[4] = {xv.x, xv.y, xv.z, xv.w};
                    const uint32_t wa[4] = {w[q].x, w[q].y, w[q].z, w[q].w};
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        s[m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xa[t]),
                                                               __builtin_bit_cast(bf16x2, wa[t]), s[m], false);
                }
            }
        }
        const int64_t n = n0 + r;
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            if (m >= M) break;
            const float t = wave_sum_f32(s[m]);
            if (lane == 63 && n < N) store_y<OUTF32>(Y, m * N + n, alpha * t);
        }
    }
}

size_t gemv_lds_bytes(int64_t M, int64_t K) { return (size_t)(M * K * 2); }
constexpr size_t kGemvMaxLds = 128 * 1024;

// Launch of one GEMV instantiation. Above 64 KB of dynamic LDS the kernel must be allowed the larger
// size on the current device; the attribute is set before each such launch (a cheap host call), so
// it holds on whichever device the caller has made current.
template <int MM, int CH, bool OUTF32>
hipError_t gemv_launch(dim3 grid, size_t lds, hipStream_t stream, const uint16_t *X, int M, int64_t K,
                       const uint8_t *codes, const uint8_t *scales, const float *alpha, int64_t N, void *Y) {
    if (lds > 64 * 1024) {
        const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_w4a16_gemv<MM, CH, OUTF32>),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemvMaxLds);
        if (attr != hipSuccess) return attr;
    }
    hipLaunchKernelGGL((k_w4a16_gemv<MM, CH, OUTF32>), grid, dim3(kGemvThreads), lds, stream, X, M, K, codes,
                       scales, alpha, N, Y);
    return hipGetLastError();
}

// The chunk count for MM rows of X (K <= 16384: at most 8 chunks).
template <int MM>
hipError_t gemv_dispatch(int64_t chunks, bool out_f32, dim3 grid, size_t lds, hipStream_t stream, const uint16_t *X,
                         int M, int64_t K, const uint8_t *codes, const uint8_t *scales, const float *alpha, int64_t N,
                         void *Y) {
#define NVFP4_GEMV3(CH)                                                                                          \
    return out_f32 ? gemv_launch<MM, CH, true>(grid, lds, stream, X, M, K, codes, scales, alpha, N, Y)            \
                   : gemv_launch<MM, CH, false>(grid, lds, stream, X, M, K, codes, scales, alpha, N, Y)
    if (chunks <= 2) NVFP4_GEMV3(2);
    if (chunks <= 4) NVFP4_GEMV3(4);
    NVFP4_GEMV3(8);
#undef NVFP4_GEMV3
}

// Split K when the output tiles alone give fewer than 512 work-groups (two per CU): slices of at least four
// K steps, as many as bring the count to 512, and a partial buffer of at most 1 GiB.
#ifndef NVFP4_SPLIT_TARGET
#define NVFP4_SPLIT_TARGET 512
#endif
void split_k(int64_t tiles, int64_t M, int64_t N, int64_t K, int64_t &slices, int64_t &kslice) {
    slices = 1;
    kslice = K;
    const int64_t steps = (K + kBK - 1) / kBK;
    int64_t want = (NVFP4_SPLIT_TARGET + tiles - 1) / tiles;
    want = std::min(want, steps / 4);
    while (want > 1 && want * M * N * (int64_t)sizeof(float) > ((int64_t)1 << 30)) --want;
    if (want <= 1) return;
    kslice = (steps + want - 1) / want * kBK;
    slices = (K + kslice - 1) / kslice;
}

#ifndef NVFP4_NARROW_MAX_M
#define NVFP4_NARROW_MAX_M 512
#endif

// The launch the product takes for these shapes (what launch_w4a16 runs): the kernel, the tile shape,
// the K split and the grid. Tile shape by the rows of X (timed on 4096 x 4096 weights): 128 x 64 up to
// 512 rows (four times the tiles of 256 x 128, so K is split into a quarter as many, longer slices:
// 25-30 % faster at 65 <= M <= 256); above that 256 x 128 when those tiles alone give two work-groups
// per CU, else 128 x 128 (three work-groups per CU and no split: 7 % faster at M = 1024, 16-17 % at 2048
// and 3072; 256 x 128 is 20-25 % faster than 128 x 128 once it fills the GPU, M = 4096 and 8192).
W4a16Plan plan_w4a16(int64_t M, int64_t K, int64_t N) {
    W4a16Plan p = {};
    const int64_t chunks = (K + 2047) / 2048;  // 2048 k per chunk: 32 per lane
    if (M <= kGemvMaxM && gemv_lds_bytes(M, K) <= kGemvMaxLds && chunks <= 8) {
        p.kind = kW4a16Gemv;
        const int64_t waves = (N + kGemvRows - 1) / kGemvRows;
        p.grid = (waves + kGemvThreads / 64 - 1) / (kGemvThreads / 64);
        p.chunks = chunks <= 2 ? 2 : chunks <= 4 ? 4 : 8;
        p.lds = gemv_lds_bytes(M, K);
        return p;
    }
    if (M <= kSkinnyMaxM) {
        p.kind = kW4a16Skinny;
        p.grid = (N + 15) / 16;
        p.tm = 16 * (int)((M + 15) / 16);  // rows of X the kernel is compiled for
        return p;
    }
    p.kind = kW4a16Gemm;
    const bool narrow = M <= NVFP4_NARROW_MAX_M;
    const bool tall = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN) >= 512;
    p.tm = tall && !narrow ? kBM : 128;
    p.tn = narrow ? 64 : kBN;
    p.tiles_n = (N + p.tn - 1) / p.tn;
    p.tiles = p.tiles_n * ((M + p.tm - 1) / p.tm);
    split_k(p.tiles, M, N, K, p.slices, p.kslice);
    p.grid = p.tiles * p.slices;
    if (p.slices > 1) {
        p.part_bytes = (size_t)(p.slices * M * N) * sizeof(float);
        const int64_t n = M * N;
        p.reduce_grid = std::min<int64_t>((n + kReduceThreads - 1) / kReduceThreads, 4096);
    }
    return p;
}

hipError_t launch_w4a16(const uint16_t *X, int64_t M, int64_t K, const uint8_t *codes, const uint8_t *scales,
                        const float *alpha, int64_t N, void *Y, bool out_f32, float *part, hipStream_t stream) {
    const W4a16Plan p = plan_w4a16(M, K, N);
    if (p.kind == kW4a16Gemv) {
        const dim3 grid((unsigned)p.grid);
        const int m = (int)M;
        static_assert(kGemvMaxM <= 4, "the GEMV is compiled for 1 to 4 rows of X");
        switch (M) {
            case 1: return gemv_dispatch<1>(p.chunks, out_f32, grid, p.lds, stream, X, m, K, codes, scales, alpha, N, Y);
            case 2: return gemv_dispatch<2>(p.chunks, out_f32, grid, p.lds, stream, X, m, K, codes, scales, alpha, N, Y);
            case 3: return gemv_dispatch<3>(p.chunks, out_f32, grid, p.lds, stream, X, m, K, codes, scales, alpha, N, Y);
            default: return gemv_dispatch<4>(p.chunks, out_f32, grid, p.lds, stream, X, m, K, codes, scales, alpha, N, Y);
        }
    }
    if (p.kind == kW4a16Skinny) {
        const dim3 grid((unsigned)p.grid), block(kSkinnyThreads);
        const int m = (int)M;
#define NVFP4_SKINNY(MT)                                                                                          \
    do {                                                                                                          \
        if (out_f32)                                                                                              \
            hipLaunchKernelGGL((k_w4a16_skinny<MT, true>), grid, block, 0, stream, X, m, K, codes, scales, alpha, N,  \
                               Y);                                                                                \
        else                                                                                                      \
            hipLaunchKernelGGL((k_w4a16_skinny<MT, false>), grid, block, 0, stream, X, m, K, codes, scales, alpha,   \
                               N, Y);                                                                             \
    } while (0)
        switch (p.tm / 16) {
            case 1: NVFP4_SKINNY(1); break;
            case 2: NVFP4_SKINNY(2); break;
            case 3: NVFP4_SKINNY(3); break;
            default: NVFP4_SKINNY(4); break;
        }
#undef NVFP4_SKINNY
        return hipGetLastError();
    }
    if (p.slices > 1 && !part) return hipErrorInvalidValue;
    float *const pp = p.slices > 1 ? part : nullptr;
    const dim3 grid((unsigned)p.grid), block(kGemmThreads);
#define NVFP4_GEMM(TM, TN)                                                                                    \
    do {                                                                                                      \
        if (out_f32)                                                                                          \
            hipLaunchKernelGGL((k_w4a16_gemm<TM, TN, true>), grid, block, 0, stream, X, M, K, codes, scales, alpha, \
                               N, Y, (unsigned)p.tiles_n, (unsigned)p.tiles, p.kslice, pp);                     \
        else                                                                                                  \
            hipLaunchKernelGGL((k_w4a16_gemm<TM, TN, false>), grid, block, 0, stream, X, M, K, codes, scales,      \
                               alpha, N, Y, (unsigned)p.tiles_n, (unsigned)p.tiles, p.kslice, pp);              \
    } while (0)
    if (p.tn == 64)
        NVFP4_GEMM(128, 64);
    else if (p.tm == 128)
        NVFP4_GEMM(128, 128);
    else
        NVFP4_GEMM(256, 128);
#undef NVFP4_GEMM
    hipError_t err = hipGetLastError();
    if (err == hipSuccess && p.slices > 1) {
        const int64_t n = M * N;
        const dim3 rgrid((unsigned)p.reduce_grid);
        if (out_f32)
            hipLaunchKernelGGL(k_w4a16_reduce<true>, rgrid, dim3(kReduceThreads), 0, stream, pp, (int)p.slices, n,
                               alpha, Y);
        else
            hipLaunchKernelGGL(k_w4a16_reduce<false>, rgrid, dim3(kReduceThreads), 0, stream, pp, (int)p.slices, n,
                               alpha, Y);
        err = hipGetLastError();
    }
    return err;
}

}  // namespace nvfp4
