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
// Two kernels:
//   k_w4a16_gemm: 128 x 128 output tile per work-group (4 waves, 64 x 64 each as 2 x 2 tiles of
//     v_mfma_f32_32x32x16_bf16), K in steps of 64 through LDS: the X tile is copied, the weight tile is
//     decoded to bf16 (codes -> binary32 q, times Delta, high half) as it is stored.
//   k_w4a16_gemv: M <= 4 (decoding one token per row, say): bound by reading the 0.5625 bytes per weight
//     once; X sits in LDS, each wave takes whole rows n, each lane 32 consecutive k at a time, and the
//     row sum is a DPP wave reduction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.hpp"
#include "launch.hpp"

namespace nvfp4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmThreads = 256;
constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLdsStride = kBK + 8;  // bf16 per LDS row: the padding spreads rows over the banks

// 8 codes (one dword) and their scale value -> 8 dequantised weights (without alpha) as bf16 pairs.
__device__ __forceinline__ uint4 dequant8(uint32_t c, float dv) {
    const f32x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
    const f32x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
    const f32x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
    const f32x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
    // q*dv is exact and has at most 6 significant bits: its high 16 bits are the bf16 value
    auto pair = [&](float a, float b) {
        return (__float_as_uint(a * dv) >> 16) | (__float_as_uint(b * dv) & 0xFFFF0000u);
    };
    return make_uint4(pair(q0.x, q0.y), pair(q1.x, q1.y), pair(q2.x, q2.y), pair(q3.x, q3.y));
}

// Round binary32 to bf16 (nearest, ties to even; the values here are finite).
__device__ __forceinline__ uint16_t to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <bool OUTF32>
__device__ __forceinline__ void store_y(void *Y, int64_t idx, float v) {
    if (OUTF32)
        static_cast<float *>(Y)[idx] = v;
    else
        static_cast<uint16_t *>(Y)[idx] = to_bf16(v);
}

template <bool OUTF32>
__global__ __launch_bounds__(kGemmThreads) void k_w4a16_gemm(const uint16_t *__restrict__ X, int64_t M, int64_t K,
                                                             const uint8_t *__restrict__ codes,
                                                             const uint8_t *__restrict__ scales,
                                                             const float *__restrict__ alpha_p, int64_t N,
                                                             void *__restrict__ Y) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[kBM * kLdsStride];
    __shared__ __attribute__((aligned(16))) uint16_t ws[kBN * kLdsStride];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;  // the wave's 64 x 64 corner of the tile
    f32x16 acc[2][2] = {};

    for (int64_t k0 = 0; k0 < K; k0 += kBK) {
        // X tile: 128 rows x 64 k, 4 x 16 bytes per thread (rows past M and k past K read as zeros)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int idx = tid + p * kGemmThreads;  // 0..1023: row idx / 8, 8-element group idx % 8
            const int r = idx >> 3, g = idx & 7;
            const int64_t m = m0 + r, k = k0 + 8 * g;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (m < M && k < K) v = *reinterpret_cast<const uint4 *>(X + m * K + k);  // K % 16 == 0
            *reinterpret_cast<uint4 *>(&xs[r * kLdsStride + 8 * g]) = v;
        }
        // weight tile: 128 rows n x 64 k = 32 bytes of codes per row; a thread decodes 16 bytes (32 k)
        {
            const int r = tid >> 1, h = tid & 1;
            const int64_t n = n0 + r, k = k0 + 32 * h;
            uint4 c = make_uint4(0u, 0u, 0u, 0u);
            float d0 = 0.0f, d1 = 0.0f;
            if (n < N && k < K) {
                const int64_t e = n * K + k;  // element index, a multiple of 32
                if (k + 32 <= K) {
                    c = *reinterpret_cast<const uint4 *>(codes + e / 2);
                } else {  // K % 32 == 16: the last 16 k of the row
                    const uint2 c2 = *reinterpret_cast<const uint2 *>(codes + e / 2);
                    c = make_uint4(c2.x, c2.y, 0u, 0u);
                }
                d0 = e4m3_value(scales[e / 16] & 0x7Fu);
                if (k + 16 < K) d1 = e4m3_value(scales[e / 16 + 1] & 0x7Fu);
            }
            uint16_t *dst = &ws[r * kLdsStride + 32 * h];
            *reinterpret_cast<uint4 *>(dst) = dequant8(c.x, d0);
            *reinterpret_cast<uint4 *>(dst + 8) = dequant8(c.y, d0);
            *reinterpret_cast<uint4 *>(dst + 16) = dequant8(c.z, d1);
            *reinterpret_cast<uint4 *>(dst + 24) = dequant8(c.w, d1);
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 16) {
            bf16x8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                // A operand: row (lane % 32) of the 32-row tile, k = 8 * (lane / 32) .. + 7
                a[i] = *reinterpret_cast<const bf16x8 *>(
                    &xs[(wm + 32 * i + (lane & 31)) * kLdsStride + kk + 8 * (lane >> 5)]);
                // B operand: column n = lane % 32 of the tile, the same k
                b[i] = *reinterpret_cast<const bf16x8 *>(
                    &ws[(wn + 32 * i + (lane & 31)) * kLdsStride + kk + 8 * (lane >> 5)]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
    // D layout: element e of lane l is row 8 * (e / 4) + 4 * (l / 32) + e % 4, column l % 32
    const float alpha = *alpha_p;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t m = m0 + wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int64_t n = n0 + wn + 32 * j + (lane & 31);
                if (m < M && n < N) store_y<OUTF32>(Y, m * N + n, alpha * acc[i][j][e]);
            }
}

// ------------------------------------------------------------------------------------------- GEMV

constexpr int kGemvThreads = 256;
constexpr int kGemvMaxM = 4;

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

// X (M rows, K <= the LDS budget) is copied to LDS once per work-group; each wave then takes rows
// n = global wave, + total waves, ...; lane l handles k = 32 * (l + 64 i) .. + 31 (16 bytes of codes,
// two scales) and accumulates M dot products in fp32.
template <int MM, bool OUTF32>
__global__ __launch_bounds__(kGemvThreads) void k_w4a16_gemv(const uint16_t *__restrict__ X, int64_t K,
                                                             const uint8_t *__restrict__ codes,
                                                             const uint8_t *__restrict__ scales,
                                                             const float *__restrict__ alpha_p, int64_t N,
                                                             void *__restrict__ Y) {
    extern __shared__ __attribute__((aligned(16))) uint16_t xl[];  // [MM][K]
    const int tid = threadIdx.x, lane = tid & 63;
    for (int64_t i = tid; i < MM * K / 8; i += kGemvThreads)
        reinterpret_cast<uint4 *>(xl)[i] = reinterpret_cast<const uint4 *>(X)[i];
    __syncthreads();
    const float alpha = *alpha_p;
    const int64_t waves = (int64_t)gridDim.x * (kGemvThreads / 64);
    for (int64_t n = (int64_t)blockIdx.x * (kGemvThreads / 64) + (tid >> 6); n < N; n += waves) {
        float s[MM];
#pragma unroll
        for (int m = 0; m < MM; ++m) s[m] = 0.0f;
        for (int64_t k = 32 * lane; k < K; k += 32 * 64) {
            const int64_t e = n * K + k;
            const bool whole = k + 32 <= K;  // else the row's last 16 k (K % 32 == 16)
            uint4 c;
            float d1 = 0.0f;
            if (whole) {
                c = *reinterpret_cast<const uint4 *>(codes + e / 2);
                d1 = e4m3_value(scales[e / 16 + 1] & 0x7Fu);
            } else {
                const uint2 c2 = *reinterpret_cast<const uint2 *>(codes + e / 2);
                c = make_uint4(c2.x, c2.y, 0u, 0u);
            }
            const float d0 = e4m3_value(scales[e / 16] & 0x7Fu);
            const uint4 w[4] = {dequant8(c.x, d0), dequant8(c.y, d0), dequant8(c.z, d1), dequant8(c.w, d1)};
            const int nq = whole ? 4 : 2;
#pragma unroll
            for (int m = 0; m < MM; ++m) {
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
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            const float t = wave_sum_f32(s[m]);
            if (lane == 63) store_y<OUTF32>(Y, m * N + n, alpha * t);
        }
    }
}

size_t gemv_lds_bytes(int64_t M, int64_t K) { return (size_t)(M * K * 2); }

hipError_t launch_w4a16(const uint16_t *X, int64_t M, int64_t K, const uint8_t *codes, const uint8_t *scales,
                        const float *alpha, int64_t N, void *Y, bool out_f32, hipStream_t stream) {
    if (M <= kGemvMaxM && gemv_lds_bytes(M, K) <= 64 * 1024) {
        const int64_t blocks = (N + (kGemvThreads / 64) - 1) / (kGemvThreads / 64);
        const dim3 grid((unsigned)(blocks < 1024 ? blocks : 1024)), block(kGemvThreads);
        const size_t lds = gemv_lds_bytes(M, K);
#define NVFP4_GEMV(MM)                                                                                            \
    do {                                                                                                          \
        if (out_f32)                                                                                              \
            hipLaunchKernelGGL((k_w4a16_gemv<MM, true>), grid, block, lds, stream, X, K, codes, scales, alpha, N, Y); \
        else                                                                                                      \
            hipLaunchKernelGGL((k_w4a16_gemv<MM, false>), grid, block, lds, stream, X, K, codes, scales, alpha, N, Y); \
    } while (0)
        switch (M) {
            case 1: NVFP4_GEMV(1); break;
            case 2: NVFP4_GEMV(2); break;
            case 3: NVFP4_GEMV(3); break;
            default: NVFP4_GEMV(4); break;
        }
#undef NVFP4_GEMV
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM)), block(kGemmThreads);
    if (out_f32)
        hipLaunchKernelGGL(k_w4a16_gemm<true>, grid, block, 0, stream, X, M, K, codes, scales, alpha, N, Y);
    else
        hipLaunchKernelGGL(k_w4a16_gemm<false>, grid, block, 0, stream, X, M, K, codes, scales, alpha, N, Y);
    return hipGetLastError();
}

}  // namespace nvfp4
