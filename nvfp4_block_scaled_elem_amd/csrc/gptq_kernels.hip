// GPTQ with the FourOverSix block scales fixed first, on gfx950.
//
// The FourOverSix write-up ("SOAR 周冠军笔记 07", section 03) fixes every block's scale, with its M = 6 /
// M = 4 choice, before GPTQ's weight iterations run. GPTQ (Frantar et al., 2022) then quantises the
// columns in order. Each column's error is spread over the later columns so that, given the columns
// already fixed, the later weights minimise the error weighted by the input second moment H (damped,
// dead inputs removed).
//
// Published form: U = the upper Cholesky factor of H^-1. For column j, the error d_j = (w~_j - q_j) / U_jj
// and w~_k -= d_j U_jk for k > j.
//
// Form used here: the same result without an inverse. Let V = U^-1, the upper-triangular factor with
// H = V V^T, and e = w - q the errors against the original (dead-zeroed) weights. Expanding the
// updates gives d U = e, so d = e V and
//     w~_j = w_j + (sum_{i<j} e_i V_ij) / V_jj.
// V is the lower Cholesky factor of the reversed matrix P H P (P reverses the index), read back
// reversed: V_ij = L~[K-1-i][K-1-j].
//
// Kernels, all binary64:
//   k_gptq_prep     dead inputs (zero diagonal) and the damping lambda = percdamp * mean(diag)
//   k_gptq_reverse  A = P (H with dead diagonals 1, + lambda I) P, lower triangle
//   k_chol_diag,    blocked right-looking Cholesky of A in place, panels of 64 columns: the diagonal
//   k_chol_trsm,    block (one work-group), the rows below it (one lane per row), then the trailing
//   k_chol_update   lower triangle (64 x 64 fp64 tiles)
//   k_gptq_cols     columns [b0, b0 + 64): one thread per weight row walks them in order (target,
//                   E2M1 code, error e_j)
//   k_gptq_update   S[:, k] += sum over the block of e_i V_ik for every later column k (fp64 tiles)
// S holds sum_{i<b0} e_i V_ik for the columns not yet reached. Block 0's update writes it, so it needs no
// clearing.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "codec.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

constexpr int kPanel = 64;           // Cholesky panel width = GPTQ column block
constexpr int kLd = kPanel + 1;      // LDS row stride in doubles: rows land on different banks
constexpr int kTile = 64;            // output tile of the fp64 update kernels (64 x 64, 4 x 4 per thread)
constexpr int kPrepThreads = 1024;

__global__ __launch_bounds__(kPrepThreads) void k_gptq_prep(const double *__restrict__ H, int64_t K, double percdamp,
                                                            double *__restrict__ damp, uint8_t *__restrict__ dead,
                                                            int *__restrict__ flag) {
    __shared__ double part[kPrepThreads];
    double s = 0.0;
    for (int64_t j = threadIdx.x; j < K; j += kPrepThreads) {
        const double h = H[j * K + j];
        const bool d = h == 0.0;
        dead[j] = d;
        s += d ? 1.0 : h;
    }
    part[threadIdx.x] = s;
    __syncthreads();
    for (int w = kPrepThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        damp[0] = percdamp * (part[0] / (double)K);
        flag[0] = 0;
    }
}

// A[a][c] = H[K-1-a][K-1-c] for c <= a (H's upper triangle, read row by row), diagonal modified.
__global__ __launch_bounds__(256) void k_gptq_reverse(const double *__restrict__ H, int64_t K,
                                                      const double *__restrict__ damp,
                                                      const uint8_t *__restrict__ dead, double *__restrict__ A) {
    const int64_t a = blockIdx.y;
    const int64_t i = K - 1 - a;
    const double lam = damp[0];
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c <= a; c += (int64_t)gridDim.x * 256) {
        const int64_t j = K - 1 - c;  // j >= i
        double v = H[i * K + j];
        if (c == a) v = (dead[i] ? 1.0 : v) + lam;
        A[a * K + c] = v;
    }
}

// Diagonal block of panel [p0, p0 + nb), factored in LDS by one work-group and written back. Padded to
// 64 columns with an identity so that the loops have fixed bounds. A pivot that is not positive and
// finite sets *flag.
__global__ __launch_bounds__(256) void k_chol_diag(double *__restrict__ A, int64_t K, int64_t p0,
                                                   int *__restrict__ flag) {
    __shared__ double L[kPanel * kLd];
    const int nb = (int)min<int64_t>(kPanel, K - p0);
    const int tid = threadIdx.x;
    for (int idx = tid; idx < kPanel * kPanel; idx += 256) {
        const int r = idx / kPanel, c = idx % kPanel;
        double v = r == c ? 1.0 : 0.0;
        if (r < nb && c <= r) v = A[(p0 + r) * K + p0 + c];
        L[r * kLd + c] = v;
    }
    __syncthreads();
    // column c: every row r >= c (lane r of wave 0) computes the pivot from row c's finished entries,
    // then its own entry of column c
    bool bad = false;
    for (int c = 0; c < kPanel; ++c) {
        if (tid >= c && tid < kPanel) {
            double s = L[c * kLd + c];
            for (int t = 0; t < c; ++t) s -= L[c * kLd + t] * L[c * kLd + t];
            if (!(s > 0.0) || !(s < INFINITY)) bad = true;
            const double d = sqrt(s);
            if (tid == c) {
                L[c * kLd + c] = d;
            } else {
                double x = L[tid * kLd + c];
                for (int t = 0; t < c; ++t) x -= L[tid * kLd + t] * L[c * kLd + t];
                L[tid * kLd + c] = x / d;
            }
        }
        __syncthreads();
    }
    if (bad && tid < nb) flag[0] = 1;
    for (int idx = tid; idx < nb * nb; idx += 256) {
        const int r = idx / nb, c = idx % nb;
        if (c <= r) A[(p0 + r) * K + p0 + c] = L[r * kLd + c];
    }
}

// Rows below the diagonal block of panel [p0, p0 + nb), 64 per work-group (one wave): L21 = A21 L11^-T
// by forward substitution, one row per lane, the row kept in LDS (L11 factored by k_chol_diag).
constexpr int kTrsmRows = 64;
__global__ __launch_bounds__(kTrsmRows) void k_chol_trsm(double *__restrict__ A, int64_t K, int64_t p0) {
    __shared__ double L[kPanel * kLd], X[kTrsmRows * kLd];
    const int nb = (int)min<int64_t>(kPanel, K - p0);
    const int tid = threadIdx.x;
    const int64_t r0 = p0 + nb + (int64_t)blockIdx.x * kTrsmRows;
    for (int idx = tid; idx < kPanel * kPanel; idx += kTrsmRows) {
        const int r = idx / kPanel, c = idx % kPanel;
        double v = r == c ? 1.0 : 0.0;
        if (r < nb && c <= r) v = A[(p0 + r) * K + p0 + c];
        L[r * kLd + c] = v;
        X[r * kLd + c] = (r0 + r < K && c < nb) ? A[(r0 + r) * K + p0 + c] : 0.0;
    }
    __syncthreads();
    double *x = X + tid * kLd;
    for (int c = 0; c < nb; ++c) {
        double v = x[c];
        for (int t = 0; t < c; ++t) v -= x[t] * L[c * kLd + t];
        x[c] = v / L[c * kLd + c];
    }
    __syncthreads();
    for (int idx = tid; idx < kTrsmRows * kPanel; idx += kTrsmRows) {
        const int r = idx / kPanel, c = idx % kPanel;
        if (r0 + r < K && c < nb) A[(r0 + r) * K + p0 + c] = X[r * kLd + c];
    }
}

// Trailing update after panel [p0, p1): A[i][j] -= sum_t A[i][p0+t] A[j][p0+t] for p1 <= j <= i < K.
// 64 x 64 tiles of the lower triangle (tiles above it exit at once).
__global__ __launch_bounds__(256) void k_chol_update(double *__restrict__ A, int64_t K, int64_t p0, int nb) {
    const int ti = blockIdx.y, tj = blockIdx.x;
    if (tj > ti) return;
    __shared__ double Pi[kTile * kLd], Pj[kTile * kLd];
    const int64_t p1 = p0 + nb, i0 = p1 + (int64_t)ti * kTile, j0 = p1 + (int64_t)tj * kTile;
    const int tid = threadIdx.x;
    for (int idx = tid; idx < kTile * kPanel; idx += 256) {
        const int r = idx / kPanel, t = idx % kPanel;
        Pi[r * kLd + t] = (i0 + r < K && t < nb) ? A[(i0 + r) * K + p0 + t] : 0.0;
        Pj[r * kLd + t] = (j0 + r < K && t < nb) ? A[(j0 + r) * K + p0 + t] : 0.0;
    }
    __syncthreads();
    const int ty = tid / 16, tx = tid % 16;
    double acc[4][4] = {};
    for (int t = 0; t < kPanel; ++t) {
        double a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            a[u] = Pi[(ty + 16 * u) * kLd + t];
            b[u] = Pj[(tx + 16 * u) * kLd + t];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[u][v] += a[u] * b[v];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t i = i0 + ty + 16 * u, j = j0 + tx + 16 * v;
            if (i < K && j <= i) A[i * K + j] -= acc[u][v];
        }
}

__device__ __forceinline__ double load_w(const void *W, bool f32, int64_t idx) {
    if (f32) return (double)static_cast<const float *>(W)[idx];
    return (double)__uint_as_float((uint32_t) static_cast<const uint16_t *>(W)[idx] << 16);
}

// E2M1 index of the nearest magnitude to a >= 0 (ties to the even index, 6 beyond 5).
__device__ __forceinline__ uint32_t e2m1_index64(double a) {
    return (uint32_t)(a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5.0);
}

// Columns [b0, b0 + nb) of every row: one thread per row, columns in order.
__global__ __launch_bounds__(256) void k_gptq_cols(const void *__restrict__ W, bool f32, int64_t R, int64_t K,
                                                   int64_t b0, int nb, const double *__restrict__ A,
                                                   const uint8_t *__restrict__ dead,
                                                   const uint8_t *__restrict__ scales,
                                                   const float *__restrict__ alpha_p,
                                                   const double *__restrict__ S, double *__restrict__ E,
                                                   uint8_t *__restrict__ codes) {
    __shared__ double V[kPanel * kLd];  // V[i][j] = V_(b0+i, b0+j) for i <= j, identity padding
    const int tid = threadIdx.x;
    for (int idx = tid; idx < kPanel * kPanel; idx += 256) {
        const int i = idx / kPanel, j = idx % kPanel;
        double v = i == j ? 1.0 : 0.0;
        if (j < nb && i <= j) v = A[(K - 1 - b0 - i) * K + (K - 1 - b0 - j)];
        V[i * kLd + j] = v;
    }
    __syncthreads();
    const int64_t r = (int64_t)blockIdx.x * 256 + tid;
    if (r >= R) return;
    const float alpha = *alpha_p;
    double e[kPanel];
    uint32_t packed[kPanel / 8] = {};
#pragma unroll
    for (int g = 0; g < kPanel / 16; ++g) {
        if (16 * g >= nb) break;
        const int64_t col16 = b0 + 16 * g;
        const float s32 = alpha * e4m3_value(scales[r * (K / 16) + col16 / 16]);  // fl32(alpha * Delta)
        const double s = (double)s32;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int j = 16 * g + u;
            const int64_t col = b0 + j;
            const double w = dead[col] ? 0.0 : load_w(W, f32, r * K + col);
            double acc = b0 > 0 ? S[r * K + col] : 0.0;
#pragma unroll
            for (int i = 0; i < j; ++i) acc += e[i] * V[i * kLd + j];
            const double t = w + acc / V[j * kLd + j];
            uint32_t code = 0;
            double deq = 0.0;
            if (s > 0.0) {
                const double x = t / s;
                const uint32_t idx = e2m1_index64(fabs(x));
                const bool neg = x < 0.0 && idx > 0;
                code = idx | (neg ? 8u : 0u);
                const double mag = idx < 4 ? 0.5 * idx : (idx == 7 ? 6.0 : (double)(idx - 2));  // {0,..,1.5}, 2, 3, 4, 6
                deq = (neg ? -mag : mag) * s;
            }
            e[j] = w - deq;
            packed[j / 8] |= code << (4 * (j % 8));
        }
    }
#pragma unroll
    for (int j = 0; j < kPanel; ++j)
        if (j < nb) E[r * kPanel + j] = e[j];
    uint32_t *dst = reinterpret_cast<uint32_t *>(codes + r * (K / 2) + b0 / 2);  // 8-byte aligned: b0 % 16 == 0
#pragma unroll
    for (int q = 0; q < kPanel / 8; ++q)
        if (8 * q < nb) dst[q] = packed[q];
}

// S[r][k] (=, or += after block 0) sum_{i < nb} E[r][i] V_(b0+i, k) for k in [b0 + nb, K), 64 x 64 tiles.
__global__ __launch_bounds__(256) void k_gptq_update(const double *__restrict__ E, const double *__restrict__ A,
                                                     double *__restrict__ S, int64_t R, int64_t K, int64_t b0,
                                                     int nb) {
    __shared__ double Et[kTile * kLd], Vt[kTile * kLd];
    const int64_t r0 = (int64_t)blockIdx.y * kTile, k0 = b0 + nb + (int64_t)blockIdx.x * kTile;
    const int tid = threadIdx.x;
    for (int idx = tid; idx < kTile * kPanel; idx += 256) {
        const int a = idx / kPanel, i = idx % kPanel;
        Et[a * kLd + i] = (r0 + a < R && i < nb) ? E[(r0 + a) * kPanel + i] : 0.0;
    }
    for (int idx = tid; idx < kPanel * kTile; idx += 256) {
        const int i = idx / kTile, kk = idx % kTile;  // consecutive threads: consecutive (descending) A columns
        Vt[kk * kLd + i] = (k0 + kk < K && i < nb) ? A[(K - 1 - b0 - i) * K + (K - 1 - k0 - kk)] : 0.0;
    }
    __syncthreads();
    const int ty = tid / 16, tx = tid % 16;
    double acc[4][4] = {};
    for (int i = 0; i < kPanel; ++i) {
        double a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            a[u] = Et[(ty + 16 * u) * kLd + i];
            b[u] = Vt[(tx + 16 * u) * kLd + i];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[u][v] += a[u] * b[v];
    }
    const bool first = b0 == 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t r = r0 + ty + 16 * u, k = k0 + tx + 16 * v;
            if (r < R && k < K) S[r * K + k] = first ? acc[u][v] : S[r * K + k] + acc[u][v];
        }
}

// A failed factorisation (a pivot not positive and finite): alpha = NaN and every code 0. n8 = the
// number of 8-byte groups of codes (rows * cols / 2 bytes, a multiple of 8).
__global__ __launch_bounds__(256) void k_gptq_finish(const int *__restrict__ flag, int64_t n8,
                                                     uint8_t *__restrict__ codes, float *__restrict__ alpha) {
    if (flag[0] == 0) return;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n8) reinterpret_cast<uint2 *>(codes)[i] = make_uint2(0u, 0u);
    if (i == 0) alpha[0] = __builtin_nanf("");
}

}  // namespace

size_t gptq_workspace_bytes(int64_t R, int64_t K) {
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    return up((size_t)K * K * 8) + up((size_t)R * K * 8) + up((size_t)R * kPanel * 8) + up((size_t)K) + 256 +
           workspace_bytes(R * K / 16, NVFP4_MODE_FOUR_OVER_SIX);
}

hipError_t launch_gptq(const void *W, bool f32, int64_t R, int64_t K, const double *H, double percdamp,
                       uint8_t *codes, uint8_t *scales, float *alpha, void *ws_base, hipStream_t stream) {
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    char *p = static_cast<char *>(ws_base);
    double *A = reinterpret_cast<double *>(p);
    p += up((size_t)K * K * 8);
    double *S = reinterpret_cast<double *>(p);
    p += up((size_t)R * K * 8);
    double *E = reinterpret_cast<double *>(p);
    p += up((size_t)R * kPanel * 8);
    uint8_t *dead = reinterpret_cast<uint8_t *>(p);
    p += up((size_t)K);
    double *damp = reinterpret_cast<double *>(p);
    int *flag = reinterpret_cast<int *>(p + 8);
    p += 256;
    const int64_t nblk = R * K / 16;
    const Workspace q = carve(p, nblk);

    // the FourOverSix frame: scales and alpha (and codes, overwritten below)
    const int64_t n = R * K;
    const int ga = amax_groups(n * (f32 ? 4 : 2) / 16);
    hipError_t err = launch_amax(W, f32, n, q.amax_part, ga, nullptr, stream);
    if (err == hipSuccess)
        err = launch_quant(W, f32, true, nblk, q.amax_part, ga, codes, scales, alpha, nullptr, nullptr, q.m4_part,
                           stream);
    if (err != hipSuccess) return err;

    hipLaunchKernelGGL(k_gptq_prep, dim3(1), dim3(kPrepThreads), 0, stream, H, K, percdamp, damp, dead, flag);
    hipLaunchKernelGGL(k_gptq_reverse, dim3((unsigned)((K + 255) / 256), (unsigned)K), dim3(256), 0, stream, H, K,
                       damp, dead, A);
    for (int64_t p0 = 0; p0 < K; p0 += kPanel) {
        const int nb = (int)std::min<int64_t>(kPanel, K - p0);
        const int64_t below = K - p0 - nb;
        hipLaunchKernelGGL(k_chol_diag, dim3(1), dim3(256), 0, stream, A, K, p0, flag);
        if (below > 0) {
            hipLaunchKernelGGL(k_chol_trsm, dim3((unsigned)((below + kTrsmRows - 1) / kTrsmRows)), dim3(kTrsmRows), 0,
                               stream, A, K, p0);
            const unsigned t = (unsigned)((below + kTile - 1) / kTile);
            hipLaunchKernelGGL(k_chol_update, dim3(t, t), dim3(256), 0, stream, A, K, p0, nb);
        }
    }
    for (int64_t b0 = 0; b0 < K; b0 += kPanel) {
        const int nb = (int)std::min<int64_t>(kPanel, K - b0);
        hipLaunchKernelGGL(k_gptq_cols, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, stream, W, f32, R, K, b0,
                           nb, A, dead, scales, alpha, S, E, codes);
        const int64_t later = K - b0 - nb;
        if (later > 0)
            hipLaunchKernelGGL(k_gptq_update,
                               dim3((unsigned)((later + kTile - 1) / kTile), (unsigned)((R + kTile - 1) / kTile)),
                               dim3(256), 0, stream, E, A, S, R, K, b0, nb);
    }
    const int64_t n8 = R * K / 16;
    hipLaunchKernelGGL(k_gptq_finish, dim3((unsigned)std::max<int64_t>(1, (n8 + 255) / 256)), dim3(256), 0, stream,
                       flag, n8, codes, alpha);
    return hipGetLastError();
}

}  // namespace nvfp4
