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
//   k_chol_trsm,    block (one work-group, 4 x 4 register tiles), the rows below it (a wave per 16 rows), then
//   k_chol_update   the trailing lower triangle (64 x 64 tiles on the fp64 matrix cores); the update's first
//                   work-group also factors the next diagonal block, so only the first has its own launch
//   k_gptq_pack_v   V's diagonal 64 x 64 blocks, packed contiguously for the sweep
//   k_gptq_cols     columns [b0, b0 + 64), a wave per 16 rows, in order (target, E2M1 code, error e_j),
//                   each column's errors folded into the block's later columns at once
//   k_gptq_update   S[:, k] += sum over a run of blocks of e_i V_ik for later columns k (fp64 matrix
//                   cores, 64 x 64 tiles): after each block for the rest of its group of 4 blocks, after a
//                   group for every column beyond it
//   k_gptq_finish   a failed factorisation (a pivot that is not positive and finite): alpha = NaN, codes 0
// S holds sum_{i<b0} e_i V_ik for the columns not yet reached. The updates whose reduction starts at column 0
// write it, so it needs no clearing.
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
constexpr int kSuper = 256;          // column blocks are grouped by 4: S beyond a group is updated once per group

// A 64 x 64 tile of doubles into LDS by 256 threads: element (r, c) (c fastest across threads) is
// src[off(r, c)] where ok(r, c), else fill(r, c), stored at lds[pos(r, c)]. All 16 loads of a thread
// are issued before any is waited for (a masked element reads src[0], which exists, and is discarded).
template <class Off, class Ok, class Fill, class Pos>
__device__ __forceinline__ void load_tile(double *lds, const double *__restrict__ src, Off off, Ok ok, Fill fill,
                                          Pos pos) {
    double v[16];
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int idx = threadIdx.x + 256 * it, r = idx >> 6, c = idx & 63;
        v[it] = src[ok(r, c) ? off(r, c) : 0];
    }
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int idx = threadIdx.x + 256 * it, r = idx >> 6, c = idx & 63;
        lds[pos(r, c)] = ok(r, c) ? v[it] : fill(r, c);
    }
}

// The same for a 64-thread work-group (one wave): all 64 loads of a lane issued before any is used.
template <class Off, class Ok, class Fill>
__device__ __forceinline__ void load_tile_wave(double *lds, const double *__restrict__ src, Off off, Ok ok,
                                               Fill fill) {
    const int c = threadIdx.x;
    double v[kPanel];
#pragma unroll
    for (int r = 0; r < kPanel; ++r) v[r] = src[ok(r, c) ? off(r, c) : 0];
#pragma unroll
    for (int r = 0; r < kPanel; ++r) lds[r * kLd + c] = ok(r, c) ? v[r] : fill(r, c);
}

// x of lane k (0..3) of this lane's quad, by DPP quad_perm [k, k, k, k] (a few cycles; a shuffle goes
// through the LDS crossbar). k must fold to a constant after unrolling.
template <int Q>
__device__ __forceinline__ double quad_bcast_k(double x) {
    constexpr int ctrl = Q | (Q << 2) | (Q << 4) | (Q << 6);
    const unsigned long long u = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_mov_dpp((int)(unsigned)u, ctrl, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(unsigned)(u >> 32), ctrl, 0xF, 0xF, false);
    return __longlong_as_double(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ double quad_bcast(double x, int k) {
    switch (k) {
        case 0: return quad_bcast_k<0>(x);
        case 1: return quad_bcast_k<1>(x);
        case 2: return quad_bcast_k<2>(x);
        default: return quad_bcast_k<3>(x);
    }
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// One 64-deep step of a 64 x 64 output tile on the fp64 matrix cores: out[r][c] += sum_i P[r][i] Q[c][i]
// with P and Q staged in LDS (row stride kLd). Wave w computes the 32 x 32 quadrant (wm, wn) =
// (32 (w / 2), 32 (w % 2)) as 2 x 2 tiles of v_mfma_f64_16x16x4f64, whose lane layout (checked on the
// device with integer inputs) is: lane l holds A[l % 16][l / 16] and B[l / 16][l % 16], and register q of
// the result holds D[4 q + l / 16][l % 16].
__device__ __forceinline__ void mfma_tile64(const double *P, const double *Q, f64x4 (&acc)[2][2]) {
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = 32 * (w >> 1), wn = 32 * (w & 1);
#pragma unroll 4
    for (int kk = 0; kk < kPanel; kk += 4) {
        double a[2], b[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) a[m] = P[(wm + 16 * m + (l & 15)) * kLd + kk + (l >> 4)];
#pragma unroll
        for (int n = 0; n < 2; ++n) b[n] = Q[(wn + 16 * n + (l & 15)) * kLd + kk + (l >> 4)];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int n = 0; n < 2; ++n) acc[m][n] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[m], b[n], acc[m][n], 0, 0, 0);
    }
}

// Row and column (within the 64 x 64 tile) of result register q of tile (m, n) in this lane.
__device__ __forceinline__ int tile_row(int m, int q) {
    return 32 * ((threadIdx.x >> 6) >> 1) + 16 * m + 4 * q + ((threadIdx.x & 63) >> 4);
}
__device__ __forceinline__ int tile_col(int n) { return 32 * ((threadIdx.x >> 6) & 1) + 16 * n + (threadIdx.x & 15); }

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

// Factors the diagonal block of panel [p0, p0 + nb) with the 256 threads of a work-group (padded to 64 with
// an identity). T is the block's lower triangle in LDS (row stride kLd). Thread (tx, ty) = (tid / 16,
// tid % 16) holds rows ty + 16u and columns tx + 16v (u, v < 4) in registers, so the 16 threads of a column
// are lanes of one wave. Column c: its holders take the pivot from its lane by shuffle, scale the column
// and publish it (a double-buffered LDS slot, one barrier); then every thread subtracts l_rc l_tc from its
// entries in later columns. Entries above the diagonal are computed and discarded. The factor is written
// back into A and, packed column-major with zeros above the diagonal, to Lp for the row solve. A pivot that
// is not positive and finite sets *flag.
__device__ __forceinline__ void chol_diag_block(const double *T, int nb, double *__restrict__ A, int64_t K,
                                                int64_t p0, double *__restrict__ Lp, int *__restrict__ flag) {
    __shared__ double col[2][kPanel];
    const int tid = threadIdx.x, tx = tid >> 4, ty = tid & 15;
    double a[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = ty + 16 * u, t = tx + 16 * v;
            a[u][v] = r < nb && t <= r ? T[r * kLd + t] : (r == t ? 1.0 : 0.0);
        }
    bool bad = false;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
        for (int cc = 0; cc < 16; ++cc) {
            const int c = 16 * cb + cc;
            // a_cc sits in thread (tx, ty) = (cc, cc), lane 16 (cc % 4) + cc of the column's wave
            const double s = __shfl(a[cb][cb], 16 * (cc & 3) + cc);
            if (tx == cc) {
                if (ty == cc && (!(s > 0.0) || !(s < INFINITY))) bad = true;
                const double d = sqrt(s);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int r = ty + 16 * u;
                    const double l = r == c ? d : a[u][cb] / d;  // l_rc below the diagonal
                    a[u][cb] = l;
                    col[c & 1][r] = l;
                }
            }
            __syncthreads();
            const double *lc = col[c & 1];
            double lr[4], lt[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) lr[u] = lc[ty + 16 * u];
#pragma unroll
            for (int v = 0; v < 4; ++v) lt[v] = lc[tx + 16 * v];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const double m = tx + 16 * v > c ? -lt[v] : 0.0;  // later columns only
#pragma unroll
                for (int u = 0; u < 4; ++u) a[u][v] = fma(m, lr[u], a[u][v]);
            }
        }
    if (bad) flag[0] = 1;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = ty + 16 * u, t = tx + 16 * v;
            Lp[t * kPanel + r] = t <= r ? a[u][v] : 0.0;
            if (r < nb && t <= r) A[(p0 + r) * K + p0 + t] = a[u][v];
        }
}

// The first panel's diagonal block (later ones are factored by the trailing update before them).
__global__ __launch_bounds__(256) void k_chol_diag(double *__restrict__ A, int64_t K, double *__restrict__ Lp,
                                                   int *__restrict__ flag) {
    __shared__ double T[kPanel * kLd];
    const int nb = (int)min<int64_t>(kPanel, K);
    load_tile(
        T, A, [&](int r, int c) { return (int64_t)r * K + c; }, [&](int r, int c) { return r < nb && c <= r; },
        [](int, int) { return 0.0; }, [](int r, int c) { return r * kLd + c; });
    __syncthreads();
    chol_diag_block(T, nb, A, K, 0, Lp, flag);
}

// Rows below the diagonal block of panel [p0, p0 + nb): L21 = A21 L11^-T. One wave per 16 rows: lane
// (rr, cg) = (lane / 4, lane % 4) holds columns 16 cg .. 16 cg + 15 of row rr. Column c: its holders
// divide by L_cc, the finished value goes to the row's other lanes (its quad) by DPP, and every lane
// subtracts it from its later columns. No barriers after the load of L11 (packed by k_chol_diag).
__global__ __launch_bounds__(64) void k_chol_trsm(double *__restrict__ A, int64_t K, int64_t p0,
                                                  const double *__restrict__ Lp) {
    __shared__ double L[kPanel * kLd];
    const int nb = (int)min<int64_t>(kPanel, K - p0);
    {  // L11 from its column-major copy: lane = row, each load 512 contiguous bytes
        double v[kPanel];
#pragma unroll
        for (int c = 0; c < kPanel; ++c) v[c] = Lp[c * kPanel + threadIdx.x];
#pragma unroll
        for (int c = 0; c < kPanel; ++c) L[threadIdx.x * kLd + c] = v[c];
    }
    const int lane = threadIdx.x, rr = lane >> 2, cg = lane & 3;  // a row's four lanes form a quad
    const int64_t row = p0 + nb + (int64_t)blockIdx.x * 16 + rr;
    const bool in = row < K && 16 * cg < nb;  // nb % 16 == 0: a chunk is whole or absent
    const double *src = A + (in ? row * K + p0 + 16 * cg : 0);
    double x[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) x[v] = src[v];
    __syncthreads();
    __shared__ double rl[kPanel];  // 1 / L_cc, once per work-group, so no step waits for a division by it
    rl[lane] = 1.0 / L[lane * kLd + lane];
    __syncthreads();
#pragma unroll
    for (int cgs = 0; cgs < 4; ++cgs) {
        if (16 * cgs >= nb) break;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int c = 16 * cgs + v;
            const double xv = x[v] * rl[c];
            if (cg == cgs) x[v] = xv;
            const double xc = quad_bcast(xv, cgs);
            // unmasked (a zero multiplier leaves earlier columns exactly as they are), so the 16 LDS
            // reads are issued together
#pragma unroll
            for (int v2 = 0; v2 < 16; ++v2) {
                const int k = 16 * cg + v2;
                const double lkc = L[k * kLd + c];
                x[v2] = fma(k > c ? -xc : 0.0, lkc, x[v2]);
            }
        }
    }
    if (in) {
        double *dst = A + row * K + p0 + 16 * cg;
#pragma unroll
        for (int v = 0; v < 16; ++v) dst[v] = x[v];
    }
}

// Trailing update after panel [p0, p1): A[i][j] -= sum_t A[i][p0+t] A[j][p0+t] for p1 <= j <= i < K.
// 64 x 64 tiles of the lower triangle (tiles above it exit at once). Work-group (0, 0), dispatched first, holds
// the next panel's diagonal block and goes on to factor it.
__global__ __launch_bounds__(256) void k_chol_update(double *__restrict__ A, int64_t K, int64_t p0, int nb,
                                                     double *__restrict__ Lp, int *__restrict__ flag) {
    const int ti = blockIdx.y, tj = blockIdx.x;
    if (tj > ti) return;
    __shared__ double Pi[kTile * kLd], Pj[kTile * kLd];
    const int64_t p1 = p0 + nb, i0 = p1 + (int64_t)ti * kTile, j0 = p1 + (int64_t)tj * kTile;
    const auto zero = [](int, int) { return 0.0; };
    const auto at = [](int r, int t) { return r * kLd + t; };
    load_tile(
        Pi, A, [&](int r, int t) { return (i0 + r) * K + p0 + t; }, [&](int r, int t) { return i0 + r < K && t < nb; },
        zero, at);
    load_tile(
        Pj, A, [&](int r, int t) { return (j0 + r) * K + p0 + t; }, [&](int r, int t) { return j0 + r < K && t < nb; },
        zero, at);
    __syncthreads();
    f64x4 acc[2][2] = {};
    mfma_tile64(Pi, Pj, acc);
    double old[2][2][4];  // all loads issued before the stores
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t i = i0 + tile_row(m, q), j = j0 + tile_col(n);
                old[m][n][q] = A[i < K && j <= i ? i * K + j : 0];
            }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t i = i0 + tile_row(m, q), j = j0 + tile_col(n);
                if (i < K && j <= i) A[i * K + j] = old[m][n][q] - acc[m][n][q];
            }
    if (ti == 0 && tj == 0) {
        // this tile is the next panel's diagonal block, now final: factor it here, from LDS
        __syncthreads();  // every thread is done with Pi
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int q = 0; q < 4; ++q) Pi[tile_row(m, q) * kLd + tile_col(n)] = old[m][n][q] - acc[m][n][q];
        __syncthreads();
        chol_diag_block(Pi, (int)min<int64_t>(kPanel, K - p1), A, K, p1, Lp, flag);
    }
}

// The diagonal 64 x 64 blocks of V, packed contiguously for the column sweep: Vb[b][i][j] = V_(64b+i, 64b+j)
// for i <= j < nb, identity padding, zeros below the diagonal. One work-group per block.
__global__ __launch_bounds__(256) void k_gptq_pack_v(const double *__restrict__ A, int64_t K, double *__restrict__ Vb) {
    __shared__ double T[kPanel * kLd];
    const int64_t b0 = (int64_t)blockIdx.x * kPanel;
    const int nb = (int)min<int64_t>(kPanel, K - b0);
    load_tile(
        T, A, [&](int i, int j) { return (K - 1 - b0 - i) * K + (K - 1 - b0 - j); },
        [&](int i, int j) { return j < nb && i <= j; }, [](int i, int j) { return i == j ? 1.0 : 0.0; },
        [](int i, int j) { return i * kLd + j; });
    __syncthreads();
    double *dst = Vb + b0 * kPanel;
    for (int idx = threadIdx.x; idx < kPanel * kPanel; idx += 256) dst[idx] = T[(idx >> 6) * kLd + (idx & 63)];
}

// E2M1 index of the nearest magnitude to a >= 0 (ties to the even index, 6 beyond 5).
__device__ __forceinline__ uint32_t e2m1_index64(double a) {
    return (uint32_t)(a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5.0);
}

// Columns [b0, b0 + nb), one wave per 16 rows. Lane (rr, cg) = (lane / 4, lane % 4) holds columns
// b0 + 16 cg .. + 15 of row rr (one NVFP4 block, so one scale): their weights and running sums
// acc = S + sum over the block's earlier columns of e_i V_ik. Column j: its holders turn their sum into the
// target, code and error e_j; e_j reaches the row's other lanes (its quad) by DPP; every lane adds e_j V_jk
// to its later columns. No barriers after the load of V.
template <bool F32>
__global__ __launch_bounds__(64) void k_gptq_cols(const void *__restrict__ W, int64_t R, int64_t K, int64_t b0,
                                                  int nb, const double *__restrict__ Vb,
                                                  const uint8_t *__restrict__ dead,
                                                  const uint8_t *__restrict__ scales,
                                                  const float *__restrict__ alpha_p, const double *__restrict__ S,
                                                  double *__restrict__ E, int ldE, int ecol0,
                                                  uint8_t *__restrict__ codes) {
    __shared__ double V[kPanel * kLd];  // V[i][j] = V_(b0+i, b0+j) for i <= j, identity padding
    load_tile_wave(
        V, Vb + (b0 / kPanel) * kPanel * kPanel, [](int i, int j) { return i * kPanel + j; },
        [](int, int) { return true; }, [](int, int) { return 0.0; });
    const int lane = threadIdx.x, rr = lane >> 2, cg = lane & 3;  // a row's four lanes form a quad
    const int64_t row = (int64_t)blockIdx.x * 16 + rr;
    const bool in = row < R && 16 * cg < nb;  // nb % 16 == 0: a chunk is whole or absent
    const int64_t base = in ? row * K + b0 + 16 * cg : 0;  // element index, a multiple of 16
    // every load of the lane issued before any is used (masked lanes read element 0 and discard it)
    double acc[16], w[16];
    const double *sp = S + (b0 > 0 ? base : 0);
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = sp[v];
    uint32_t wr[16];
    if (F32) {
        const uint4 *wp = reinterpret_cast<const uint4 *>(static_cast<const float *>(W) + base);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 t = wp[q];
            wr[4 * q] = t.x, wr[4 * q + 1] = t.y, wr[4 * q + 2] = t.z, wr[4 * q + 3] = t.w;
        }
    } else {
        const uint4 *wp = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(W) + base);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint4 t = wp[q];
            const uint32_t d[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) wr[8 * q + 2 * h] = d[h] << 16, wr[8 * q + 2 * h + 1] = d[h] & 0xFFFF0000u;
        }
    }
    const uint4 dd = *reinterpret_cast<const uint4 *>(dead + (in ? b0 + 16 * cg : 0));
    const uint32_t sb = scales[in ? base / 16 : 0];
    const float alpha = *alpha_p;
    const uint32_t dw[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const bool isdead = ((dw[v / 4] >> (8 * (v % 4))) & 0xFFu) != 0;
        acc[v] = in && b0 > 0 ? acc[v] : 0.0;
        w[v] = in && !isdead ? (double)__uint_as_float(wr[v]) : 0.0;
    }
    const double s = in ? (double)(alpha * e4m3_value(sb)) : 0.0;  // fl32(alpha Delta) of the lane's block
    __syncthreads();
    __shared__ double rv[kPanel];  // 1 / V_jj, once per work-group, so no step waits for a division by it
    rv[lane] = 1.0 / V[lane * kLd + lane];
    __syncthreads();
    double ev[16] = {};
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int cgs = 0; cgs < 4; ++cgs) {
        if (16 * cgs >= nb) break;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int j = 16 * cgs + v;
            // branch-free: a block scale that is not positive (s = 0, or NaN) gives code 0 and no dequantised value
            const double t = w[v] + acc[v] * rv[j];
            const bool live = s > 0.0;
            const double x = t / (live ? s : 1.0);
            const uint32_t idx = live ? e2m1_index64(fabs(x)) : 0u;
            const bool neg = x < 0.0 && idx > 0;
            const uint32_t code = idx | (neg ? 8u : 0u);
            const double mag = idx < 4 ? 0.5 * idx : (idx == 7 ? 6.0 : (double)(idx - 2));
            const double deq = live ? (neg ? -mag : mag) * s : 0.0;
            const double e = w[v] - deq;
            const bool own = cg == cgs;
            ev[v] = own ? e : ev[v];
            packed[v / 8] |= (own ? code : 0u) << (4 * (v % 8));
            const double ej = quad_bcast(e, cgs);
            // unmasked (a zero multiplier leaves earlier columns exactly as they are), so the 16 LDS
            // reads are issued together
#pragma unroll
            for (int v2 = 0; v2 < 16; ++v2) {
                const int k = 16 * cg + v2;
                const double vjk = V[j * kLd + k];
                acc[v2] = fma(k > j ? ej : 0.0, vjk, acc[v2]);
            }
        }
    }
    if (in) {
        double *ep = E + row * ldE + ecol0 + 16 * cg;
#pragma unroll
        for (int v = 0; v < 16; ++v) ep[v] = ev[v];
        *reinterpret_cast<uint2 *>(codes + base / 2) = make_uint2(packed[0], packed[1]);  // 8-byte aligned
    }
}

// S[r][k] (=, when the reduction starts at column 0, else +=) sum_{i < depth} E[r][ecol0 + i] V_(vrow0+i, k)
// for k in [kbeg, kend), in 64 x 64 tiles on the fp64 matrix cores, the reduction in 64-deep steps.
__global__ __launch_bounds__(256) void k_gptq_update(const double *__restrict__ E, int ldE, int ecol0,
                                                     const double *__restrict__ A, double *__restrict__ S, int64_t R,
                                                     int64_t K, int64_t vrow0, int depth, int64_t kbeg, int64_t kend) {
    __shared__ double Et[kTile * kLd], Vt[kTile * kLd];
    const int64_t r0 = (int64_t)blockIdx.y * kTile, k0 = kbeg + (int64_t)blockIdx.x * kTile;
    const auto zero = [](int, int) { return 0.0; };
    f64x4 acc[2][2] = {};
    for (int d0 = 0; d0 < depth; d0 += kPanel) {
        const int dn = min(kPanel, depth - d0);
        if (d0 > 0) __syncthreads();  // the previous step's reads are done
        load_tile(
            Et, E, [&](int a, int i) { return (r0 + a) * ldE + ecol0 + d0 + i; },
            [&](int a, int i) { return r0 + a < R && i < dn; }, zero, [](int a, int i) { return a * kLd + i; });
        // reduction row i, consecutive threads on consecutive (descending) A columns; stored transposed
        load_tile(
            Vt, A, [&](int i, int kk) { return (K - 1 - vrow0 - d0 - i) * K + (K - 1 - k0 - kk); },
            [&](int i, int kk) { return k0 + kk < kend && i < dn; }, zero, [](int i, int kk) { return kk * kLd + i; });
        __syncthreads();
        mfma_tile64(Et, Vt, acc);
    }
    const bool first = vrow0 == 0;
    double old[2][2][4];  // all loads issued before the stores
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t r = r0 + tile_row(m, q), k = k0 + tile_col(n);
                old[m][n][q] = first ? 0.0 : S[r < R && k < kend ? r * K + k : 0];
            }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t r = r0 + tile_row(m, q), k = k0 + tile_col(n);
                if (r < R && k < kend) S[r * K + k] = old[m][n][q] + acc[m][n][q];
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
    const size_t nblocks = (size_t)(K + kPanel - 1) / kPanel;
    return up((size_t)K * K * 8) + up((size_t)R * K * 8) + up((size_t)R * kSuper * 8) +
           up(nblocks * kPanel * kPanel * 8) + up((size_t)kPanel * kPanel * 8) + up((size_t)K) + 256 +
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
    p += up((size_t)R * kSuper * 8);
    const int64_t nblocks = (K + kPanel - 1) / kPanel;
    double *Vb = reinterpret_cast<double *>(p);
    p += up((size_t)nblocks * kPanel * kPanel * 8);
    double *Lp = reinterpret_cast<double *>(p);
    p += up((size_t)kPanel * kPanel * 8);
    uint8_t *dead = reinterpret_cast<uint8_t *>(p);
    p += up((size_t)K);
    double *damp = reinterpret_cast<double *>(p);
    int *flag = reinterpret_cast<int *>(p + 8);
    p += 256;
    const int64_t nblk = R * K / 16;
    const Workspace q = carve(p, nblk);

    // the FourOverSix frame: scales and alpha (and codes, overwritten below)
    int ga = 0;
    hipError_t err = launch_amax(W, f32, nblk, false, q.amax_part, ga, nullptr, stream);
    if (err == hipSuccess)
        err = launch_quant(W, f32, true, nblk, q.amax_part, ga, codes, scales, alpha, nullptr, nullptr, q.m4_part,
                           stream);
    if (err != hipSuccess) return err;

    hipLaunchKernelGGL(k_gptq_prep, dim3(1), dim3(kPrepThreads), 0, stream, H, K, percdamp, damp, dead, flag);
    hipLaunchKernelGGL(k_gptq_reverse, dim3((unsigned)((K + 255) / 256), (unsigned)K), dim3(256), 0, stream, H, K,
                       damp, dead, A);
    hipLaunchKernelGGL(k_chol_diag, dim3(1), dim3(256), 0, stream, A, K, Lp, flag);
    for (int64_t p0 = 0; p0 < K; p0 += kPanel) {
        const int nb = (int)std::min<int64_t>(kPanel, K - p0);
        const int64_t below = K - p0 - nb;
        if (below > 0) {
            hipLaunchKernelGGL(k_chol_trsm, dim3((unsigned)((below + 15) / 16)), dim3(64), 0, stream, A, K, p0, Lp);
            const unsigned t = (unsigned)((below + kTile - 1) / kTile);
            hipLaunchKernelGGL(k_chol_update, dim3(t, t), dim3(256), 0, stream, A, K, p0, nb, Lp, flag);
        }
    }
    hipLaunchKernelGGL(k_gptq_pack_v, dim3((unsigned)nblocks), dim3(256), 0, stream, A, K, Vb);
    // Column blocks of 64, grouped by 4 (the last group may be shorter). E holds the group's errors. After a
    // block, S is updated only for the rest of its group; after the group's last block, for every later
    // column at once, with the group's whole error block as the reduction.
    const unsigned row_tiles = (unsigned)((R + kTile - 1) / kTile);
    for (int64_t b0 = 0; b0 < K; b0 += kPanel) {
        const int nb = (int)std::min<int64_t>(kPanel, K - b0);
        const int64_t sb0 = b0 / kSuper * kSuper, sb1 = std::min<int64_t>(sb0 + kSuper, K), b1 = b0 + nb;
        const dim3 grid((unsigned)((R + 15) / 16));
        if (f32)
            hipLaunchKernelGGL(k_gptq_cols<true>, grid, dim3(64), 0, stream, W, R, K, b0, nb, Vb, dead, scales, alpha,
                               S, E, kSuper, (int)(b0 - sb0), codes);
        else
            hipLaunchKernelGGL(k_gptq_cols<false>, grid, dim3(64), 0, stream, W, R, K, b0, nb, Vb, dead, scales, alpha,
                               S, E, kSuper, (int)(b0 - sb0), codes);
        if (b1 < sb1)
            hipLaunchKernelGGL(k_gptq_update, dim3((unsigned)((sb1 - b1 + kTile - 1) / kTile), row_tiles), dim3(256), 0,
                               stream, E, kSuper, (int)(b0 - sb0), A, S, R, K, b0, nb, b1, sb1);
        else if (sb1 < K)
            hipLaunchKernelGGL(k_gptq_update, dim3((unsigned)((K - sb1 + kTile - 1) / kTile), row_tiles), dim3(256), 0,
                               stream, E, kSuper, 0, A, S, R, K, sb0, (int)(sb1 - sb0), sb1, K);
    }
    const int64_t n8 = R * K / 16;
    hipLaunchKernelGGL(k_gptq_finish, dim3((unsigned)std::max<int64_t>(1, (n8 + 255) / 256)), dim3(256), 0, stream,
                       flag, n8, codes, alpha);
    return hipGetLastError();
}

}  // namespace nvfp4
