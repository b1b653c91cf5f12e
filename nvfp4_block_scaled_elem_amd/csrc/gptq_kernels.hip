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
//   k_chol_diag,    blocked Cholesky of A in place, panels of 64 columns: the diagonal block (one
//   k_chol_trsm,    work-group, LDL^T by four waves in groups of 8 columns), the rows below it (16 lanes per
//                   row), and the updates
//   k_chol_update   (64 x 64 tiles on the fp64 matrix cores), delayed over groups of 4 panels: a panel's stripe
//                   takes its group's earlier panels just before it is factored, the trailing triangle the whole
//                   group after it; an update's first work-group also factors the diagonal block it completes,
//                   so only the first has its own launch
//   k_gptq_pack_v   the 64 x 64 blocks of V the sweep reads (each column block's diagonal block and the
//                   blocks above it within its group), packed contiguously
//   k_gptq_cols     columns [b0, b0 + 64), 16 lanes per row, in order (target, E2M1 code, error e_j),
//                   each column's errors folded into the block's later columns at once
//   k_gptq_update   after each group of 4 blocks, S[:, k] += sum over the group of e_i V_ik for every
//                   column k beyond it (fp64 matrix cores, 64 x 64 tiles); within a group, the sweep adds the
//                   group's earlier blocks itself (fp64 matrix cores, operands read straight from memory)
//   k_gptq_finish   a failed factorisation (a pivot that is not positive and finite): alpha = NaN, codes 0
// S holds sum_{i<g0} e_i V_ik for the columns not yet reached, g0 the start of the current group. The update
// after the first group writes it, so it needs no clearing.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

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

// load_tile in two halves, so that the next tile's global loads can be in flight while the current one is
// used: fetch_tile issues the 16 loads of a thread, put_tile stores them.
template <class Off, class Ok>
__device__ __forceinline__ void fetch_tile(double (&v)[16], const double *__restrict__ src, Off off, Ok ok) {
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int idx = threadIdx.x + 256 * it, r = idx >> 6, c = idx & 63;
        v[it] = src[ok(r, c) ? off(r, c) : 0];
    }
}
template <class Ok, class Pos>
__device__ __forceinline__ void put_tile(double *lds, const double (&v)[16], Ok ok, Pos pos) {
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int idx = threadIdx.x + 256 * it, r = idx >> 6, c = idx & 63;
        lds[pos(r, c)] = ok(r, c) ? v[it] : 0.0;
    }
}

// x of lane N (0..15) of this lane's DPP row (16 lanes), by row_newbcast (gfx90a and later): a few cycles,
// where a shuffle goes through the LDS crossbar. n must fold to a constant after unrolling.
template <int N>
__device__ __forceinline__ double row_bcast_k(double x) {
    const unsigned long long u = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_mov_dpp((int)(unsigned)u, 0x150 + N, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(unsigned)(u >> 32), 0x150 + N, 0xF, 0xF, false);
    return __longlong_as_double(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ double row_bcast(double x, int n) {
    switch (n) {
        case 0: return row_bcast_k<0>(x);
        case 1: return row_bcast_k<1>(x);
        case 2: return row_bcast_k<2>(x);
        case 3: return row_bcast_k<3>(x);
        case 4: return row_bcast_k<4>(x);
        case 5: return row_bcast_k<5>(x);
        case 6: return row_bcast_k<6>(x);
        case 7: return row_bcast_k<7>(x);
        case 8: return row_bcast_k<8>(x);
        case 9: return row_bcast_k<9>(x);
        case 10: return row_bcast_k<10>(x);
        case 11: return row_bcast_k<11>(x);
        case 12: return row_bcast_k<12>(x);
        case 13: return row_bcast_k<13>(x);
        case 14: return row_bcast_k<14>(x);
        default: return row_bcast_k<15>(x);
    }
}

// A 64 x 64 tile of doubles stored contiguously (row stride 64) into LDS with the same layout, by 256
// threads in 16-byte pieces, all 8 loads of a thread issued before any store.
__device__ __forceinline__ void copy_tile256(double *lds, const double *__restrict__ src) {
    const double2 *s2 = reinterpret_cast<const double2 *>(src);
    double2 *d2 = reinterpret_cast<double2 *>(lds);
    double2 v[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) v[it] = s2[threadIdx.x + 256 * it];
#pragma unroll
    for (int it = 0; it < 8; ++it) d2[threadIdx.x + 256 * it] = v[it];
}

// Entries 4 c .. 4 c + 3 of row j of a row-stride-64 LDS tile (two 16-byte reads).
__device__ __forceinline__ void lds_row4(const double *T, int j, int c, double (&out)[4]) {
    const double2 *p = reinterpret_cast<const double2 *>(T + j * kPanel + 4 * c);
    const double2 a = p[0], b = p[1];
    out[0] = a.x, out[1] = a.y, out[2] = b.x, out[3] = b.y;
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

// x of lane `lane` (a constant after unrolling) in every lane.
__device__ __forceinline__ double readlane_f64(double x, int lane) {
    const unsigned long long u = __double_as_longlong(x);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, lane);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), lane);
    return __longlong_as_double(((unsigned long long)hi << 32) | lo);
}

// 1 / sqrt(p): the hardware estimate and two Newton steps y += y (1 - p y^2) / 2, each doubling the correct bits.
__device__ __forceinline__ double rsqrt_nr(double p) {
    double y = __builtin_amdgcn_rsq(p);
#pragma unroll
    for (int it = 0; it < 2; ++it) y = fma(0.5 * y, fma(-(p * y), y, 1.0), y);
    return y;
}

// 1 / p: the hardware estimate and two Newton steps y += y (1 - p y).
__device__ __forceinline__ double rcp_nr(double p) {
    double y = __builtin_amdgcn_rcp(p);
#pragma unroll
    for (int it = 0; it < 2; ++it) y = fma(y, fma(-p, y, 1.0), y);
    return y;
}

// Factors the diagonal block of panel [p0, p0 + nb), held in T (LDS, row stride kLd, lower triangle), as
// A = L~ D L~^T (then L = L~ D^(1/2)), so that the chain from one pivot to the next holds a reciprocal and no
// square root. The 64 columns form groups of kG; wave w holds groups w, w + 4, ..., lane r the entries of row r
// of the symmetric Schur complement S in those columns (padded to 64 with an identity). Group g: its wave runs
// the kG steps. Step c: the pivot p_c = S_cc comes from lane c by readlane, every lane takes m_r = S_rc / p_c and
// subtracts m_r S_ck from its group's later columns k, S_ck read from lane c. The lanes r <= c take part
// unmasked: what they change lies above their diagonal, which no later step reads, and a row's entries at and
// below its diagonal are final once its own step is done (S_rc at step c, and p_r). The wave then publishes
// S_rc and m_r of the group in LDS, and after a barrier every wave applies the rank-kG update to its later
// groups; the next group's wave updates that group first and the rest after its steps. At the end,
// L_rc = S_rc / sqrt(p_c) and L_rr = sqrt(p_r). The factor goes back into T, then into A, and packed
// column-major with zeros above the diagonal into Lp for the row solve. A pivot that is not positive and finite
// sets *flag. Called by all 256 threads of the work-group; pub is LDS that the caller no longer needs.
constexpr int kPubDoubles = 4 * kPanel * 8;  // LDS the factorisation of a diagonal block publishes its groups in

template <int kG>
__device__ __forceinline__ void chol_diag_block_g(double *T, double *pub, int nb, double *__restrict__ A, int64_t K,
                                                  int64_t p0, double *__restrict__ Lp, int *__restrict__ flag) {
    constexpr int kS = kPanel / kG / 4;  // groups per wave
    // the published group, double-buffered by group parity: [buf][row][i] = S_(row, c0 + i), m_(row, i), in
    // pub (at least 4 * 64 * kG doubles, 16-byte aligned)
    double(*s_pub)[kPanel * kG] = reinterpret_cast<double(*)[kPanel * kG]>(pub);
    double(*m_pub)[kPanel * kG] = reinterpret_cast<double(*)[kPanel * kG]>(pub + 2 * kPanel * kG);
    const int r = threadIdx.x & 63, w = threadIdx.x >> 6;
    double a[kS][kG];  // slot j: group w + 4 j
#pragma unroll
    for (int j = 0; j < kS; ++j)
#pragma unroll
        for (int i = 0; i < kG; ++i) {
            const int k = kG * (w + 4 * j) + i;
            const int hi = k > r ? k : r, lo = k > r ? r : k;  // the lower triangle, mirrored
            a[j][i] = hi < nb ? T[hi * kLd + lo] : (r == k ? 1.0 : 0.0);
        }
    bool bad = false;
    // The rank-kG update of columns [k0, k0 + kG) of this wave with group g's published values.
    const auto update = [&](double(&x)[kG], int k0, int g) {
        double mr[kG];
        const double2 *sm = reinterpret_cast<const double2 *>(m_pub[g & 1] + r * kG);
#pragma unroll
        for (int i = 0; i < kG; i += 2) {
            const double2 v = sm[i / 2];
            mr[i] = v.x, mr[i + 1] = v.y;
        }
        // every load is issued before the first product (the scheduler barrier keeps them there), so their
        // latencies overlap instead of adding up
        double2 sv[kG][kG / 2];
#pragma unroll
        for (int i2 = 0; i2 < kG; ++i2) {
            const double2 *sk = reinterpret_cast<const double2 *>(s_pub[g & 1] + (k0 + i2) * kG);
#pragma unroll
            for (int i = 0; i < kG; i += 2) sv[i2][i / 2] = sk[i / 2];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i2 = 0; i2 < kG; ++i2) {
            double e = x[i2], o = 0.0;
#pragma unroll
            for (int i = 0; i < kG; i += 2) {
                e = fma(-mr[i], sv[i2][i / 2].x, e);
                o = fma(-mr[i + 1], sv[i2][i / 2].y, o);
            }
            x[i2] = e + o;
        }
    };
    // Group g, held in slot J of wave g % 4. The group index is a runtime value (one loop per slot), so the
    // register arrays keep constant indices and each pass is one straight-line body.
    const auto group = [&](int g, auto slot) {
        constexpr int J = decltype(slot)::value;
        if (w == g % 4) {
            double mb[kG];
#pragma unroll
            for (int i = 0; i < kG; ++i) {
                const int c = kG * g + i;
                const double p = readlane_f64(a[J][i], c);  // the same in every lane
                bad = bad || !(p > 0.0) || !(p < INFINITY);
                const double m = a[J][i] * rcp_nr(p);
                mb[i] = m;
#pragma unroll
                for (int i2 = i + 1; i2 < kG; ++i2) a[J][i2] = fma(-m, readlane_f64(a[J][i2], c), a[J][i2]);
            }
            double2 *ds = reinterpret_cast<double2 *>(s_pub[g & 1] + r * kG);
            double2 *dm = reinterpret_cast<double2 *>(m_pub[g & 1] + r * kG);
#pragma unroll
            for (int i = 0; i < kG; i += 2) {
                ds[i / 2] = make_double2(a[J][i], a[J][i + 1]);
                dm[i / 2] = make_double2(mb[i], mb[i + 1]);
            }
            // this wave's later slots take the previous group's update now (left from before these steps; its
            // values stay published until the barrier after this group)
            if (g > 0) {
#pragma unroll
                for (int jj = J + 1; jj < kS; ++jj) update(a[jj], kG * (w + 4 * jj), g - 1);
            }
        }
        if (g + 1 == kPanel / kG) return;
        __syncthreads();
        // the update of this wave's later groups; the next group's wave updates that group only, runs its steps
        // first, and then the rest
        const bool next_owner = w == (g + 1) % 4;
#pragma unroll
        for (int jj = 0; jj < kS; ++jj) {
            if (w + 4 * jj <= g || (next_owner && jj > (g + 1) / 4)) continue;
            update(a[jj], kG * (w + 4 * jj), g);
        }
    };
    const auto pass = [&](auto slot) {
        constexpr int J = decltype(slot)::value;
#pragma unroll 1
        for (int g = 4 * J; g < 4 * J + 4; ++g) group(g, slot);
    };
    pass(std::integral_constant<int, 0>());
    if constexpr (kS > 1) pass(std::integral_constant<int, 1>());
    if constexpr (kS > 2) pass(std::integral_constant<int, 2>());
    if constexpr (kS > 3) pass(std::integral_constant<int, 3>());
    if (bad) flag[0] = 1;  // uniform within the wave that found it
#pragma unroll
    for (int j = 0; j < kS; ++j)
#pragma unroll
        for (int i = 0; i < kG; ++i) {
            const int c = kG * (w + 4 * j) + i;
            const double p = readlane_f64(a[j][i], c);
            const double y = rsqrt_nr(p);
            const double v = c < r ? a[j][i] * y : (c == r ? p * y : 0.0);
            T[r * kLd + c] = v;
            Lp[c * kPanel + r] = v;  // lanes on consecutive addresses
        }
    __syncthreads();
    for (int idx = threadIdx.x; idx < kPanel * kPanel; idx += 256) {
        const int rr = idx >> 6, k = idx & 63;
        if (rr < nb && k <= rr) A[(p0 + rr) * K + p0 + k] = T[rr * kLd + k];
    }
}

// Groups of 8 (groups of 4 measured the same; the pivot chain, not the group count, sets the time).
__device__ __forceinline__ void chol_diag_block(double *T, double *pub, int nb, double *__restrict__ A, int64_t K,
                                                int64_t p0, double *__restrict__ Lp, int *__restrict__ flag) {
    chol_diag_block_g<8>(T, pub, nb, A, K, p0, Lp, flag);
}

// The first panel's diagonal block (later ones are factored by the trailing update before them).
__global__ __launch_bounds__(256) void k_chol_diag(double *__restrict__ A, int64_t K, double *__restrict__ Lp,
                                                   int *__restrict__ flag) {
    __shared__ double T[kPanel * kLd];
    __shared__ __align__(16) double pub[kPubDoubles];
    const int nb = (int)min<int64_t>(kPanel, K);
    load_tile(
        T, A, [&](int r, int c) { return (int64_t)r * K + c; }, [&](int r, int c) { return r < nb && c <= r; },
        [](int, int) { return 0.0; }, [](int r, int c) { return r * kLd + c; });
    __syncthreads();
    chol_diag_block(T, pub, nb, A, K, 0, Lp, flag);
}

// Rows below the diagonal block of panel [p0, p0 + nb): L21 = A21 L11^-T, 16 rows per work-group. A row's 16
// lanes form one DPP row; lane c holds columns 4 c .. 4 c + 3. Column t: its holder scales it by 1 / L_tt, the
// finished value goes to the row's other lanes by DPP, and every lane subtracts it times L_kt from its
// columns k > t. No barriers after the load of L11 (packed column-major by the diagonal factorisation).
__global__ __launch_bounds__(256) void k_chol_trsm(double *__restrict__ A, int64_t K, int64_t p0,
                                                   const double *__restrict__ Lp) {
    __shared__ double LT[kPanel * kPanel];  // LT[t][k] = L_kt: zero above the diagonal, identity padding
    copy_tile256(LT, Lp);
    const int nb = (int)min<int64_t>(kPanel, K - p0);
    const int c = threadIdx.x & 15;
    const int64_t row = p0 + nb + (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const bool in = row < K && 4 * c < nb;  // nb % 16 == 0: a lane's four columns are whole or absent
    double2 *src = reinterpret_cast<double2 *>(A + (in ? row * K + p0 + 4 * c : 0));  // 32-byte aligned
    const double2 x01 = src[0], x23 = src[1];
    double x[4] = {x01.x, x01.y, x23.x, x23.y};
    __syncthreads();
    double rl[4];  // 1 / L_kk of the lane's own columns, so no step waits for a division
#pragma unroll
    for (int v = 0; v < 4; ++v) rl[v] = 1.0 / LT[(4 * c + v) * kPanel + 4 * c + v];
    double l[4];
    lds_row4(LT, 0, c, l);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        if (16 * cb >= nb) break;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int t = 16 * cb + u, h = t >> 2, v = t & 3;
            double ln[4];  // the next column's entries, read ahead
            lds_row4(LT, (t + 1) & 63, c, ln);
            const double xv = x[v] * rl[v];  // final in the holder (h == c); discarded elsewhere
            if (c == h) x[v] = xv;
            const double xt = row_bcast(xv, h);
            const double mlater = c > h ? -xt : 0.0, mfrom = c >= h ? -xt : 0.0;
#pragma unroll
            for (int v2 = 0; v2 < 4; ++v2) x[v2] = fma(v2 > v ? mfrom : mlater, l[v2], x[v2]);  // k = 4c + v2 > t
#pragma unroll
            for (int v2 = 0; v2 < 4; ++v2) l[v2] = ln[v2];
        }
    }
    if (in) {
        src[0] = make_double2(x[0], x[1]);
        src[1] = make_double2(x[2], x[3]);
    }
}

// A[i][j] -= sum_{t in [s0, s0 + depth)} A[i][t] A[j][t] for o0 <= j <= i < K, in 64 x 64 tiles of the lower
// triangle at (o0 + 64 y, o0 + 64 x) (tiles above it exit at once), the reduction in 64-deep steps on the fp64
// matrix cores. Columns [s0, s0 + depth) are final factor columns. The grid's x extent bounds the columns: the
// whole trailing triangle, or one stripe of 64. Work-group (0, 0), dispatched first, holds the diagonal block at
// o0, which these columns complete, and goes on to factor it.
__global__ __launch_bounds__(256) void k_chol_update(double *__restrict__ A, int64_t K, int64_t s0, int depth,
                                                     int64_t o0, double *__restrict__ Lp, int *__restrict__ flag) {
    const int ti = blockIdx.y, tj = blockIdx.x;
    if (tj > ti) return;
    __shared__ __align__(16) double Pi[kTile * kLd], Pj[kTile * kLd];
    static_assert(kPubDoubles <= kTile * kLd, "the published groups reuse Pj");
    const int64_t i0 = o0 + (int64_t)ti * kTile, j0 = o0 + (int64_t)tj * kTile;
    const auto zero = [](int, int) { return 0.0; };
    const auto at = [](int r, int t) { return r * kLd + t; };
    f64x4 acc[2][2] = {};
    for (int d0 = 0; d0 < depth; d0 += kPanel) {
        if (d0 > 0) __syncthreads();  // the previous step's reads are done
        const int64_t c0 = s0 + d0;
        load_tile(
            Pi, A, [&](int r, int t) { return (i0 + r) * K + c0 + t; }, [&](int r, int) { return i0 + r < K; }, zero,
            at);
        load_tile(
            Pj, A, [&](int r, int t) { return (j0 + r) * K + c0 + t; }, [&](int r, int) { return j0 + r < K; }, zero,
            at);
        __syncthreads();
        mfma_tile64(Pi, Pj, acc);
    }
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
        // this tile is the diagonal block at o0, now final: factor it here, from LDS
        __syncthreads();  // every thread is done with Pi
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int q = 0; q < 4; ++q) Pi[tile_row(m, q) * kLd + tile_col(n)] = old[m][n][q] - acc[m][n][q];
        __syncthreads();
        chol_diag_block(Pi, Pj, (int)min<int64_t>(kPanel, K - o0), A, K, o0, Lp, flag);
    }
}

// The 64 x 64 blocks of V the column sweep reads, packed contiguously: for column block b (columns
// [64 b, 64 b + 64)) at position q in its group of 4, slot t <= q holds V_(64 (b - q + t) + i, 64 b + k): the
// group's earlier blocks (t < q) whole, the diagonal block (t = q) for i <= k with identity padding and zeros
// below. Columns beyond K are zero. One work-group per (block, slot).
__global__ __launch_bounds__(256) void k_gptq_pack_v(const double *__restrict__ A, int64_t K, double *__restrict__ Vb) {
    __shared__ double T[kPanel * kLd];
    const int64_t b0 = (int64_t)blockIdx.x * kPanel;
    const int t = blockIdx.y, q = (int)((b0 % kSuper) / kPanel);
    if (t > q) return;
    const int64_t pb = b0 - (int64_t)(q - t) * kPanel;  // the slot's first row of V
    const int nb = (int)min<int64_t>(kPanel, K - b0);
    const bool diag = t == q;
    load_tile(
        T, A, [&](int i, int j) { return (K - 1 - pb - i) * K + (K - 1 - b0 - j); },
        [&](int i, int j) { return j < nb && (!diag || i <= j); },
        [&](int i, int j) { return diag && i == j ? 1.0 : 0.0; }, [](int i, int j) { return i * kLd + j; });
    __syncthreads();
    double *dst = Vb + ((int64_t)blockIdx.x * 4 + t) * kPanel * kPanel;
    for (int idx = threadIdx.x; idx < kPanel * kPanel; idx += 256) dst[idx] = T[(idx >> 6) * kLd + (idx & 63)];
}

// Columns [b0, b0 + nb), 16 rows per work-group, in order. A row's 16 lanes form one DPP row; lane c holds
// columns b0 + 4 c .. 4 c + 3 (a quarter of an NVFP4 block) with their weights and running sums
// acc = S + sum over the earlier columns of the group of 4 blocks of e_i V_ik (S holds the groups before; the
// group's earlier blocks are added here, each 64 x 64 block of V staged in LDS, the errors of a row going to
// its lanes by DPP) + sum over the panel's earlier columns of e_i V_ik. Column j: its holder forms the target
// t = w + acc / V_jj, the code and the error e_j = w - q_j; e_j goes to the row's other lanes by DPP, and every
// lane adds e_j V_jk to its columns. No barriers after the load of V.
//
// The code is the nearest E2M1 value to t / s, ties to the even index, s = fl32(alpha Delta) of the block. The
// quotient is never formed: |t| is compared with the decision points times s, products that binary64 holds
// exactly (three significant bits times a binary32 value), so each comparison is that of the exact t / s.
// A block scale that is not positive (0, or NaN) gives code 0 and no dequantised value.
template <bool F32>
__global__ __launch_bounds__(256) void k_gptq_cols(const void *__restrict__ W, int64_t R, int64_t K, int64_t b0,
                                                   int nb, const double *__restrict__ Vb,
                                                   const uint8_t *__restrict__ dead,
                                                   const uint8_t *__restrict__ scales,
                                                   const float *__restrict__ alpha_p, const double *__restrict__ S,
                                                   double *__restrict__ E, int ldE, int ecol0,
                                                   uint8_t *__restrict__ codes) {
    __shared__ __align__(16) double V[kPanel * kPanel];  // a 64 x 64 block of V, row stride 64
    const int c = threadIdx.x & 15;
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const bool in = row < R && 4 * c < nb;  // nb % 16 == 0: a lane's four columns are whole or absent
    const int64_t base = in ? row * K + b0 + 4 * c : 0;  // element index, a multiple of 4
    const int64_t sb0 = b0 / kSuper * kSuper;           // the group's first column
    // every load of the lane issued before any is used (masked lanes read element 0 and discard it)
    const double2 *sp = reinterpret_cast<const double2 *>(S + (sb0 > 0 ? base : 0));  // 32-byte aligned
    const double2 s01 = sp[0], s23 = sp[1];
    uint32_t wr[4];
    if (F32) {
        const uint4 t = *reinterpret_cast<const uint4 *>(static_cast<const float *>(W) + base);
        wr[0] = t.x, wr[1] = t.y, wr[2] = t.z, wr[3] = t.w;
    } else {
        const uint2 t = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(W) + base);
        wr[0] = t.x << 16, wr[1] = t.x & 0xFFFF0000u, wr[2] = t.y << 16, wr[3] = t.y & 0xFFFF0000u;
    }
    const uint32_t dd = *reinterpret_cast<const uint32_t *>(dead + (in ? b0 + 4 * c : 0));
    const uint32_t sb = scales[base / 16];
    const float alpha = *alpha_p;
    const double sv[4] = {s01.x, s01.y, s23.x, s23.y};
    double acc[4], w[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        acc[v] = in && sb0 > 0 ? sv[v] : 0.0;
        w[v] = in && ((dd >> (8 * v)) & 0xFFu) == 0 ? (double)__uint_as_float(wr[v]) : 0.0;
    }
    // the group's earlier blocks: acc_k += sum_i e_i V_ik, i over blocks [pb, pb + 64) before this one, from
    // the packed slots of this column block (slot q, the last, is the diagonal block). On the fp64 matrix
    // cores: the work-group's 16 rows of errors (the A operand, from E) times each earlier block of V (the B
    // operand); wave wv takes the columns 16 wv .. 16 wv + 15 of the block. Both operands of every earlier
    // block are read straight from global memory, all at once, so their latencies overlap (through LDS, one
    // block at a time, each block cost a load-to-use latency of its own).
    const int q = (int)((b0 - sb0) / kPanel);
    const double *vt = Vb + (b0 / kPanel) * 4 * kPanel * kPanel;
    if (q > 0) {
        const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
        const int64_t arow = (int64_t)blockIdx.x * 16 + (l & 15);  // the A row of this lane
        // A[r][4 s + l / 16] = E[row r][64 t + 4 s + l / 16], B[4 s + l / 16][n] = V_t[4 s + l / 16][16 wv + n]
        // for the 16 steps s of block t (rows past R and blocks t >= q read as 0; the earlier blocks are whole)
        double ea[kSuper / kPanel - 1][16], vb[kSuper / kPanel - 1][16];
        const double *ep = E + (arow < R ? arow * ldE + (l >> 4) : 0);
        const double *bp = vt + (l >> 4) * kPanel + 16 * wv + (l & 15);
#pragma unroll
        for (int t = 0; t < kSuper / kPanel - 1; ++t)
#pragma unroll
            for (int st = 0; st < 16; ++st) {
                ea[t][st] = t < q && arow < R ? ep[kPanel * t + 4 * st] : 0.0;
                vb[t][st] = t < q ? bp[t * kPanel * kPanel + 4 * st * kPanel] : 0.0;
            }
        f64x4 g = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int t = 0; t < kSuper / kPanel - 1; ++t)
            if (t < q)
#pragma unroll
                for (int st = 0; st < 16; ++st) g = __builtin_amdgcn_mfma_f64_16x16x4f64(ea[t][st], vb[t][st], g, 0, 0, 0);
        // to the sweep's layout through LDS: register qq holds row 4 qq + l / 16, column 16 wv + l % 16
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) V[(4 * qq + (l >> 4)) * kPanel + 16 * wv + (l & 15)] = g[qq];
        __syncthreads();
#pragma unroll
        for (int v2 = 0; v2 < 4; ++v2) acc[v2] += V[(threadIdx.x >> 4) * kPanel + 4 * c + v2];
        __syncthreads();  // done with the sums before the diagonal block replaces them
    }
    copy_tile256(V, vt + q * kPanel * kPanel);  // the diagonal block
    const double s = in ? (double)(alpha * e4m3_value(sb)) : 0.0;
    const bool live = s > 0.0;
    // decision points between E2M1 magnitudes k and k + 1, times s; ties go to the even index, so the
    // comparison is > where k is even and >= where k is odd. Without a live scale they are NaN, so every
    // comparison fails (code 0), and the half-step is 0 (no dequantised value).
    const double sd = live ? s : __builtin_nan(""), hs = live ? 0.5 * s : 0.0;
    const double d0 = 0.25 * sd, d1 = 0.75 * sd, d2 = 1.25 * sd, d3 = 1.75 * sd, d4 = 2.5 * sd, d5 = 3.5 * sd,
                 d6 = 5.0 * sd;
    __syncthreads();
    double rv[4];  // 1 / V_kk of the lane's own columns, so no step waits for a division
#pragma unroll
    for (int v = 0; v < 4; ++v) rv[v] = 1.0 / V[(4 * c + v) * kPanel + 4 * c + v];
    double ev[4] = {}, eg[4], vj[4];
    uint32_t packed = 0u, cg[4];
    lds_row4(V, 0, c, vj);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        if (16 * cb >= nb) break;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int j = 16 * cb + u, h = j >> 2, v = j & 3;
            double vn[4];  // the next column's row of V, read ahead of this column's arithmetic
            lds_row4(V, (j + 1) & 63, c, vn);
            // the holder's (h == c) column; other lanes' results are discarded
            const double t = fma(acc[v], rv[v], w[v]);
            const double a = fabs(t);
            const uint32_t idx =
                (uint32_t)(a > d0) + (a >= d1) + (a > d2) + (a >= d3) + (a > d4) + (a >= d5) + (a > d6);
            // twice the magnitude: idx below 4, then 4, 6, 8, 12
            const uint32_t m2 = idx + (max(idx, 4u) - 4u) + 2u * (max(idx, 6u) - 6u);
            const uint32_t thi = (uint32_t)(__double_as_longlong(t) >> 32);
            // the dequantised value carries t's sign (a zero one too, which leaves e = w)
            const double q = __longlong_as_double(__double_as_longlong((double)m2 * hs) |
                                                  ((long long)(thi & 0x80000000u) << 32));
            eg[v] = w[v] - q;
            cg[v] = idx | ((thi >> 28) & (idx + 7u) & 8u);  // the sign bit only with a nonzero magnitude
            const double ej = row_bcast(eg[v], h);
            // unmasked: V_jk = 0 below the diagonal, and a column's sum is not read after its own step
#pragma unroll
            for (int v2 = 0; v2 < 4; ++v2) acc[v2] = fma(ej, vj[v2], acc[v2]);
#pragma unroll
            for (int v2 = 0; v2 < 4; ++v2) vj[v2] = vn[v2];
            if (v == 3) {  // the end of lane h's columns: keep them in the holder
                const bool own = c == h;
#pragma unroll
                for (int v2 = 0; v2 < 4; ++v2) {
                    ev[v2] = own ? eg[v2] : ev[v2];
                    packed |= (own ? cg[v2] : 0u) << (4 * v2);
                }
            }
        }
    }
    if (in) {
        double2 *ep = reinterpret_cast<double2 *>(E + row * ldE + ecol0 + 4 * c);  // 32-byte aligned
        ep[0] = make_double2(ev[0], ev[1]);
        ep[1] = make_double2(ev[2], ev[3]);
        *reinterpret_cast<uint16_t *>(codes + base / 2) = (uint16_t)packed;  // 2-byte aligned
    }
}

// S[r][k] (=, when the reduction starts at column 0, else +=) sum_{i < depth} E[r][ecol0 + i] V_(vrow0+i, k)
// for k in [kbeg, kend), in 64 x 64 tiles on the fp64 matrix cores, the reduction in 64-deep steps.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_gptq_update(
    const double *__restrict__ E, int ldE, int ecol0, const double *__restrict__ A, double *__restrict__ S, int64_t R,
    int64_t K, int64_t vrow0, int depth, int64_t kbeg, int64_t kend) {
    __shared__ double Et[kTile * kLd], Vt[kTile * kLd];
    const int64_t r0 = (int64_t)blockIdx.y * kTile, k0 = kbeg + (int64_t)blockIdx.x * kTile;
    f64x4 acc[2][2] = {};
    // step d0's tiles: E rows r0.., reduction columns d0..; V reduction rows d0.. (consecutive threads on
    // consecutive, descending, A columns), stored transposed
    const auto e_off = [&](int d0) { return [=](int a, int i) { return (r0 + a) * ldE + ecol0 + d0 + i; }; };
    const auto e_ok = [&](int d0) { return [=](int a, int i) { return r0 + a < R && i < depth - d0; }; };
    const auto v_off = [&](int d0) {
        return [=](int i, int kk) { return (K - 1 - vrow0 - d0 - i) * K + (K - 1 - k0 - kk); };
    };
    const auto v_ok = [&](int d0) { return [=](int i, int kk) { return k0 + kk < kend && i < depth - d0; }; };
    double fe[16], fv[16];  // the next step's tiles, in flight while the current one is multiplied
    fetch_tile(fe, E, e_off(0), e_ok(0));
    fetch_tile(fv, A, v_off(0), v_ok(0));
    for (int d0 = 0; d0 < depth; d0 += kPanel) {
        if (d0 > 0) __syncthreads();  // the previous step's reads are done
        put_tile(Et, fe, e_ok(d0), [](int a, int i) { return a * kLd + i; });
        put_tile(Vt, fv, v_ok(d0), [](int i, int kk) { return kk * kLd + i; });
        __syncthreads();
        if (d0 + kPanel < depth) {
            fetch_tile(fe, E, e_off(d0 + kPanel), e_ok(d0 + kPanel));
            fetch_tile(fv, A, v_off(d0 + kPanel), v_ok(d0 + kPanel));
        }
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
           up(nblocks * 4 * kPanel * kPanel * 8) + up((size_t)kPanel * kPanel * 8) + up((size_t)K) + 256 +
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
    p += up((size_t)nblocks * 4 * kPanel * kPanel * 8);
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
    // Cholesky with the updates delayed over groups of 4 panels: within a group, a panel's column stripe takes
    // the updates of the group's earlier panels just before it is factored; after the group, the rest of the
    // trailing triangle takes the whole group's update at once (reduction depth 256).
    hipLaunchKernelGGL(k_chol_diag, dim3(1), dim3(256), 0, stream, A, K, Lp, flag);
    for (int64_t g0 = 0; g0 < K; g0 += kSuper) {
        const int64_t g1 = std::min<int64_t>(g0 + kSuper, K);
        for (int64_t p0 = g0; p0 < g1; p0 += kPanel) {
            if (p0 > g0)
                hipLaunchKernelGGL(k_chol_update, dim3(1, (unsigned)((K - p0 + kTile - 1) / kTile)), dim3(256), 0,
                                   stream, A, K, g0, (int)(p0 - g0), p0, Lp, flag);
            const int64_t below = K - p0 - std::min<int64_t>(kPanel, K - p0);
            if (below > 0)
                hipLaunchKernelGGL(k_chol_trsm, dim3((unsigned)((below + 15) / 16)), dim3(256), 0, stream, A, K, p0,
                                   Lp);
        }
        if (g1 < K) {
            const unsigned t = (unsigned)((K - g1 + kTile - 1) / kTile);
            hipLaunchKernelGGL(k_chol_update, dim3(t, t), dim3(256), 0, stream, A, K, g0, (int)(g1 - g0), g1, Lp,
                               flag);
        }
    }
    hipLaunchKernelGGL(k_gptq_pack_v, dim3((unsigned)nblocks, 4), dim3(256), 0, stream, A, K, Vb);
    // Column blocks of 64, grouped by 4 (the last group may be shorter). E holds the group's errors. Within a
    // group, each block's sweep adds the group's earlier blocks to its sums itself; after the group's last
    // block, S takes every later column at once, with the group's whole error block as the reduction.
    const unsigned row_tiles = (unsigned)((R + kTile - 1) / kTile);
    for (int64_t b0 = 0; b0 < K; b0 += kPanel) {
        const int nb = (int)std::min<int64_t>(kPanel, K - b0);
        const int64_t sb0 = b0 / kSuper * kSuper, sb1 = std::min<int64_t>(sb0 + kSuper, K), b1 = b0 + nb;
        const dim3 grid((unsigned)((R + 15) / 16));
        if (f32)
            hipLaunchKernelGGL(k_gptq_cols<true>, grid, dim3(256), 0, stream, W, R, K, b0, nb, Vb, dead, scales,
                               alpha, S, E, kSuper, (int)(b0 - sb0), codes);
        else
            hipLaunchKernelGGL(k_gptq_cols<false>, grid, dim3(256), 0, stream, W, R, K, b0, nb, Vb, dead, scales,
                               alpha, S, E, kSuper, (int)(b0 - sb0), codes);
        if (b1 == sb1 && sb1 < K)
            hipLaunchKernelGGL(k_gptq_update, dim3((unsigned)((K - sb1 + kTile - 1) / kTile), row_tiles), dim3(256), 0,
                               stream, E, kSuper, 0, A, S, R, K, sb0, (int)(sb1 - sb0), sb1, K);
    }
    const int64_t n8 = R * K / 16;
    hipLaunchKernelGGL(k_gptq_finish, dim3((unsigned)std::max<int64_t>(1, (n8 + 255) / 256)), dim3(256), 0, stream,
                       flag, n8, codes, alpha);
    return hipGetLastError();
}

}  // namespace nvfp4
