// C ABI of the gfx950 NVFP4 quantizer (declared in include/nvfp4.h): argument checks on the host, the
// kernel sequence of each mode, and the stream-ordered scratch workspace.
//
// Kernel sequence per call (all on the caller's stream):
//   MAX / FourOverSix : k_amax -> k_quant
//   CJSO(T)           : k_amax -> k_cjso_init -> T x k_cjso_iter
//   SOAR(T)           : CJSO(T) -> k_soar
//   GPTQ (nvfp4_gptq) : k_amax -> k_quant (the FourOverSix frame) -> k_gptq_prep -> k_gptq_reverse ->
//                       k_chol_diag -> per group of 4 panels {per panel: k_chol_update (its stripe, but
//                       not for the group's first), k_chol_trsm; then k_chol_update (the trailing triangle)}
//                       -> k_gptq_pack_v -> per group of 4 column blocks {4 x k_gptq_cols, k_gptq_update}
//                       -> k_gptq_finish
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.hpp"

#define NVFP4_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxIters = 1000;
// At most 2^35 elements per matrix (64 GiB of bf16): kernels with one thread per 16-element block or per
// 8 values then stay below 2^32 threads per grid.
constexpr int64_t kMaxElems = (int64_t)1 << 35;

}  // namespace

namespace nvfp4 {

int kernel_count(int mode, int iters) {
    if (iters < 0 || iters > kMaxIters) return -1;
    switch (mode) {
        case NVFP4_MODE_MAX:
        case NVFP4_MODE_FOUR_OVER_SIX: return 2;
        case NVFP4_MODE_CJSO: return iters + 2;
        case NVFP4_MODE_SOAR: return iters + 3;
        default: return -1;
    }
}

int check_args(const nvfp4_args_t *a) {
    if (!a || !a->W || !a->codes_out || !a->scales_out || !a->alpha_out) return NVFP4_ERR_INVALID_ARG;
    if (a->rows <= 0 || a->cols <= 0) return NVFP4_ERR_INVALID_ARG;
    if (a->mode < NVFP4_MODE_MAX || a->mode > NVFP4_MODE_SOAR) return NVFP4_ERR_INVALID_ARG;
    if (a->dtype != NVFP4_DTYPE_BF16 && a->dtype != NVFP4_DTYPE_F32) return NVFP4_ERR_INVALID_ARG;
    if (a->iters < 0 || a->iters > kMaxIters) return NVFP4_ERR_INVALID_ARG;
    if (a->cols % 16 != 0) return NVFP4_ERR_SHAPE;
    if (a->rows > kMaxElems / a->cols) return NVFP4_ERR_SHAPE;
    if (((uintptr_t)a->W & 15u) != 0 || ((uintptr_t)a->codes_out & 7u) != 0 || ((uintptr_t)a->alpha_out & 3u) != 0)
        return NVFP4_ERR_INVALID_ARG;
    if (a->workspace && ((uintptr_t)a->workspace & 255u) != 0) return NVFP4_ERR_INVALID_ARG;
    if (a->stats_out && ((uintptr_t)a->stats_out & 3u) != 0) return NVFP4_ERR_INVALID_ARG;
    if (a->stage_events && a->n_stage_events < kernel_count(a->mode, a->iters) + 1) return NVFP4_ERR_INVALID_ARG;
    if (a->flags & ~(NVFP4_FLAG_FULL_SEARCH | NVFP4_FLAG_INIT_4O6)) return NVFP4_ERR_INVALID_ARG;
    if ((a->flags & NVFP4_FLAG_INIT_4O6) && a->mode != NVFP4_MODE_CJSO && a->mode != NVFP4_MODE_SOAR)
        return NVFP4_ERR_INVALID_ARG;
    const bool pages_grid = a->search_num0 == 0 && a->search_den == 0 && a->search_count == 0;
    if (!pages_grid || a->dd_rule != NVFP4_DD_CJSO) {
        if (a->mode != NVFP4_MODE_SOAR) return NVFP4_ERR_INVALID_ARG;
        if (a->dd_rule < NVFP4_DD_CJSO || a->dd_rule > NVFP4_DD_LSQ) return NVFP4_ERR_INVALID_ARG;
        if (!pages_grid &&
            (a->search_den < 1 || a->search_den > (1 << 24) || a->search_num0 < 1 || a->search_count < 1 ||
             a->search_count > NVFP4_SEARCH_MAX_COUNT ||
             (int64_t)a->search_num0 + a->search_count - 1 > 16 * (int64_t)a->search_den))
            return NVFP4_ERR_INVALID_ARG;
    }
    return NVFP4_OK;
}

// Records stage event j (profiling hook; no-op without events or for a NULL entry).
bool mark(const nvfp4_args_t *a, int j) {
    if (!a->stage_events || !a->stage_events[j]) return true;
    return hipEventRecord(static_cast<hipEvent_t>(a->stage_events[j]), static_cast<hipStream_t>(a->stream)) ==
           hipSuccess;
}

int run_quantize(const nvfp4_args_t *a, void *ws_base) {
    hipStream_t st = static_cast<hipStream_t>(a->stream);
    const bool f32 = a->dtype == NVFP4_DTYPE_F32;
    const int64_t n = a->rows * a->cols, nblk = n / 16;
    const Workspace ws = carve(ws_base, nblk);
    const bool cjso = a->mode == NVFP4_MODE_CJSO || a->mode == NVFP4_MODE_SOAR;
    int ga = 0;
    int j = 0;
    if (!mark(a, j++)) return NVFP4_ERR_HIP;
    if (launch_amax(a->W, f32, nblk, cjso, ws.amax_part, ga, a->stats_out, st) != hipSuccess || !mark(a, j++))
        return NVFP4_ERR_HIP;
    if (a->mode == NVFP4_MODE_MAX || a->mode == NVFP4_MODE_FOUR_OVER_SIX) {
        const bool fos = a->mode == NVFP4_MODE_FOUR_OVER_SIX;
        if (launch_quant(a->W, f32, fos, nblk, ws.amax_part, ga, a->codes_out, a->scales_out, a->alpha_out,
                         fos ? a->mchoice_out : nullptr, a->stats_out, ws.m4_part, st) != hipSuccess ||
            !mark(a, j++))
            return NVFP4_ERR_HIP;
        return NVFP4_OK;
    }
    const bool soar = a->mode == NVFP4_MODE_SOAR;
    const int gc = cjso_groups(nblk);
    const bool fos_init = (a->flags & NVFP4_FLAG_INIT_4O6) != 0;
    if (launch_cjso_init(a->W, f32, soar, fos_init, nblk, ws.amax_part, ga, a->iters, a->codes_out, a->scales_out,
                         a->alpha_out, ws, gc, a->stats_out, st) != hipSuccess ||
        !mark(a, j++))
        return NVFP4_ERR_HIP;
    for (int t = 1; t <= a->iters; ++t)
        if (launch_cjso_iter(a->W, f32, soar, nblk, t, a->iters, a->codes_out, a->scales_out, a->alpha_out, ws, gc,
                             st) != hipSuccess ||
            !mark(a, j++))
            return NVFP4_ERR_HIP;
    if (soar) {
        const bool pages_grid = a->search_count == 0;
        if (launch_soar(a->W, f32, nblk, ws.alpha_state + (a->iters & 1), a->codes_out, a->scales_out, ws.brackets,
                        (a->flags & NVFP4_FLAG_FULL_SEARCH) != 0, pages_grid ? 50 : a->search_num0,
                        pages_grid ? 100 : a->search_den, pages_grid ? 101 : a->search_count, a->dd_rule,
                        st) != hipSuccess ||
            !mark(a, j++))
            return NVFP4_ERR_HIP;
    }
    return NVFP4_OK;
}

}  // namespace nvfp4

NVFP4_API int nvfp4_kernel_count(int mode, int iters) { return nvfp4::kernel_count(mode, iters); }

NVFP4_API size_t nvfp4_workspace_bytes(int64_t rows, int64_t cols, int mode) {
    if (rows <= 0 || cols <= 0 || cols % 16 != 0 || rows > kMaxElems / cols) return 0;
    if (mode < NVFP4_MODE_MAX || mode > NVFP4_MODE_SOAR) return 0;
    return nvfp4::workspace_bytes(rows * cols / 16, mode);
}

NVFP4_API int nvfp4_quantize_ex(const nvfp4_args_t *a) {
    const int c = nvfp4::check_args(a);
    if (c != NVFP4_OK) return c;
    const size_t need = nvfp4::workspace_bytes(a->rows * a->cols / 16, a->mode);
    if (a->workspace) {
        if (a->workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
        return nvfp4::run_quantize(a, a->workspace);
    }
    hipStream_t st = static_cast<hipStream_t>(a->stream);
    void *ws = nullptr;
    if (hipMallocAsync(&ws, need, st) != hipSuccess) return NVFP4_ERR_HIP;
    const int r = nvfp4::run_quantize(a, ws);
    if (hipFreeAsync(ws, st) != hipSuccess) return NVFP4_ERR_HIP;
    return r;
}

NVFP4_API int nvfp4_quantize(const void *W, int64_t rows, int64_t cols, int mode, int iters, uint8_t *codes_out,
                             uint8_t *scales_out, float *alpha_out, void *stream) {
    nvfp4_args_t a = {};
    a.W = W;
    a.dtype = NVFP4_DTYPE_BF16;
    a.rows = rows;
    a.cols = cols;
    a.mode = mode;
    a.iters = iters;
    a.codes_out = codes_out;
    a.scales_out = scales_out;
    a.alpha_out = alpha_out;
    a.stream = stream;
    return nvfp4_quantize_ex(&a);
}

NVFP4_API int nvfp4_quantize_f32(const float *W, int64_t rows, int64_t cols, int mode, int iters, uint8_t *codes_out,
                                 uint8_t *scales_out, float *alpha_out, void *stream) {
    nvfp4_args_t a = {};
    a.W = W;
    a.dtype = NVFP4_DTYPE_F32;
    a.rows = rows;
    a.cols = cols;
    a.mode = mode;
    a.iters = iters;
    a.codes_out = codes_out;
    a.scales_out = scales_out;
    a.alpha_out = alpha_out;
    a.stream = stream;
    return nvfp4_quantize_ex(&a);
}

NVFP4_API int nvfp4_encode_e2m1(const float *x, int64_t n, uint8_t *codes, void *stream) {
    if (!x || !codes || n < 0) return NVFP4_ERR_INVALID_ARG;
    if (n > kMaxElems) return NVFP4_ERR_SHAPE;
    if (((uintptr_t)codes & 7u) != 0 || ((uintptr_t)x & 3u) != 0) return NVFP4_ERR_INVALID_ARG;
    if (n == 0) return NVFP4_OK;
    return nvfp4::launch_encode_e2m1(x, n, codes, static_cast<hipStream_t>(stream)) == hipSuccess ? NVFP4_OK
                                                                                                   : NVFP4_ERR_HIP;
}

NVFP4_API int nvfp4_reciprocal_f32(const float *s, int64_t n, float *r, void *stream) {
    if (!s || !r || n < 0) return NVFP4_ERR_INVALID_ARG;
    if (n > kMaxElems) return NVFP4_ERR_SHAPE;
    if (((uintptr_t)s & 3u) != 0 || ((uintptr_t)r & 3u) != 0) return NVFP4_ERR_INVALID_ARG;
    if (n == 0) return NVFP4_OK;
    return nvfp4::launch_reciprocal(s, n, r, static_cast<hipStream_t>(stream)) == hipSuccess ? NVFP4_OK
                                                                                           : NVFP4_ERR_HIP;
}

NVFP4_API int nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, const float *alpha, int64_t rows,
                               int64_t cols, void *out, int out_dtype, void *stream) {
    if (!codes || !scales || !alpha || !out || rows <= 0 || cols <= 0) return NVFP4_ERR_INVALID_ARG;
    if (out_dtype != NVFP4_DTYPE_BF16 && out_dtype != NVFP4_DTYPE_F32) return NVFP4_ERR_INVALID_ARG;
    if (cols % 16 != 0 || rows > kMaxElems / cols) return NVFP4_ERR_SHAPE;
    if (((uintptr_t)codes & 7u) != 0 || ((uintptr_t)out & 15u) != 0 || ((uintptr_t)alpha & 3u) != 0)
        return NVFP4_ERR_INVALID_ARG;
    return nvfp4::launch_dequant(codes, scales, alpha, rows * cols / 16, out, out_dtype == NVFP4_DTYPE_F32,
                                 static_cast<hipStream_t>(stream)) == hipSuccess
               ? NVFP4_OK
               : NVFP4_ERR_HIP;
}

NVFP4_API int nvfp4_error_stats(const void *W, int dtype, int64_t rows, int64_t cols, const uint8_t *codes,
                                const uint8_t *scales, const float *alpha, double *sse_out,
                                unsigned long long *hist_out, void *stream) {
    if (!W || !codes || !scales || !alpha || !sse_out || !hist_out || rows <= 0 || cols <= 0)
        return NVFP4_ERR_INVALID_ARG;
    if (dtype != NVFP4_DTYPE_BF16 && dtype != NVFP4_DTYPE_F32) return NVFP4_ERR_INVALID_ARG;
    if (cols % 16 != 0 || rows > kMaxElems / cols) return NVFP4_ERR_SHAPE;
    if (((uintptr_t)W & 15u) != 0 || ((uintptr_t)codes & 7u) != 0 || ((uintptr_t)alpha & 3u) != 0 ||
        ((uintptr_t)sse_out & 7u) != 0 || ((uintptr_t)hist_out & 7u) != 0)
        return NVFP4_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    if (hipMallocAsync(&ws, nvfp4::stats_workspace_bytes(), st) != hipSuccess) return NVFP4_ERR_HIP;
    const bool ok = nvfp4::launch_stats(W, dtype == NVFP4_DTYPE_F32, rows * cols / 16, codes, scales, alpha, sse_out,
                                        hist_out, ws, st) == hipSuccess;
    if (hipFreeAsync(ws, st) != hipSuccess) return NVFP4_ERR_HIP;
    return ok ? NVFP4_OK : NVFP4_ERR_HIP;
}

namespace {
int matmul_check(const void *X, int64_t M, int64_t K, const uint8_t *codes, const uint8_t *scales, const float *alpha,
                 int64_t N, void *Y, int y_dtype) {
    if (!X || !codes || !scales || !alpha || !Y || M <= 0 || K <= 0 || N <= 0) return NVFP4_ERR_INVALID_ARG;
    if (y_dtype != NVFP4_DTYPE_BF16 && y_dtype != NVFP4_DTYPE_F32) return NVFP4_ERR_INVALID_ARG;
    if (K % 16 != 0 || N > ((int64_t)1 << 25) || N > kMaxElems / K || M > kMaxElems / K || M > kMaxElems / N ||
        ((M + 255) / 256) * ((N + 127) / 128) >= ((int64_t)1 << 24))
        return NVFP4_ERR_SHAPE;
    if (((uintptr_t)X & 15u) != 0 || ((uintptr_t)codes & 15u) != 0 || ((uintptr_t)Y & 15u) != 0 ||
        ((uintptr_t)alpha & 3u) != 0)
        return NVFP4_ERR_INVALID_ARG;
    return NVFP4_OK;
}
}  // namespace

NVFP4_API size_t nvfp4_matmul_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (M <= 0 || K <= 0 || N <= 0 || K % 16 != 0 || N > ((int64_t)1 << 25) || N > kMaxElems / K ||
        M > kMaxElems / K || M > kMaxElems / N || ((M + 255) / 256) * ((N + 127) / 128) >= ((int64_t)1 << 24))
        return 0;
    return nvfp4::plan_w4a16(M, K, N).part_bytes;
}

NVFP4_API int nvfp4_matmul_plan(int64_t M, int64_t K, int64_t N, int64_t *plan_out) {
    if (!plan_out || M <= 0 || K <= 0 || N <= 0 || K % 16 != 0) return NVFP4_ERR_INVALID_ARG;
    const nvfp4::W4a16Plan p = nvfp4::plan_w4a16(M, K, N);
    const int64_t v[10] = {p.kind, p.tm, p.tn, p.tiles_n, p.tiles, p.slices, p.kslice, p.grid, p.reduce_grid,
                           (int64_t)p.part_bytes};
    for (int i = 0; i < 10; ++i) plan_out[i] = v[i];
    return NVFP4_OK;
}

NVFP4_API int nvfp4_matmul_ex(const void *X, int64_t M, int64_t K, const uint8_t *codes, const uint8_t *scales,
                              const float *alpha, int64_t N, void *Y, int y_dtype, void *workspace,
                              size_t workspace_bytes, void *stream) {
    const int c = matmul_check(X, M, K, codes, scales, alpha, N, Y, y_dtype);
    if (c != NVFP4_OK) return c;
    if (workspace && ((uintptr_t)workspace & 255u) != 0) return NVFP4_ERR_INVALID_ARG;
    const nvfp4::W4a16Plan plan = nvfp4::plan_w4a16(M, K, N);
    const size_t need = plan.part_bytes;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (workspace && need > 0 && workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (plan.kind == nvfp4::kW4a16Gemm && plan.tn == 128) {
        // The 128 x 128 and 256 x 128 tile forms are not run under stream capture (see the header).
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cs) != hipSuccess) return NVFP4_ERR_HIP;
        if (cs != hipStreamCaptureStatusNone) return NVFP4_ERR_UNSUPPORTED;
    }
    const bool f32 = y_dtype == NVFP4_DTYPE_F32;
    const uint16_t *x = static_cast<const uint16_t *>(X);
    if (need == 0 || workspace) {
        return nvfp4::launch_w4a16(x, M, K, codes, scales, alpha, N, Y, f32, static_cast<float *>(workspace), st) ==
                       hipSuccess
                   ? NVFP4_OK
                   : NVFP4_ERR_HIP;
    }
    void *ws = nullptr;
    if (hipMallocAsync(&ws, need, st) != hipSuccess) return NVFP4_ERR_HIP;
    const bool ok =
        nvfp4::launch_w4a16(x, M, K, codes, scales, alpha, N, Y, f32, static_cast<float *>(ws), st) == hipSuccess;
    if (hipFreeAsync(ws, st) != hipSuccess) return NVFP4_ERR_HIP;
    return ok ? NVFP4_OK : NVFP4_ERR_HIP;
}

NVFP4_API int nvfp4_matmul(const void *X, int64_t M, int64_t K, const uint8_t *codes, const uint8_t *scales,
                           const float *alpha, int64_t N, void *Y, int y_dtype, void *stream) {
    return nvfp4_matmul_ex(X, M, K, codes, scales, alpha, N, Y, y_dtype, nullptr, 0, stream);
}

namespace {
constexpr int64_t kGptqMaxCols = 32768;
constexpr int64_t kGptqMaxElems = (int64_t)1 << 32;
constexpr int64_t kGptqMaxRows = (int64_t)65535 * 64;  // row tiles of 64 along the update grid's y

bool gptq_shape_ok(int64_t rows, int64_t cols) {
    return cols % 16 == 0 && cols <= kGptqMaxCols && rows <= kGptqMaxElems / cols && rows <= kGptqMaxRows;
}
}  // namespace

NVFP4_API size_t nvfp4_gptq_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0 || !gptq_shape_ok(rows, cols)) return 0;
    return nvfp4::gptq_workspace_bytes(rows, cols);
}

NVFP4_API int nvfp4_gptq(const void *W, int dtype, int64_t rows, int64_t cols, const double *H, double percdamp,
                         uint8_t *codes_out, uint8_t *scales_out, float *alpha_out, void *workspace,
                         size_t workspace_bytes, void *stream) {
    if (!W || !H || !codes_out || !scales_out || !alpha_out || rows <= 0 || cols <= 0) return NVFP4_ERR_INVALID_ARG;
    if (dtype != NVFP4_DTYPE_BF16 && dtype != NVFP4_DTYPE_F32) return NVFP4_ERR_INVALID_ARG;
    if (!(percdamp >= 0.0) || !(percdamp < INFINITY)) return NVFP4_ERR_INVALID_ARG;
    if (!gptq_shape_ok(rows, cols)) return NVFP4_ERR_SHAPE;
    if (((uintptr_t)W & 15u) != 0 || ((uintptr_t)H & 7u) != 0 || ((uintptr_t)codes_out & 7u) != 0 ||
        ((uintptr_t)alpha_out & 3u) != 0 || (workspace && ((uintptr_t)workspace & 255u) != 0))
        return NVFP4_ERR_INVALID_ARG;
    const size_t need = nvfp4::gptq_workspace_bytes(rows, cols);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool f32 = dtype == NVFP4_DTYPE_F32;
    if (workspace) {
        if (workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
        return nvfp4::launch_gptq(W, f32, rows, cols, H, percdamp, codes_out, scales_out, alpha_out, workspace,
                                  st) == hipSuccess
                   ? NVFP4_OK
                   : NVFP4_ERR_HIP;
    }
    void *ws = nullptr;
    if (hipMallocAsync(&ws, need, st) != hipSuccess) return NVFP4_ERR_HIP;
    const bool ok =
        nvfp4::launch_gptq(W, f32, rows, cols, H, percdamp, codes_out, scales_out, alpha_out, ws, st) == hipSuccess;
    if (hipFreeAsync(ws, st) != hipSuccess) return NVFP4_ERR_HIP;
    return ok ? NVFP4_OK : NVFP4_ERR_HIP;
}

NVFP4_API const char *nvfp4_status_string(int status) {
    switch (status) {
        case NVFP4_OK: return "ok";
        case NVFP4_ERR_INVALID_ARG: return "invalid argument";
        case NVFP4_ERR_SHAPE: return "unsupported shape (a dimension that must be a multiple of 16 is not, or a size limit is exceeded)";
        case NVFP4_ERR_WORKSPACE: return "workspace too small";
        case NVFP4_ERR_HIP: return "HIP launch or allocation failed";
        case NVFP4_ERR_TOO_LARGE: return "the call needs more scratch than the library's fixed device array holds";
        case NVFP4_ERR_UNSUPPORTED: return "not supported under stream capture for this shape (128 x 128 or 256 x 128 product tiles)";
        default: return "unknown status";
    }
}
