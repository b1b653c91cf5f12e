/*
 * nvfp4.h - C ABI of the MI355X (gfx950) NVFP4 weight quantizer.
 *
 * What the calls compute:
 *   NVFP4 quantisation of a weight matrix W into FP4 (E2M1) codes Q, one FP8 (E4M3) scale Delta_i per
 *   block of 16 consecutive elements of a row, and one FP32 global scale alpha, so that
 *   W ~ Q * Delta_i * alpha. The four modes are the ones the two pages describe:
 *     NVFP4_MODE_MAX           the max rule of the SOAR page ("SOAR: Scale Optimization for Accurate
 *                              Reconstruction in NVFP4 Quantization", quantisation equations):
 *                              alpha = max|W| / (6*448), Delta_i = E4M3(max|W_i| / (6*alpha)).
 *     NVFP4_MODE_FOUR_OVER_SIX the FourOverSix choice of the write-up "SOAR 周冠军笔记 07 |
 *                              香草小张：NVFP4 量化改进与推测解码实践", section 02: per block, the M=4
 *                              scale E4M3(1.5*Delta_i) replaces Delta_i when its squared reconstruction
 *                              error is strictly smaller.
 *     NVFP4_MODE_CJSO          the SOAR page's closed-form joint scale optimisation: from the max rule,
 *                              `iters` rounds of {least-squares alpha, re-quantise, least-squares Delta_i
 *                              rounded to E4M3, re-quantise}.
 *     NVFP4_MODE_SOAR          CJSO followed by the SOAR page's decoupled search: per block, quantise with
 *                              Delta_q = Delta_c * f (f = 0.50, 0.51, ..., 1.50) and reconstruct with
 *                              Delta_d, one of the two E4M3 values around the unrounded CJSO scale; keep
 *                              the least squared error (202 candidates, CJSO's own point first, strict <).
 *   Arithmetic: scaled values are x = w * (1/(alpha*Delta)) in binary32, rounded to the nearest E2M1
 *   value with ties to the even code and |x| > 6 saturating to 6 (a value rounding to 0 gets code 0);
 *   every choice between candidates compares exact squared errors. The results are bit-identical to
 *   the CPU oracle that defines them.
 *
 * Layout (row-major, contiguous, caller-owned):
 *   W          [rows][cols] bf16 (nvfp4_quantize) or fp32 (nvfp4_quantize_f32), 16-byte aligned.
 *   codes_out  [rows][cols/2] bytes, 8-byte aligned: byte k of a row holds column 2k in its low nibble
 *              and column 2k+1 in its high nibble; a code is sign (bit 3) | index into
 *              {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 *   scales_out [rows][cols/16] E4M3 bytes (sign bit 0; at most 0x7E = 448).
 *   alpha_out  one float. Dequantisation: w_hat = e2m1(code) * e4m3(scale) * alpha.
 *   All pointers are device pointers (hipMalloc'd or torch CUDA tensors); `stream` is a hipStream_t
 *   (NULL = the default stream).
 *
 * Calls are asynchronous: they validate their arguments on the host, enqueue kernels on `stream` and
 * return. Results are valid once the stream has reached that point. The library keeps no pointer after
 * the enqueued work ends and has no mutable global state: calls on different streams may overlap, and
 * calls that share output buffers must be ordered by the caller.
 *
 * Errors: negative return values are reported synchronously and nothing is enqueued, except
 * NVFP4_ERR_HIP (a launch or allocation failed; work enqueued before the failure may still run).
 * Data-dependent conditions are reported in band: a NaN or an infinity anywhere in W gives
 * alpha_out = NaN and all-zero codes and scales (and sets NVFP4_STATUS_NONFINITE in the stats); an
 * all-zero W gives alpha = 0 with all-zero codes and scales.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum nvfp4_mode {
    NVFP4_MODE_MAX = 0,
    NVFP4_MODE_FOUR_OVER_SIX = 1,
    NVFP4_MODE_CJSO = 2,
    NVFP4_MODE_SOAR = 3
};

enum nvfp4_dtype { NVFP4_DTYPE_BF16 = 0, NVFP4_DTYPE_F32 = 1 };

/* How the SOAR search picks each candidate's two E4M3 reconstruct scales Delta_d (SOAR page, decoupled
 * search: "the two E4M3 values nearest the current value"). CJSO: the pair around the unrounded CJSO
 * scale, for every candidate (the reading of the page the default search takes). QUANT: the pair
 * around the candidate's quantisation scale Delta_q. LSQ: the pair around the least-squares scale of
 * the candidate's own codes (the block-scale step applied to them; a candidate whose codes are all
 * zero keeps Delta_c). */
enum nvfp4_dd_rule { NVFP4_DD_CJSO = 0, NVFP4_DD_QUANT = 1, NVFP4_DD_LSQ = 2 };
#define NVFP4_SEARCH_MAX_COUNT 1024

enum nvfp4_error {
    NVFP4_OK = 0,
    NVFP4_ERR_INVALID_ARG = -1, /* null or misaligned pointer, rows/cols <= 0, unknown mode or dtype,
                                   iters outside [0, 1000] */
    NVFP4_ERR_SHAPE = -2,       /* cols % 16 != 0, or more than 2^35 elements */
    NVFP4_ERR_WORKSPACE = -3,   /* caller workspace smaller than nvfp4_workspace_bytes() */
    NVFP4_ERR_HIP = -4,         /* a HIP call failed */
    NVFP4_ERR_TOO_LARGE = -5,   /* nvfp4_quantize_noalloc: the call needs more scratch than its fixed
                                   device array holds */
    NVFP4_ERR_UNSUPPORTED = -6  /* nvfp4_matmul / nvfp4_matmul_ex on a capturing stream with a shape
                                   that takes the 128 x 128 or 256 x 128 output tiles */
};

/* In-band status bits, written to nvfp4_stats_t.status by the device. */
#define NVFP4_STATUS_NONFINITE 1u

/* Optional per-call statistics in device memory (written by the call). */
typedef struct nvfp4_stats {
    uint32_t status;    /* NVFP4_STATUS_* bits */
    uint32_t m4_blocks; /* FourOverSix: number of blocks that kept M=4 */
    uint32_t reserved[2];
} nvfp4_stats_t;

/* Quantise a bf16 matrix. `iters` is the number of CJSO rounds (modes 2 and 3; ignored otherwise,
 * 0 makes CJSO equal to MAX). A scratch workspace is taken from a stream-ordered pool and given
 * back on the same stream. */
int nvfp4_quantize(const void *W, int64_t rows, int64_t cols, int mode, int iters, uint8_t *codes_out,
                   uint8_t *scales_out, float *alpha_out, void *stream);

/* Same for an fp32 matrix. */
int nvfp4_quantize_f32(const float *W, int64_t rows, int64_t cols, int mode, int iters,
                       uint8_t *codes_out, uint8_t *scales_out, float *alpha_out, void *stream);

/* Full argument set. */
typedef struct nvfp4_args {
    const void *W;
    int dtype; /* enum nvfp4_dtype */
    int64_t rows, cols;
    int mode; /* enum nvfp4_mode */
    int iters;
    uint8_t *codes_out;
    uint8_t *scales_out;
    float *alpha_out;
    uint8_t *mchoice_out;     /* nullable: [rows][cols/16] bytes, 1 where FourOverSix kept M=4 (mode 1) */
    nvfp4_stats_t *stats_out; /* nullable, device memory */
    void *workspace;          /* nullable: device memory of workspace_bytes, 256-byte aligned; NULL =
                                 the library allocates on `stream` */
    size_t workspace_bytes;
    void *stream;             /* hipStream_t */
    void *const *stage_events; /* nullable: nvfp4_kernel_count(mode, iters) + 1 hipEvent_t handles; the
                                  call records stage_events[0] before its first kernel and
                                  stage_events[j + 1] after kernel j, so each kernel can be timed on
                                  `stream`; NULL entries are skipped (fewer records, smaller gaps) */
    int n_stage_events;
    unsigned flags; /* NVFP4_FLAG_* bits (0 for the defaults) */
    /* SOAR search grid (mode 3; all three 0 elsewhere and for the page's grid, f_k = (50 + k)/100 for
     * k = 0..100): multipliers f_k = the binary32 value nearest (search_num0 + k) / search_den for
     * k < search_count, with 1 <= search_den <= 2^24, search_num0 >= 1,
     * 1 <= search_count <= NVFP4_SEARCH_MAX_COUNT and search_num0 + search_count - 1 <= 16 * search_den
     * (multipliers at most 16). Any other setting is NVFP4_ERR_INVALID_ARG. */
    int search_num0, search_den, search_count;
    int dd_rule; /* enum nvfp4_dd_rule (mode 3; 0 elsewhere). QUANT and LSQ scan every multiplier. */
} nvfp4_args_t;

/* SOAR: visit all 202 candidates of every block. Without it the search evaluates, per reconstruct
 * scale, only the two or three quantise scales next to it, which is exact: the block error is
 * unimodal in the quantise scale around that window (the kernel source gives the argument), so the
 * outputs are identical either way. The flag exists to check that and to time the full search. */
#define NVFP4_FLAG_FULL_SEARCH 1u
/* CJSO and SOAR: start from FourOverSix's block scales (each block's M=6 or M=4 choice, FourOverSix
 * write-up, section 02) instead of the max rule; alpha still starts from the max rule. For SOAR with no
 * rounds, the unrounded scale whose E4M3 neighbours the search tries is max|w|/(6 alpha), or 1.5*Delta6
 * for a block that took M=4. Not accepted for modes 0 and 1. */
#define NVFP4_FLAG_INIT_4O6 2u

int nvfp4_quantize_ex(const nvfp4_args_t *args);

/* nvfp4_quantize_ex for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. It allocates nothing (no hipMalloc, hipMallocAsync or
 * hipFree, neither here nor in any library it calls): its scratch is a fixed device array inside the
 * library, of nvfp4_noalloc_scratch_bytes() = 16 MiB, that every GPU the library runs on holds until the
 * process ends. The array of the current device is used, so the current device must be the stream's.
 * Same arguments, outputs and errors as nvfp4_quantize_ex, except:
 *   - args->workspace must be NULL and args->workspace_bytes 0 (else NVFP4_ERR_INVALID_ARG);
 *   - NVFP4_ERR_TOO_LARGE when nvfp4_workspace_bytes(rows, cols, mode) exceeds the array: MAX,
 *     FourOverSix and CJSO need 35 KB whatever the size; SOAR needs 2 more bytes per 16-element block,
 *     which caps it at about 134 million elements;
 *   - the first call on a device looks up that device's address of the array (NVFP4_ERR_HIP if that
 *     fails).
 * All calls on one GPU share its array: two calls that may overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller. Nothing in the array needs clearing between calls. */
int nvfp4_quantize_noalloc(const nvfp4_args_t *args);

/* Size in bytes of the fixed device array nvfp4_quantize_noalloc uses. */
size_t nvfp4_noalloc_scratch_bytes(void);

/* Number of kernels one call of this mode enqueues (MAX and FourOverSix: 2; CJSO: iters + 2; SOAR:
 * iters + 3; the last SOAR kernel is the decoupled search), or -1 for an unknown mode or bad iters. */
int nvfp4_kernel_count(int mode, int iters);

/* Device scratch needed by one call with these arguments (0 for an invalid shape). */
size_t nvfp4_workspace_bytes(int64_t rows, int64_t cols, int mode);

/* Round n binary32 values to E2M1 codes (one code per output byte, same rule as the quantiser:
 * nearest, ties to the even code, saturating at 6, NaN -> 0, negative results that round to zero ->
 * code 0). x and codes are device pointers; n <= 2^35 (else NVFP4_ERR_SHAPE). */
int nvfp4_encode_e2m1(const float *x, int64_t n, uint8_t *codes, void *stream);

/* The binary32 reciprocal the decoupled search uses for its quantisation scales (the candidates
 * x = w * fl(1/s) of the SOAR page's decoupled search), element-wise: r[i] = fl(1/s[i]), the correctly
 * rounded reciprocal for every input (for 2^-125 <= s < 2^125 it is computed from the hardware's
 * approximate reciprocal and one residual correction; elsewhere by IEEE division). Exported so that the
 * equality with IEEE division can be checked on the device. s and r are device pointers (4-byte
 * aligned, may not overlap); n <= 2^35 (else NVFP4_ERR_SHAPE). */
int nvfp4_reciprocal_f32(const float *s, int64_t n, float *r, void *stream);

/* Dequantise codes/scales/alpha (device pointers, layout above; alpha is a device pointer to one
 * float) into out [rows][cols] as bf16 (out_dtype 0) or fp32 (out_dtype 1):
 * out = e2m1(code) * e4m3(scale) * alpha, rounded once to the output type (SOAR page, dequantisation
 * equation). */
int nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, const float *alpha, int64_t rows,
                     int64_t cols, void *out, int out_dtype, void *stream);

/* Reconstruction statistics of an encoding of W (SOAR page, dequantisation: w is reconstructed as
 * e2m1(code) * e4m3(scale) * alpha). W is [rows][cols] of dtype (enum nvfp4_dtype); codes, scales and
 * alpha are laid out as the quantiser writes them (scale sign bits are ignored). All pointers are device
 * pointers. On completion of the stream work:
 *   sse_out[0]  = sum over elements of d^2, d = w - (q * alpha) * Delta formed in binary64 (exact up to the
 *                 rounding of that difference) and the squares summed as double-doubles, then rounded to
 *                 binary64 (mean squared error = sse / (rows * cols));
 *   hist_out[c] = number of elements whose 4-bit code is c, c = 0..15.
 * Scratch is taken from a stream-ordered pool and given back on the same stream. Errors: as
 * nvfp4_quantize (arguments are checked on the host; nothing is enqueued on error). */
int nvfp4_error_stats(const void *W, int dtype, int64_t rows, int64_t cols, const uint8_t *codes,
                      const uint8_t *scales, const float *alpha, double *sse_out,
                      unsigned long long *hist_out, void *stream);

/* W4A16 product with NVFP4 weights, the use the format exists for: Y[M][N] = X[M][K] * What[N][K]^T with
 * What = e2m1(code) * e4m3(scale) * alpha (SOAR page, dequantisation equation), for a weight matrix [N][K]
 * stored as the quantiser writes it (codes [N][K/2], scales [N][K/16], alpha one float). X is bf16
 * [M][K] row-major; Y is [M][N] of y_dtype (NVFP4_DTYPE_BF16 or _F32). All pointers are device pointers;
 * X, codes and Y 16-byte aligned; K % 16 == 0, N <= 2^25 and fewer than 2^24 output tiles of 256 x 128
 * (else NVFP4_ERR_SHAPE). Arithmetic: every q * Delta is a bf16 value,
 * so the products with X are exact; the sum over k is accumulated in fp32 (packed bf16 dot products when
 * M <= 4, M * K * 2 <= 128 KiB and K <= 16384; bf16 MFMA otherwise) in an order the caller does not
 * control, then multiplied by alpha and
 * rounded once to the output type. When the output tiles are too few to fill the GPU, K is split and the
 * slices' fp32 sums (slices * M * N * 4 bytes, at most 1 GiB) go through scratch taken from a
 * stream-ordered pool and given back on the same stream; the slices are added in a fixed order, so
 * results are reproducible. Enqueued on `stream`; argument errors are returned synchronously. */
int nvfp4_matmul(const void *X, int64_t M, int64_t K, const uint8_t *codes, const uint8_t *scales,
                 const float *alpha, int64_t N, void *Y, int y_dtype, void *stream);

/* nvfp4_matmul with caller-supplied scratch for the K split: `workspace` (device memory, 256-byte aligned,
 * nullable) of `workspace_bytes` >= nvfp4_matmul_workspace_bytes(M, K, N) bytes. With a workspace nothing
 * is allocated, so the call may be captured into a HIP graph as plain kernel nodes; the workspace must then
 * stay allocated while the graph may run. NULL behaves as nvfp4_matmul. NVFP4_ERR_WORKSPACE if it is too
 * small. Same arithmetic, layout and errors as nvfp4_matmul.
 * Stream capture: shapes whose plan takes the 128 x 128 or 256 x 128 output tiles (nvfp4_matmul_plan:
 * kernel 2, tile columns 128) are refused on a capturing stream with NVFP4_ERR_UNSUPPORTED (nothing is
 * enqueued): one graph-captured run of those forms ended in a device memory fault whose cause has not been
 * found. The GEMV, the skinny kernel and the 128 x 64 tiles (with or without the K split) may be
 * captured. Eager calls of every shape are unaffected. */
int nvfp4_matmul_ex(const void *X, int64_t M, int64_t K, const uint8_t *codes, const uint8_t *scales,
                    const float *alpha, int64_t N, void *Y, int y_dtype, void *workspace, size_t workspace_bytes,
                    void *stream);

/* Scratch bytes nvfp4_matmul_ex needs for these shapes: slices * M * N * 4 when K is split, else 0 (also 0
 * for shapes nvfp4_matmul rejects). */
size_t nvfp4_matmul_workspace_bytes(int64_t M, int64_t K, int64_t N);

/* The launch nvfp4_matmul takes for these shapes, for tests and tuning (no device work): plan_out[10] gets
 * {kernel (0 GEMV, 1 skinny MFMA, 2 tiled MFMA), tile rows (tiled; the rows of X compiled for, skinny),
 * tile columns, tiles along N, tiles, K slices, K per slice, work-groups, reduction work-groups, scratch
 * bytes}. Returns NVFP4_ERR_INVALID_ARG for a null pointer, a dimension <= 0 or K % 16 != 0. */
int nvfp4_matmul_plan(int64_t M, int64_t K, int64_t N, int64_t *plan_out);

/* GPTQ with the FourOverSix block scales fixed first (FourOverSix write-up, section 03: every block's
 * scale and its M = 6 / M = 4 choice are settled before GPTQ's weight iterations, which then run inside
 * that frame; GPTQ as published by Frantar, Ashkboos, Hoefler and Alistarh, 2022).
 *
 * Steps:
 *   1. The frame. scales_out and alpha_out are exactly nvfp4_quantize's FourOverSix result for W.
 *   2. GPTQ's preparation of H [cols][cols], the second moment of the layer's inputs. Inputs with a zero
 *      diagonal are dead: their weights count as zero and their diagonal as one. Every diagonal entry then
 *      gains percdamp * mean(diagonal).
 *   3. The columns in order. Each is quantised to the nearest E2M1 value of w~ / s in binary64, where
 *      s = fl32(alpha * Delta) of its block (ties to the even code; s = 0 gives code 0). Its error is spread
 *      over the later columns as GPTQ specifies: given the columns already fixed, the later weights are the
 *      minimiser of the H-weighted error. All of this runs in binary64.
 *   codes_out gets the resulting codes.
 *
 * Arguments:
 *   W           [rows][cols], dtype bf16 or fp32, 16-byte aligned.
 *   H           device binary64, row-major, symmetric; only its upper triangle (H[i][j], i <= j) is read.
 *   percdamp    finite and >= 0 (GPTQ's usual value is 0.01).
 *   codes_out, scales_out, alpha_out
 *               as for nvfp4_quantize.
 *   workspace   nullable; 256-byte aligned, of nvfp4_gptq_workspace_bytes(rows, cols) bytes, about
 *               8 * (cols^2 + rows * cols) bytes. NULL = the library allocates on `stream` and gives the
 *               scratch back on `stream`.
 *
 * Limits: cols % 16 == 0, cols <= 32768, rows <= 65535 * 64 and rows * cols <= 2^32 (else
 *         NVFP4_ERR_SHAPE).
 *
 * Errors:
 *   - Arguments are checked on the host, as for nvfp4_quantize.
 *   - If the damped H is not positive definite in binary64 (a Cholesky pivot that is not positive and
 *     finite), alpha_out = NaN and every code is 0 when the stream work ends.
 *   - A NaN or infinity in W gives FourOverSix's in-band result (alpha NaN, all-zero codes and scales). */
int nvfp4_gptq(const void *W, int dtype, int64_t rows, int64_t cols, const double *H, double percdamp,
               uint8_t *codes_out, uint8_t *scales_out, float *alpha_out, void *workspace,
               size_t workspace_bytes, void *stream);

/* Device scratch one nvfp4_gptq call needs (0 for an invalid shape). */
size_t nvfp4_gptq_workspace_bytes(int64_t rows, int64_t cols);

/* Text of an nvfp4_error value. */
const char *nvfp4_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif
