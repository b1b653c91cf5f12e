/*
 * NVFP4 weight-quantizer ORACLE — host-only C interface.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg load this
 * library. The product library (include/nvfp4.h) never links, loads or calls it, and the two share no
 * code, headers, tables or helpers.
 *
 * Every pointer is a host pointer owned by the caller. All calls are synchronous and single-threaded.
 * Layout matches the product library: W is row-major [rows][cols], a block is 16 consecutive elements
 * of one row (block b of the matrix covers elements 16b..16b+15 of the flat array), codes are
 * [rows][cols/2] bytes with the even column in the low nibble, scales are [rows][cols/16] E4M3 bytes.
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { NVFP4_REF_BF16 = 0, NVFP4_REF_F32 = 1 };
enum { NVFP4_REF_MAX = 0, NVFP4_REF_FOUR_OVER_SIX = 1, NVFP4_REF_CJSO = 2, NVFP4_REF_SOAR = 3 };
/* Starting point of CJSO (and so of SOAR): the max rule, or FourOverSix's block scales. */
enum { NVFP4_REF_INIT_MAX = 0, NVFP4_REF_INIT_4O6 = 1 };

/* Returns 0, 1 when W holds a NaN or an infinity (then alpha = NaN and every code, scale and mchoice
 * byte is 0), or -1 on a bad argument (null pointer, rows or cols <= 0, cols % 16 != 0, unknown
 * dtype or mode, iters < 0).
 * mchoice (nullable): one byte per block, 1 where FourOverSix kept M=4 (mode 1 only; 0 otherwise).
 * dstar   (nullable): per block, the CJSO block scale before its FP8 rounding (modes 2 and 3; for
 *                     iters = 0 the max-rule quotient); in mode 3 this is the value the search used.
 * alpha_trace (nullable): iters+1 floats, alpha after initialisation and after each alpha-step. */
int nvfp4_ref_quantize(const void *W, int dtype, int64_t rows, int64_t cols, int mode, int iters,
                       uint8_t *codes, uint8_t *scales, float *alpha, uint8_t *mchoice, double *dstar,
                       float *alpha_trace);

/* Same, with CJSO/SOAR started from `init` (NVFP4_REF_INIT_*; modes 0 and 1 accept only INIT_MAX). With
 * INIT_4O6 the first scales are FourOverSix's (alpha from the max rule); mchoice is written only in
 * mode 1. */
int nvfp4_ref_quantize_ex(const void *W, int dtype, int64_t rows, int64_t cols, int mode, int iters, int init,
                          uint8_t *codes, uint8_t *scales, float *alpha, uint8_t *mchoice, double *dstar,
                          float *alpha_trace);

/* Reconstruct-scale rules of the decoupled search (R8, R11): the E4M3 pair bracketing the unrounded
 * CJSO scale (the pages' rule), the candidate's quantisation scale Delta_q, or the least-squares scale
 * of the candidate's own codes. */
enum { NVFP4_REF_DD_CJSO = 0, NVFP4_REF_DD_QUANT = 1, NVFP4_REF_DD_LSQ = 2 };

/* SOAR (mode 3) with a configurable search: multipliers f_k = binary32 nearest (num0 + k)/den for
 * k = 0..count-1 and reconstruct pairs by dd_rule. (50, 100, 101, NVFP4_REF_DD_CJSO) is the search of
 * nvfp4_ref_quantize_ex. Returns as nvfp4_ref_quantize_ex, and -1 for a grid outside 1 <= den <= 2^24,
 * num0 >= 1, 1 <= count <= 1024, (num0 + count - 1) / den <= 16, or an unknown rule. */
int nvfp4_ref_quantize_search(const void *W, int dtype, int64_t rows, int64_t cols, int iters, int init,
                              int num0, int den, int count, int dd_rule, uint8_t *codes, uint8_t *scales,
                              float *alpha, double *dstar);

/* Decoupled-scale search on selected blocks, given the CJSO state of the whole matrix (alpha, the
 * E4M3 block scales dcode[] and the pre-rounding scales dstar[], one per block of the matrix).
 * blocks[] lists nsel block indices; codes_sel is nsel*8 bytes, scales_sel nsel bytes. */
int nvfp4_ref_soar_blocks(const void *W, int dtype, int64_t rows, int64_t cols, float alpha,
                          const uint8_t *dcode, const double *dstar, const int64_t *blocks, int64_t nsel,
                          uint8_t *codes_sel, uint8_t *scales_sel);
/* The same with the search of nvfp4_ref_quantize_search. */
int nvfp4_ref_soar_blocks_search(const void *W, int dtype, int64_t rows, int64_t cols, float alpha,
                                 const uint8_t *dcode, const double *dstar, const int64_t *blocks, int64_t nsel,
                                 int num0, int den, int count, int dd_rule, uint8_t *codes_sel,
                                 uint8_t *scales_sel);

/* Mean squared reconstruction error sum((w - e2m1(code)*e4m3(scale)*alpha)^2)/n of an output triple. */
/* W4A16 product Y = X * What^T (What = dequantised [N][K] weights), exact products summed in binary128,
 * rounded to binary64. X is [M][K] (x_dtype), codes/scales/alpha as written by the quantiser for the
 * [N][K] matrix, Y is [M][N]. */
int nvfp4_ref_matmul(const void *X, int x_dtype, int64_t M, int64_t K, const uint8_t *codes,
                     const uint8_t *scales, float alpha, int64_t N, double *Y);

double nvfp4_ref_mse(const void *W, int dtype, int64_t rows, int64_t cols, const uint8_t *codes,
                     const uint8_t *scales, float alpha);

/* Dequantised matrix in binary64: out[i] = e2m1(code_i) * e4m3(scale_block(i)) * alpha (exact). */
void nvfp4_ref_dequantize(const uint8_t *codes, const uint8_t *scales, float alpha, int64_t rows,
                          int64_t cols, double *out);

/* Format codecs and single steps, exposed so the tests can pin them one by one. */
unsigned nvfp4_ref_e2m1_code(float x);
float nvfp4_ref_e2m1_value(unsigned code);
double nvfp4_ref_e4m3_value(unsigned code);
unsigned nvfp4_ref_e4m3_rne(double v);
void nvfp4_ref_e4m3_bracket(double v, unsigned *lo, unsigned *hi);
float nvfp4_ref_search_multiplier(int k);
float nvfp4_ref_grid_multiplier(int num0, int den, int k);
void nvfp4_ref_e2m1_codes(const float *x, int64_t n, uint8_t *out);
void nvfp4_ref_e4m3_rne_many(const double *v, int64_t n, uint8_t *out);
void nvfp4_ref_quantize_block(const float *w16, float alpha, float delta, uint8_t *codes16);
double nvfp4_ref_block_err(const float *w16, const uint8_t *codes16, float alpha, double delta_d);
/* alpha-step on nblk blocks of 16 floats with fixed E4M3 block scales and fixed codes (one code per
 * byte); returns 1 and sets *alpha when the denominator is positive; *num and *den receive the sums. */
int nvfp4_ref_alpha_step(const float *w, int64_t nblk, const uint8_t *dcode, const uint8_t *codes16,
                         float *alpha, double *num, double *den);
/* block-scale step on one block; returns 1 and sets *dstar when some code is nonzero. */
int nvfp4_ref_delta_step(const float *w16, const uint8_t *codes16, float alpha, double *dstar);

#ifdef __cplusplus
}
#endif
#endif
