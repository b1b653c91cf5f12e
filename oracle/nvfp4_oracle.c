/*
 * NVFP4 weight-quantizer ORACLE: a plain, slow, single-threaded CPU implementation in C.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * this library. The product library never links, loads or calls it, and the two share no code.
 *
 * It follows two pages:
 *   [4/6]  "SOAR 周冠军笔记 07 | 香草小张：NVFP4 量化改进与推测解码实践" (openbmb.cn blog), section
 *          "02 FourOverSix：在 M=6 与 M=4 之间自适应选择": the FP4 (E2M1) value set and the per-block
 *          choice between the block scales of M=6 and M=4.
 *   [SOAR] "SOAR: Scale Optimization for Accurate Reconstruction in NVFP4 Quantization"
 *          (july-h5kf3.github.io, tag feed "soar"): the max rule (equations for alpha and Delta_i), the
 *          piecewise FP4 rounding, the CJSO objective and its closed-form global and block scales, and
 *          the decoupled quantise/dequantise block-scale search.
 *
 * Readings taken where the pages leave a step open (each is stated again where it is used):
 *   R1 FP4 rounding goes to the nearest E2M1 value with ties to the even code (the page's rounding
 *      brackets are garbled), |x| > 6 saturates to 6, and a value that rounds to zero has code 0.
 *   R2 FP8 (E4M3, bias 7, no infinities, largest value 448) rounding goes to the nearest value with ties
 *      to the even code; anything above 448 becomes 448.
 *   R3 The quantiser's arithmetic is binary32: s = fl(alpha*Delta), r = fl(1/s), x = fl(w*r). A zero s
 *      quantises a whole block to code 0.
 *   R4 alpha = fl(max|W| / 2688) in binary32; the block scale is the E4M3 rounding of the real quotient
 *      max|W_i| / (6 alpha) (decided exactly through binary64).
 *   R5 Errors are exact: the reconstruction of w is Q*alpha*Delta_d as a real number and each block's
 *      squared error is summed without loss (binary128), so choices never hinge on rounding.
 *   R6 The printed alpha* fraction is garbled (alpha stands where Delta_i belongs); the least-squares
 *      minimiser over alpha of the CJSO objective is used.
 *   R7 CJSO order: alpha-step, re-quantise, Delta-step (rounded to E4M3), re-quantise; T rounds; a zero
 *      denominator keeps the previous scale.
 *   R8 Search: multipliers f_k = binary32 nearest (50+k)/100 for k = 0..100, Delta_q = fl(Delta_c*f_k);
 *      Delta_d from the two E4M3 values bracketing the CJSO scale before its FP8 rounding; the CJSO
 *      point is the incumbent and only a strictly smaller error replaces it (order k up, lower
 *      Delta_d first). alpha is left as CJSO produced it.
 *   R9 Blocks are 16 consecutive elements of a row; input with a NaN or an infinity yields alpha = NaN
 *      and all-zero codes and scales; an all-zero matrix yields alpha = 0.
 *   R10 CJSO started from FourOverSix (a composition the pages suggest, not a mode they define): the
 *      first scales are FourOverSix's choice under the max-rule alpha; the "unrounded" value of a chosen
 *      Delta4 is 1.5*Delta6, the quantity FourOverSix rounds to get it (for Delta6 it is max|w|/(6 alpha)).
 *   R11 Search variants (not modes the pages define): the grid f_k = binary32 nearest (num0+k)/den,
 *      k < count (R8 is 50, 100, 101); and the reconstruct pair of each candidate taken as the E4M3
 *      values bracketing either its Delta_q or the least-squares scale of its own codes (the block-scale
 *      step's binary64 quotient; a block whose codes are all zero keeps {Delta_c, Delta_c}), in place of
 *      R8's bracket of the unrounded CJSO scale. The incumbent, the visiting order and the strict
 *      improvement rule stay as in R8.
 *
 * Build: gcc -O2 -std=gnu11 -ffp-contract=off (no fast-math): every float expression below is the
 * IEEE operation it spells, in the order written.
 */
#include "nvfp4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

typedef __float128 quad;

/* ------------------------------------------------------------------------------------------------ */
/* Number formats                                                                                   */
/* ------------------------------------------------------------------------------------------------ */

/* [4/6] §01 lists the NVFP4 values {0, ±0.5, ±1, ±1.5, ±2, ±3, ±4, ±6}; [SOAR] gives M_FP4 = 6. The
 * code of a magnitude is its position in this list, bit 3 carries the sign. */
static const float E2M1_MAGNITUDE[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

float nvfp4_ref_e2m1_value(unsigned code) {
    float v = E2M1_MAGNITUDE[code & 7u];
    return (code & 8u) ? -v : v;
}

/* [SOAR] piecewise FP4 rounding of t = |x|: below 2 the spacing is 0.5 (½·round(2t)), on [2,4] it is 1
 * (round(t)), on [4,6] it is 2 (2·round(t/2)). R1: round = half-to-even (rintf in the default mode),
 * which puts every tie on the even code; t > 6 (and infinity) saturates to 6; NaN gives 0. */
unsigned nvfp4_ref_e2m1_code(float x) {
    float t = fabsf(x);
    float v;
    unsigned idx = 0;
    if (!(t > 0.0f)) return 0u;
    if (t < 2.0f)
        v = 0.5f * rintf(2.0f * t);
    else if (t <= 4.0f)
        v = rintf(t);
    else if (t <= 6.0f)
        v = 2.0f * rintf(0.5f * t);
    else
        v = 6.0f;
    while (E2M1_MAGNITUDE[idx] != v) ++idx; /* v is always one of the eight magnitudes */
    return (idx != 0u && signbit(x)) ? (idx | 8u) : idx;
}

/* [SOAR] FP8 block scale, E4M3 with M_FP8 = 448: sign, four exponent bits (bias 7), three mantissa
 * bits, subnormals m·2^-9, no infinities (0x7F is NaN). Non-negative finite codes 0x00..0x7E are in
 * increasing order of value. */
double nvfp4_ref_e4m3_value(unsigned code) {
    unsigned e = (code >> 3) & 15u, m = code & 7u;
    double v = (e == 0u) ? ldexp((double)m, -9) : ldexp((double)(8u + m), (int)e - 10);
    return (code & 0x80u) ? -v : v;
}

/* The E4M3 values around v >= 0: lo = the largest code whose value is <= v, hi = the smallest whose
 * value is >= v; both are 0x7E (448) for v >= 448. */
void nvfp4_ref_e4m3_bracket(double v, unsigned *lo, unsigned *hi) {
    unsigned c = 0u;
    while (c < 0x7Eu && nvfp4_ref_e4m3_value(c + 1u) <= v) ++c;
    *lo = c;
    *hi = (c == 0x7Eu || nvfp4_ref_e4m3_value(c) == v) ? c : c + 1u;
}

/* R2: nearest E4M3 value, ties to the even code, saturating at 448 (v >= 0). */
unsigned nvfp4_ref_e4m3_rne(double v) {
    unsigned lo, hi;
    double mid;
    nvfp4_ref_e4m3_bracket(v, &lo, &hi);
    if (lo == hi) return lo;
    mid = 0.5 * (nvfp4_ref_e4m3_value(lo) + nvfp4_ref_e4m3_value(hi)); /* exact */
    if (v < mid) return lo;
    if (v > mid) return hi;
    return (lo & 1u) ? hi : lo;
}

/* Element-wise forms of the two codecs, for exhaustive sweeps. */
void nvfp4_ref_e2m1_codes(const float *x, int64_t n, uint8_t *out) {
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = (uint8_t)nvfp4_ref_e2m1_code(x[i]);
}

void nvfp4_ref_e4m3_rne_many(const double *v, int64_t n, uint8_t *out) {
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = (uint8_t)nvfp4_ref_e4m3_rne(v[i]);
}

/* ------------------------------------------------------------------------------------------------ */
/* One block                                                                                         */
/* ------------------------------------------------------------------------------------------------ */

/* [SOAR] Q = Q_fp4(W / (alpha·Delta)), evaluated as R3 states. */
void nvfp4_ref_quantize_block(const float *w16, float alpha, float delta, uint8_t *codes16) {
    float s = alpha * delta;
    float r;
    int j;
    if (s == 0.0f) {
        memset(codes16, 0, 16);
        return;
    }
    r = 1.0f / s;
    for (j = 0; j < 16; ++j) codes16[j] = (uint8_t)nvfp4_ref_e2m1_code(w16[j] * r);
}

/* [SOAR] reconstruction error of one block, ||W_i - Q_i·(alpha·Delta_d)||^2, exactly (R5): Q·alpha·
 * Delta_d has at most 30 significant bits, so each difference is exact in binary64, its square is exact
 * in binary128, and the sixteen squares are summed in binary128. */
static quad block_err(const float *w16, const uint8_t *codes16, float alpha, double delta_d) {
    quad acc = 0;
    int j;
    for (j = 0; j < 16; ++j) {
        double q = (double)nvfp4_ref_e2m1_value(codes16[j]);
        double d = (double)w16[j] - q * (double)alpha * delta_d;
        acc += (quad)d * (quad)d;
    }
    return acc;
}

double nvfp4_ref_block_err(const float *w16, const uint8_t *codes16, float alpha, double delta_d) {
    return (double)block_err(w16, codes16, alpha, delta_d);
}

/* Sum_j W_ij Q_ij and Sum_j Q_ij^2 of one block, exactly. */
static void block_sums(const float *w16, const uint8_t *codes16, quad *swq, quad *sqq) {
    quad a = 0, b = 0;
    int j;
    for (j = 0; j < 16; ++j) {
        quad q = (quad)nvfp4_ref_e2m1_value(codes16[j]);
        a += (quad)w16[j] * q;
        b += q * q;
    }
    *swq = a;
    *sqq = b;
}

/* ------------------------------------------------------------------------------------------------ */
/* Max rule                                                                                          */
/* ------------------------------------------------------------------------------------------------ */

/* [SOAR] alpha = max|X| / (M_FP4·M_FP8) with M_FP4·M_FP8 = 6·448 = 2688, in binary32 (R4). */
static float max_rule_alpha(float amax) { return amax / 2688.0f; }

/* [SOAR] the argument of Q_E4M3 in Delta_i = Q_E4M3(max|X_i| / (alpha·M_FP4)). a and 6·alpha have at
 * most 26 significant bits, so the binary64 quotient lies on an E4M3 midpoint only when the real one
 * does, and its E4M3 rounding is that of the real quotient (R4). */
static double max_rule_quotient(float block_amax, float alpha) {
    if (block_amax == 0.0f) return 0.0;
    return (double)block_amax / (6.0 * (double)alpha);
}

static float block_amax(const float *w16) {
    float a = 0.0f;
    int j;
    for (j = 0; j < 16; ++j)
        if (fabsf(w16[j]) > a) a = fabsf(w16[j]);
    return a;
}

/* ------------------------------------------------------------------------------------------------ */
/* CJSO                                                                                              */
/* ------------------------------------------------------------------------------------------------ */

/* [SOAR] global-scale step. With Q and the block scales fixed, sum_i sum_j (W_ij - alpha·Delta_i·Q_ij)^2
 * is quadratic in alpha; its minimiser is
 *      alpha* = sum_i Delta_i sum_j W_ij Q_ij  /  sum_i Delta_i^2 sum_j Q_ij^2
 * (R6: the page prints alpha in place of Delta_i). Both sums are exact in binary128 and alpha* is
 * rounded once to binary32. */
int nvfp4_ref_alpha_step(const float *w, int64_t nblk, const uint8_t *dcode, const uint8_t *codes16,
                         float *alpha, double *num, double *den) {
    quad n = 0, d = 0;
    int64_t i;
    for (i = 0; i < nblk; ++i) {
        quad swq, sqq;
        quad delta = (quad)nvfp4_ref_e4m3_value(dcode[i]);
        block_sums(w + 16 * i, codes16 + 16 * i, &swq, &sqq);
        n += delta * swq;
        d += delta * delta * sqq;
    }
    if (num) *num = (double)n;
    if (den) *den = (double)d;
    if (d > 0) {
        *alpha = (float)(n / d);
        return 1;
    }
    return 0;
}

/* [SOAR] block-scale step: Delta_i* = sum_j W_ij Q_ij / (alpha · sum_j Q_ij^2) with alpha fixed. The
 * numerator and alpha·sum Q^2 are exact in binary64 and the quotient is taken there. */
int nvfp4_ref_delta_step(const float *w16, const uint8_t *codes16, float alpha, double *dstar) {
    quad swq, sqq;
    block_sums(w16, codes16, &swq, &sqq);
    if (!(sqq > 0)) return 0;
    *dstar = (double)swq / ((double)alpha * (double)sqq);
    return 1;
}

/* [4/6] §02 for one block under alpha a: the max-rule scale Delta6 = E4M3(max|w|/(6a)) and
 * Delta4 = fp8(1.5·Delta6) (the product is exact; fp8 saturates per R2); M=4 is kept iff its block error
 * is strictly smaller (mse = error/16, the same order). Writes the block's codes and scale; returns
 * 1 for M=4. *dstar gets the unrounded value of the chosen scale: max|w|/(6a) for M=6, 1.5·Delta6 for
 * M=4 (R10). */
static int four_over_six_block(const float *wb, float a, uint8_t *c16, uint8_t *dcode, double *dstar) {
    uint8_t c4[16];
    double q6 = max_rule_quotient(block_amax(wb), a);
    unsigned d6 = nvfp4_ref_e4m3_rne(q6);
    unsigned d4 = nvfp4_ref_e4m3_rne(1.5 * nvfp4_ref_e4m3_value(d6));
    quad e6, e4;
    nvfp4_ref_quantize_block(wb, a, (float)nvfp4_ref_e4m3_value(d6), c16);
    nvfp4_ref_quantize_block(wb, a, (float)nvfp4_ref_e4m3_value(d4), c4);
    e6 = block_err(wb, c16, a, nvfp4_ref_e4m3_value(d6));
    e4 = block_err(wb, c4, a, nvfp4_ref_e4m3_value(d4));
    *dcode = (uint8_t)d6;
    *dstar = q6;
    if (e4 < e6) {
        memcpy(c16, c4, 16);
        *dcode = (uint8_t)d4;
        *dstar = 1.5 * nvfp4_ref_e4m3_value(d6);
        return 1;
    }
    return 0;
}

/* [SOAR] CJSO: start from the max rule (or, with init = NVFP4_REF_INIT_4O6, from FourOverSix's choice of
 * block scale under the max-rule alpha), then repeat {global-scale step, re-quantise, block-scale step,
 * re-quantise} (R7). The stored block scale is FP8, so each Delta-step rounds Delta_i* to E4M3 (the
 * page notes that this rounding reaches both quantisation and dequantisation). On return dcode[] holds
 * the E4M3 scales, dstar[] the last unrounded scales and codes16[] one code per element. */
static void cjso(const float *w, int64_t nblk, int iters, int init, float amax, float *alpha, uint8_t *dcode,
                 double *dstar, uint8_t *codes16, float *alpha_trace) {
    int64_t i;
    int t;
    *alpha = max_rule_alpha(amax);
    for (i = 0; i < nblk; ++i) {
        if (init == NVFP4_REF_INIT_4O6) {
            four_over_six_block(w + 16 * i, *alpha, codes16 + 16 * i, &dcode[i], &dstar[i]);
            continue;
        }
        dstar[i] = max_rule_quotient(block_amax(w + 16 * i), *alpha);
        dcode[i] = (uint8_t)nvfp4_ref_e4m3_rne(dstar[i]);
        nvfp4_ref_quantize_block(w + 16 * i, *alpha, (float)nvfp4_ref_e4m3_value(dcode[i]), codes16 + 16 * i);
    }
    if (alpha_trace) alpha_trace[0] = *alpha;
    for (t = 1; t <= iters; ++t) {
        nvfp4_ref_alpha_step(w, nblk, dcode, codes16, alpha, NULL, NULL);
        for (i = 0; i < nblk; ++i)
            nvfp4_ref_quantize_block(w + 16 * i, *alpha, (float)nvfp4_ref_e4m3_value(dcode[i]), codes16 + 16 * i);
        for (i = 0; i < nblk; ++i) {
            double ds;
            if (nvfp4_ref_delta_step(w + 16 * i, codes16 + 16 * i, *alpha, &ds)) {
                dstar[i] = ds;
                dcode[i] = (uint8_t)nvfp4_ref_e4m3_rne(ds);
            } else {
                dstar[i] = nvfp4_ref_e4m3_value(dcode[i]);
            }
        }
        for (i = 0; i < nblk; ++i)
            nvfp4_ref_quantize_block(w + 16 * i, *alpha, (float)nvfp4_ref_e4m3_value(dcode[i]), codes16 + 16 * i);
        if (alpha_trace) alpha_trace[t] = *alpha;
    }
}

/* ------------------------------------------------------------------------------------------------ */
/* Decoupled quantise / dequantise scale search                                                      */
/* ------------------------------------------------------------------------------------------------ */

/* The search's multiplier grid and the rule that gives each candidate its two reconstruct scales.
 * The pages fix one grid (R8) and one rule; the others are the variants R11 describes. */
typedef struct {
    int num0, den, count, dd_rule;
} search_cfg;

static const search_cfg pages_search = {50, 100, 101, NVFP4_REF_DD_CJSO};

/* f_k = the binary32 value nearest (num0+k)/den. The binary64 quotient of the two integers is within
 * half a binary64 ulp of the rational, and for den <= 2^24 that cannot land on a binary32 midpoint
 * unless the rational is one, so converting it to binary32 rounds the rational itself (R8, R11). */
float nvfp4_ref_grid_multiplier(int num0, int den, int k) { return (float)((double)(num0 + k) / (double)den); }

/* [SOAR] Delta_q is perturbed multiplicatively over [0.5, 1.5] in steps of 0.01: f_k for k = 0..100 is
 * the binary32 value nearest to (50+k)/100 (R8). */
float nvfp4_ref_search_multiplier(int k) { return nvfp4_ref_grid_multiplier(50, 100, k); }

static int bad_search(int num0, int den, int count, int dd_rule) {
    return den < 1 || den > (1 << 24) || num0 < 1 || count < 1 || count > 1024 ||
           (int64_t)num0 + count - 1 > 16 * (int64_t)den || dd_rule < NVFP4_REF_DD_CJSO ||
           dd_rule > NVFP4_REF_DD_LSQ;
}

/* [SOAR] for one block: Delta_q (high precision) quantises, Delta_d (E4M3) reconstructs. Start from the
 * CJSO scale (Delta_d = Delta_q = Delta_c); try Delta_q = fl(Delta_c·f_k) against two values of
 * Delta_d and keep the least error. The pages' rule (R8) takes the E4M3 values bracketing the unrounded
 * CJSO scale for every candidate; the R11 rules bracket the candidate's Delta_q, or the least-squares
 * scale of the candidate's own codes (the block-scale step applied to them). */
static void soar_block(const float *w16, float alpha, unsigned dc, double dstar, const search_cfg *cfg,
                       uint8_t *codes16, uint8_t *scale) {
    unsigned dd[2];
    float dcv = (float)nvfp4_ref_e4m3_value(dc);
    uint8_t cand[16];
    quad best;
    int k, m;
    nvfp4_ref_e4m3_bracket(dstar, &dd[0], &dd[1]);
    nvfp4_ref_quantize_block(w16, alpha, dcv, codes16);
    best = block_err(w16, codes16, alpha, (double)dcv);
    *scale = (uint8_t)dc;
    for (k = 0; k < cfg->count; ++k) {
        float dq = dcv * nvfp4_ref_grid_multiplier(cfg->num0, cfg->den, k);
        nvfp4_ref_quantize_block(w16, alpha, dq, cand);
        if (cfg->dd_rule == NVFP4_REF_DD_QUANT) {
            nvfp4_ref_e4m3_bracket((double)dq, &dd[0], &dd[1]);
        } else if (cfg->dd_rule == NVFP4_REF_DD_LSQ) {
            double ls;
            if (nvfp4_ref_delta_step(w16, cand, alpha, &ls))
                nvfp4_ref_e4m3_bracket(ls, &dd[0], &dd[1]);
            else /* every code is zero: every scale reconstructs zero */
                dd[0] = dd[1] = dc;
        }
        for (m = 0; m < 2; ++m) {
            quad e = block_err(w16, cand, alpha, nvfp4_ref_e4m3_value(dd[m]));
            if (e < best) {
                best = e;
                *scale = (uint8_t)dd[m];
                memcpy(codes16, cand, 16);
            }
        }
    }
}

/* ------------------------------------------------------------------------------------------------ */
/* Whole matrix                                                                                      */
/* ------------------------------------------------------------------------------------------------ */

static float *widen(const void *W, int dtype, int64_t n) {
    float *w = (float *)malloc((size_t)n * sizeof(float));
    int64_t i;
    if (!w) return NULL;
    if (dtype == NVFP4_REF_F32) {
        memcpy(w, W, (size_t)n * sizeof(float));
    } else {
        const uint16_t *h = (const uint16_t *)W;
        for (i = 0; i < n; ++i) { /* bf16 is the upper half of a binary32 */
            uint32_t u = (uint32_t)h[i] << 16;
            memcpy(&w[i], &u, 4);
        }
    }
    return w;
}

static void pack_codes(const uint8_t *codes16, int64_t nblk, uint8_t *out) {
    int64_t i;
    for (i = 0; i < nblk * 8; ++i) out[i] = (uint8_t)(codes16[2 * i] | (codes16[2 * i + 1] << 4));
}

static int bad_shape(int64_t rows, int64_t cols, int dtype) {
    return rows <= 0 || cols <= 0 || (cols % 16) != 0 || (dtype != NVFP4_REF_BF16 && dtype != NVFP4_REF_F32);
}

int nvfp4_ref_quantize(const void *W, int dtype, int64_t rows, int64_t cols, int mode, int iters,
                       uint8_t *codes, uint8_t *scales, float *alpha, uint8_t *mchoice, double *dstar,
                       float *alpha_trace) {
    return nvfp4_ref_quantize_ex(W, dtype, rows, cols, mode, iters, NVFP4_REF_INIT_MAX, codes, scales, alpha,
                                 mchoice, dstar, alpha_trace);
}

static int quantize_impl(const void *W, int dtype, int64_t rows, int64_t cols, int mode, int iters, int init,
                         const search_cfg *cfg, uint8_t *codes, uint8_t *scales, float *alpha, uint8_t *mchoice,
                         double *dstar, float *alpha_trace);

int nvfp4_ref_quantize_ex(const void *W, int dtype, int64_t rows, int64_t cols, int mode, int iters, int init,
                          uint8_t *codes, uint8_t *scales, float *alpha, uint8_t *mchoice, double *dstar,
                          float *alpha_trace) {
    return quantize_impl(W, dtype, rows, cols, mode, iters, init, &pages_search, codes, scales, alpha, mchoice,
                         dstar, alpha_trace);
}

int nvfp4_ref_quantize_search(const void *W, int dtype, int64_t rows, int64_t cols, int iters, int init,
                              int num0, int den, int count, int dd_rule, uint8_t *codes, uint8_t *scales,
                              float *alpha, double *dstar) {
    search_cfg cfg;
    if (bad_search(num0, den, count, dd_rule)) return -1;
    cfg.num0 = num0;
    cfg.den = den;
    cfg.count = count;
    cfg.dd_rule = dd_rule;
    return quantize_impl(W, dtype, rows, cols, NVFP4_REF_SOAR, iters, init, &cfg, codes, scales, alpha, NULL,
                         dstar, NULL);
}

static int quantize_impl(const void *W, int dtype, int64_t rows, int64_t cols, int mode, int iters, int init,
                         const search_cfg *cfg, uint8_t *codes, uint8_t *scales, float *alpha, uint8_t *mchoice,
                         double *dstar, float *alpha_trace) {
    int64_t n, nblk, i;
    float *w, amax = 0.0f;
    uint8_t *c16, *dcode;
    double *ds;
    int nonfinite = 0;

    if (!W || !codes || !scales || !alpha || bad_shape(rows, cols, dtype) || mode < 0 || mode > 3 || iters < 0)
        return -1;
    if (init != NVFP4_REF_INIT_MAX && (init != NVFP4_REF_INIT_4O6 || mode < NVFP4_REF_CJSO)) return -1;
    n = rows * cols;
    nblk = n / 16;
    w = widen(W, dtype, n);
    c16 = (uint8_t *)calloc((size_t)n, 1);
    dcode = (uint8_t *)calloc((size_t)nblk, 1);
    ds = (double *)calloc((size_t)nblk, sizeof(double));
    if (!w || !c16 || !dcode || !ds) {
        free(w); free(c16); free(dcode); free(ds);
        return -2;
    }
    for (i = 0; i < n; ++i) {
        if (!isfinite(w[i])) nonfinite = 1;
        else if (fabsf(w[i]) > amax) amax = fabsf(w[i]);
    }
    if (mchoice) memset(mchoice, 0, (size_t)nblk);

    if (nonfinite) { /* R9 */
        memset(codes, 0, (size_t)nblk * 8);
        memset(scales, 0, (size_t)nblk);
        *alpha = NAN;
        if (dstar) memset(dstar, 0, (size_t)nblk * sizeof(double));
        if (alpha_trace) for (i = 0; i <= iters; ++i) alpha_trace[i] = NAN;
        free(w); free(c16); free(dcode); free(ds);
        return 1;
    }

    if (mode == NVFP4_REF_MAX || mode == NVFP4_REF_FOUR_OVER_SIX) {
        float a = max_rule_alpha(amax);
        *alpha = a;
        for (i = 0; i < nblk; ++i) {
            const float *wb = w + 16 * i;
            if (mode == NVFP4_REF_FOUR_OVER_SIX) {
                double unused;
                int m4 = four_over_six_block(wb, a, c16 + 16 * i, &dcode[i], &unused);
                if (mchoice) mchoice[i] = (uint8_t)m4;
                continue;
            }
            unsigned d6 = nvfp4_ref_e4m3_rne(max_rule_quotient(block_amax(wb), a));
            nvfp4_ref_quantize_block(wb, a, (float)nvfp4_ref_e4m3_value(d6), c16 + 16 * i);
            dcode[i] = (uint8_t)d6;
        }
        if (alpha_trace) alpha_trace[0] = a;
    } else {
        cjso(w, nblk, iters, init, amax, alpha, dcode, ds, c16, alpha_trace);
        if (mode == NVFP4_REF_SOAR)
            for (i = 0; i < nblk; ++i)
                soar_block(w + 16 * i, *alpha, dcode[i], ds[i], cfg, c16 + 16 * i, &dcode[i]);
        if (dstar) memcpy(dstar, ds, (size_t)nblk * sizeof(double));
    }
    pack_codes(c16, nblk, codes);
    memcpy(scales, dcode, (size_t)nblk);
    free(w); free(c16); free(dcode); free(ds);
    return 0;
}

int nvfp4_ref_soar_blocks(const void *W, int dtype, int64_t rows, int64_t cols, float alpha,
                          const uint8_t *dcode, const double *dstar, const int64_t *blocks, int64_t nsel,
                          uint8_t *codes_sel, uint8_t *scales_sel) {
    return nvfp4_ref_soar_blocks_search(W, dtype, rows, cols, alpha, dcode, dstar, blocks, nsel, pages_search.num0,
                                        pages_search.den, pages_search.count, pages_search.dd_rule, codes_sel,
                                        scales_sel);
}

int nvfp4_ref_soar_blocks_search(const void *W, int dtype, int64_t rows, int64_t cols, float alpha,
                                 const uint8_t *dcode, const double *dstar, const int64_t *blocks, int64_t nsel,
                                 int num0, int den, int count, int dd_rule, uint8_t *codes_sel,
                                 uint8_t *scales_sel) {
    int64_t nblk, s;
    search_cfg cfg;
    if (!W || !dcode || !dstar || !blocks || !codes_sel || !scales_sel || bad_shape(rows, cols, dtype) ||
        nsel < 0 || bad_search(num0, den, count, dd_rule))
        return -1;
    cfg.num0 = num0;
    cfg.den = den;
    cfg.count = count;
    cfg.dd_rule = dd_rule;
    nblk = rows * cols / 16;
    for (s = 0; s < nsel; ++s) {
        int64_t b = blocks[s];
        float w16[16];
        uint8_t c16[16];
        int j;
        if (b < 0 || b >= nblk) return -1;
        if (dtype == NVFP4_REF_F32) {
            memcpy(w16, (const float *)W + 16 * b, sizeof(w16));
        } else {
            const uint16_t *h = (const uint16_t *)W + 16 * b;
            for (j = 0; j < 16; ++j) {
                uint32_t u = (uint32_t)h[j] << 16;
                memcpy(&w16[j], &u, 4);
            }
        }
        soar_block(w16, alpha, dcode[b], dstar[b], &cfg, c16, &scales_sel[s]);
        pack_codes(c16, 1, codes_sel + 8 * s);
    }
    return 0;
}

void nvfp4_ref_dequantize(const uint8_t *codes, const uint8_t *scales, float alpha, int64_t rows,
                          int64_t cols, double *out) {
    int64_t n = rows * cols, i;
    for (i = 0; i < n; ++i) {
        unsigned c = (codes[i / 2] >> (4 * (i & 1))) & 15u;
        out[i] = (double)nvfp4_ref_e2m1_value(c) * nvfp4_ref_e4m3_value(scales[i / 16]) * (double)alpha;
    }
}

/* Y[m][n] = sum_k X[m][k] * What[n][k] with What = e2m1(code) * e4m3(scale) * alpha, the reconstruction
 * the SOAR page defines (dequantisation equation), applied to a weight matrix [N][K] stored as the
 * quantiser writes it: the product a W4A16 matrix multiply computes. Each product is exact in
 * binary128 (X has at most 24 significant bits, the weight 2 + 4 + 24) and the sum over k is taken in
 * binary128 in k order; Y is that sum rounded to binary64. X is [M][K] bf16 or fp32. */
int nvfp4_ref_matmul(const void *X, int x_dtype, int64_t M, int64_t K, const uint8_t *codes,
                     const uint8_t *scales, float alpha, int64_t N, double *Y) {
    int64_t m, n, k;
    float *x;
    if (!X || !codes || !scales || !Y || bad_shape(M, K, x_dtype) || N <= 0) return -1;
    x = widen(X, x_dtype, M * K);
    if (!x) return -2;
    for (m = 0; m < M; ++m)
        for (n = 0; n < N; ++n) {
            quad acc = 0;
            for (k = 0; k < K; ++k) {
                int64_t i = n * K + k;
                unsigned c = (codes[i / 2] >> (4 * (i & 1))) & 15u;
                quad wv = (quad)nvfp4_ref_e2m1_value(c) * (quad)nvfp4_ref_e4m3_value(scales[i / 16]) * (quad)alpha;
                acc += (quad)x[m * K + k] * wv;
            }
            Y[m * N + n] = (double)acc;
        }
    free(x);
    return 0;
}

double nvfp4_ref_mse(const void *W, int dtype, int64_t rows, int64_t cols, const uint8_t *codes,
                     const uint8_t *scales, float alpha) {
    int64_t n = rows * cols, nblk = n / 16, i;
    quad acc = 0;
    float *w = widen(W, dtype, n);
    uint8_t c16[16];
    if (!w) return NAN;
    for (i = 0; i < nblk; ++i) {
        int j;
        for (j = 0; j < 8; ++j) {
            c16[2 * j] = codes[8 * i + j] & 15u;
            c16[2 * j + 1] = codes[8 * i + j] >> 4;
        }
        acc += block_err(w + 16 * i, c16, alpha, nvfp4_ref_e4m3_value(scales[i]));
    }
    free(w);
    return (double)(acc / (quad)n);
}
