/*
 * Drives every entry point of the C oracle once or more on small inputs, for a build of the oracle with
 * AddressSanitizer and UndefinedBehaviorSanitizer (host code only). Test infrastructure: it is compiled
 * and run by tests/test_oracle_sanitize.py and exits non-zero on any failed call; the sanitizers abort on
 * any memory or undefined-behaviour error they find.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "nvfp4_oracle.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;

static double uniform(void) { /* xorshift64*, top 53 bits */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (double)((state * 0x2545F4914F6CDD1Dull) >> 11) * 0x1p-53;
}

static float draw(void) {
    double u = uniform(), v = uniform();
    double z = sqrt(-2.0 * log(u > 0 ? u : 1e-300)) * cos(6.283185307179586 * v);
    if (uniform() < 0.002) z *= 20.0; /* a few outliers */
    return (float)(0.02 * z);
}

static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            return 1;                                                      \
        }                                                                  \
    } while (0)

static int run_matrix(const void *W, int dtype, int64_t rows, int64_t cols) {
    int64_t nblk = rows * cols / 16, i;
    uint8_t *codes = malloc((size_t)nblk * 8), *scales = malloc((size_t)nblk), *mch = malloc((size_t)nblk);
    double *dstar = malloc((size_t)nblk * sizeof(double));
    float trace[4], alpha;
    int mode, init, rule;
    CHECK(codes && scales && mch && dstar);
    for (mode = 0; mode < 4; ++mode)
        for (init = 0; init < 2; ++init) {
            int st;
            if (init == 1 && mode < 2) continue;
            st = nvfp4_ref_quantize_ex(W, dtype, rows, cols, mode, 3, init, codes, scales, &alpha, mch, dstar, trace);
            CHECK(st == 0 || st == 1);
            (void)nvfp4_ref_mse(W, dtype, rows, cols, codes, scales, alpha);
        }
    for (rule = 0; rule < 3; ++rule)
        CHECK(nvfp4_ref_quantize_search(W, dtype, rows, cols, 2, 0, 97, 200, 7, rule, codes, scales, &alpha, dstar) >= 0);
    {
        int64_t blocks[3] = {0, nblk / 2, nblk - 1};
        uint8_t cs[24], ss[3];
        CHECK(nvfp4_ref_quantize(W, dtype, rows, cols, 2, 2, codes, scales, &alpha, NULL, dstar, NULL) >= 0);
        CHECK(nvfp4_ref_soar_blocks(W, dtype, rows, cols, alpha, scales, dstar, blocks, 3, cs, ss) == 0);
        for (rule = 0; rule < 3; ++rule)
            CHECK(nvfp4_ref_soar_blocks_search(W, dtype, rows, cols, alpha, scales, dstar, blocks, 3, 50, 100, 101, rule,
                                               cs, ss) == 0);
    }
    {
        double *deq = malloc((size_t)(rows * cols) * sizeof(double));
        double *Y = malloc((size_t)(3 * rows) * sizeof(double));
        float *X = malloc((size_t)(3 * cols) * sizeof(float));
        CHECK(deq && Y && X);
        for (i = 0; i < 3 * cols; ++i) X[i] = draw();
        nvfp4_ref_dequantize(codes, scales, alpha, rows, cols, deq);
        CHECK(nvfp4_ref_matmul(X, NVFP4_REF_F32, 3, cols, codes, scales, alpha, rows, Y) == 0);
        free(deq);
        free(Y);
        free(X);
    }
    free(codes);
    free(scales);
    free(mch);
    free(dstar);
    return 0;
}

int main(void) {
    const int64_t rows = 8, cols = 96, n = rows * cols;
    float *wf = malloc((size_t)n * sizeof(float));
    uint16_t *wb = malloc((size_t)n * sizeof(uint16_t));
    int64_t i;
    unsigned c, lo, hi;
    CHECK(wf && wb);
    for (i = 0; i < n; ++i) {
        wf[i] = draw();
        wb[i] = to_bf16(wf[i]);
    }
    for (i = 16; i < 32; ++i) wf[i] = 0.0f;        /* a zero block */
    for (i = 32; i < 48; ++i) wf[i] *= 1e-30f;     /* a block whose scale underflows */
    CHECK(run_matrix(wf, NVFP4_REF_F32, rows, cols) == 0);
    CHECK(run_matrix(wb, NVFP4_REF_BF16, rows, cols) == 0);
    wf[5] = NAN;
    CHECK(run_matrix(wf, NVFP4_REF_F32, rows, cols) == 0);
    wf[5] = -INFINITY;
    CHECK(run_matrix(wf, NVFP4_REF_F32, rows, cols) == 0);
    memset(wf, 0, (size_t)n * sizeof(float));
    CHECK(run_matrix(wf, NVFP4_REF_F32, rows, cols) == 0);
    /* step functions and codecs */
    {
        uint8_t dcode[2] = {60, 70}, c16[32];
        float a = 1e-4f, w32[32];
        double num, den, ds;
        for (i = 0; i < 32; ++i) w32[i] = draw();
        nvfp4_ref_quantize_block(w32, a, 30.0f, c16);
        nvfp4_ref_quantize_block(w32 + 16, a, 40.0f, c16 + 16);
        CHECK(nvfp4_ref_alpha_step(w32, 2, dcode, c16, &a, &num, &den) >= 0);
        CHECK(nvfp4_ref_delta_step(w32, c16, a, &ds) >= 0);
        (void)nvfp4_ref_block_err(w32, c16, a, 30.0);
    }
    for (c = 0; c < 16; ++c) (void)nvfp4_ref_e2m1_value(c);
    for (c = 0; c < 256; ++c) (void)nvfp4_ref_e4m3_value(c);
    {
        const double probes[] = {-1.0, 0.0, 1e-300, 0x1p-10, 0.3, 1.0625, 447.9, 448.0, 1e300, INFINITY};
        for (i = 0; i < (int64_t)(sizeof(probes) / sizeof(probes[0])); ++i) {
            nvfp4_ref_e4m3_bracket(probes[i], &lo, &hi);
            (void)nvfp4_ref_e4m3_rne(probes[i]);
        }
    }
    {
        const float probes[] = {NAN, -INFINITY, -6.5f, -0.25f, -0.0f, 0.0f, 0.25f, 2.5f, 5.0f, 1e30f};
        uint8_t out[10];
        nvfp4_ref_e2m1_codes(probes, 10, out);
    }
    (void)nvfp4_ref_search_multiplier(100);
    (void)nvfp4_ref_grid_multiplier(1, 1 << 24, 1023);
    /* rejected arguments */
    CHECK(nvfp4_ref_quantize(wf, NVFP4_REF_F32, rows, 24, 0, 0, (uint8_t *)wb, (uint8_t *)wb, wf, NULL, NULL, NULL) == -1);
    free(wf);
    free(wb);
    puts("oracle sanitizer run: ok");
    return 0;
}
