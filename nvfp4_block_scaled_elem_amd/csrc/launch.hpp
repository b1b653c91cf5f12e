// Internal launchers of the gfx950 kernels (host side). Every launcher enqueues on `stream` and
// returns the hipError_t of the launch. Shapes are validated by the C ABI before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/nvfp4.h"

namespace nvfp4 {

// Shapes of the streaming passes. Each pass writes one partial result per work-group that every
// work-group of the next kernel reduces, so they use a fixed grid (at most G work-groups of T threads,
// each thread walking at least kMinBlocksPerThread blocks) and keep D blocks per thread in flight in a
// register ring. The MAX/FourOverSix pass (k_quant) and the CJSO passes (k_cjso_init, k_cjso_iter) are
// tuned separately: the defaults are the fastest of the settings timed on an MI355X for a 4096 x 4096
// matrix, and the macros exist so that other settings can be built and timed. For the CJSO passes that
// weighs a call alone against calls on three streams at once: 1024 x 256 is 6 % faster alone but, at
// 16 waves per CU with up to 105 VGPRs each, leaves no room for another stream's work-groups and loses
// 18 % over three streams; 512 x 256 is 3 % faster alone than 256 x 512 and as fast over three streams.
#ifndef NVFP4_QUANT_THREADS
#define NVFP4_QUANT_THREADS 512
#endif
#ifndef NVFP4_QUANT_GROUPS
#define NVFP4_QUANT_GROUPS 512
#endif
#ifndef NVFP4_QUANT_DEPTH
#define NVFP4_QUANT_DEPTH 2
#endif
#ifndef NVFP4_CJSO_THREADS
#define NVFP4_CJSO_THREADS 512
#endif
#ifndef NVFP4_CJSO_GROUPS
#define NVFP4_CJSO_GROUPS 256
#endif
#ifndef NVFP4_CJSO_DEPTH
#define NVFP4_CJSO_DEPTH 1
#endif
#ifndef NVFP4_CJSO_WAVES
#define NVFP4_CJSO_WAVES 4
#endif
// How a work-group's waves combine their double-double sums (see wg_sum_dd2): 0 through wave 0,
// 1 per-wave first, 2 a tree across waves.
#ifndef NVFP4_WG_SUM
#define NVFP4_WG_SUM 2
#endif
// Size of the fixed device array behind nvfp4_quantize_noalloc (16 MiB).
#ifndef NVFP4_NOALLOC_SCRATCH_BYTES
#define NVFP4_NOALLOC_SCRATCH_BYTES (16u << 20)
#endif
constexpr int kQuantThreads = NVFP4_QUANT_THREADS;
constexpr int kQuantGroups = NVFP4_QUANT_GROUPS;
constexpr int kQuantDepth = NVFP4_QUANT_DEPTH;
constexpr int kCjsoThreads = NVFP4_CJSO_THREADS;
constexpr int kCjsoGroups = NVFP4_CJSO_GROUPS;
constexpr int kCjsoDepth = NVFP4_CJSO_DEPTH;
// the max pass runs on the grid of its consumer (k_quant or k_cjso_init)
constexpr int kAmaxMaxGroups = kQuantGroups > kCjsoGroups ? kQuantGroups : kCjsoGroups;
constexpr int kMinBlocksPerThread = 2;

int quant_groups(int64_t nblk);
int cjso_groups(int64_t nblk);

// Scratch layout inside the workspace (byte offsets, 256-byte aligned pieces).
struct Workspace {
    uint32_t *amax_part;  // [kAmaxMaxGroups]   max |w| bits per work-group of the max pass
    float *alpha_state;   // [2]                alpha of the previous / current CJSO round
    double *cjso_part;    // [2][kCjsoGroups][4] (N.hi, N.lo, D.hi, D.lo) per work-group
    uint16_t *brackets;   // [nblk]             E4M3 codes lo | hi << 8 around the unrounded CJSO scale (SOAR)
    uint32_t *m4_part;    // [kQuantGroups] FourOverSix M=4 counts per work-group (same offset)
};
size_t workspace_bytes(int64_t nblk, int mode);

// The quantiser's host side (api.cpp): argument checks (NVFP4_OK or an nvfp4_error) and the kernel
// sequence of a mode, enqueued on a->stream with `ws` as scratch (workspace_bytes of it).
int kernel_count(int mode, int iters);
int check_args(const nvfp4_args_t *a);
int run_quantize(const nvfp4_args_t *a, void *ws);
Workspace carve(void *base, int64_t nblk);

// The global max pass, on the grid of the pass that consumes it (k_cjso_init when for_cjso, else k_quant);
// `groups` gets the number of per-work-group partials written.
hipError_t launch_amax(const void *W, bool f32, int64_t nblk, bool for_cjso, uint32_t *amax_part, int &groups,
                       nvfp4_stats_t *stats, hipStream_t stream);
hipError_t launch_quant(const void *W, bool f32, bool four_over_six, int64_t nblk, const uint32_t *amax_part,
                        int amax_n, uint8_t *codes, uint8_t *scales, float *alpha_out, uint8_t *mchoice,
                        nvfp4_stats_t *stats, uint32_t *m4_part, hipStream_t stream);
hipError_t launch_cjso_init(const void *W, bool f32, bool soar, bool fos, int64_t nblk, const uint32_t *amax_part,
                            int amax_n, int iters, uint8_t *codes, uint8_t *scales, float *alpha_out,
                            const Workspace &ws, int groups, nvfp4_stats_t *stats, hipStream_t stream);
hipError_t launch_cjso_iter(const void *W, bool f32, bool soar, int64_t nblk, int t, int iters, uint8_t *codes,
                            uint8_t *scales, float *alpha_out, const Workspace &ws, int groups, hipStream_t stream);
hipError_t launch_soar(const void *W, bool f32, int64_t nblk, const float *alpha, uint8_t *codes, uint8_t *scales,
                       const uint16_t *brackets, bool full_search, int num0, int den, int count, int rule,
                       hipStream_t stream);
hipError_t launch_encode_e2m1(const float *x, int64_t n, uint8_t *codes, hipStream_t stream);
hipError_t launch_reciprocal(const float *s, int64_t n, float *r, hipStream_t stream);
// The W4A16 product's launch for given shapes: which kernel, its tile shape, the K split and the grid.
enum { kW4a16Gemv = 0, kW4a16Skinny = 1, kW4a16Gemm = 2 };
struct W4a16Plan {
    int kind;             // kW4a16*
    int tm, tn;           // output tile (gemm); tm = rows of X compiled for (skinny)
    int64_t tiles_n, tiles, slices, kslice, grid, reduce_grid;
    int64_t chunks;       // gemv: 2048-k chunks compiled for
    size_t lds;           // gemv: dynamic LDS bytes
    size_t part_bytes;    // fp32 partial sums of the K slices (0 without a split)
};
W4a16Plan plan_w4a16(int64_t M, int64_t K, int64_t N);
// `part` holds plan.part_bytes (256-byte aligned) when the plan splits K; otherwise it is unused.
hipError_t launch_w4a16(const uint16_t *X, int64_t M, int64_t K, const uint8_t *codes, const uint8_t *scales,
                        const float *alpha, int64_t N, void *Y, bool out_f32, float *part, hipStream_t stream);
size_t stats_workspace_bytes();
hipError_t launch_stats(const void *W, bool f32, int64_t nblk, const uint8_t *codes, const uint8_t *scales,
                        const float *alpha, double *sse_out, unsigned long long *hist_out, void *workspace,
                        hipStream_t stream);
size_t gptq_workspace_bytes(int64_t rows, int64_t cols);
hipError_t launch_gptq(const void *W, bool f32, int64_t rows, int64_t cols, const double *H, double percdamp,
                       uint8_t *codes, uint8_t *scales, float *alpha, void *workspace, hipStream_t stream);
hipError_t launch_dequant(const uint8_t *codes, const uint8_t *scales, const float *alpha, int64_t nblk, void *out,
                          bool out_f32, hipStream_t stream);

}  // namespace nvfp4
