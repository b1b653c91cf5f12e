// nvfp4_quantize_noalloc: the quantiser without any allocation, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid it).
//
// Its scratch (the per-work-group partial results of the global max and of the CJSO sums, the alpha of
// each round, and for SOAR the two-byte E4M3 bracket of every block) lives in `scratch`, a file-scope
// device array of kNoallocScratchBytes that every GPU the library runs on holds until the process ends.
// Host code never passes the array's name to a kernel (on the host it is only a stand-in for the
// symbol): on the first call on a device, with that device current, hipGetSymbolAddress gives this
// device's address of its copy, which is kept per device and used from then on.
//
// Every call on a GPU shares that GPU's array and leaves its contents behind. Nothing in it needs to
// start at zero: each kernel writes its partials before the next kernel reads them. Two calls that
// overlap on one GPU (different streams, or threads without ordering) race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

#define NVFP4_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kNoallocScratchBytes = NVFP4_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::mutex g_lock;
void *g_scratch[kMaxDevices] = {};

// This device's address of `scratch` (the current device), looked up once per device.
hipError_t device_scratch(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

NVFP4_API size_t nvfp4_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

NVFP4_API int nvfp4_quantize_noalloc(const nvfp4_args_t *a) {
    const int c = nvfp4::check_args(a);
    if (c != NVFP4_OK) return c;
    if (a->workspace || a->workspace_bytes) return NVFP4_ERR_INVALID_ARG;
    if (nvfp4::workspace_bytes(a->rows * a->cols / 16, a->mode) > kNoallocScratchBytes) return NVFP4_ERR_TOO_LARGE;
    void *ws = nullptr;
    if (device_scratch(&ws) != hipSuccess) return NVFP4_ERR_HIP;
    return nvfp4::run_quantize(a, ws);
}
