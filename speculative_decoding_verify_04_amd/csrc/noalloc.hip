// Fixed device scratch of the allocation-free attention entry point
// (spec_verify_attn_noalloc).
//
// Callers that cannot allocate device memory -- code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc -- get the attention's
// arrival counters and split-K partial results from one file-scope device
// array of kScratchBytes per GPU, held by the library until the process ends.
// Its first kCounterBytes are the counter region (zero between calls: every
// completed call leaves its counters at zero), the rest the data region.
//
// In host code the array's name is only a host-side stand-in; its address on
// a device comes from hipGetSymbolAddress with that device current, looked up
// once per device and kept.  Every call on a GPU shares that GPU's array:
// calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sv_internal.h"

namespace sv {
namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per GPU
constexpr size_t kCounterBytes = size_t(256) << 10;  // 65536 arrival counters
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device (null: not set up)

__global__ void clear_words(unsigned int* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

}  // namespace

void noalloc_limits(size_t* counter_bytes, size_t* data_bytes) {
    *counter_bytes = kCounterBytes;
    *data_bytes = kScratchBytes - kCounterBytes;
}

hipError_t noalloc_scratch(hipStream_t stream, void** counters, size_t* counter_bytes,
                           void** data, size_t* data_bytes) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        // the counters start at zero (a kernel, not a memset node, so that a
        // caller may capture this first call into a graph)
        const int words = static_cast<int>(kCounterBytes / 4);
        hipLaunchKernelGGL(clear_words, dim3((words + 255) / 256), dim3(256), 0, stream,
                           static_cast<unsigned int*>(ptr), words);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_scratch[dev] = ptr;
    }
    char* base = static_cast<char*>(g_scratch[dev]);
    *counters = base;
    *counter_bytes = kCounterBytes;
    *data = base + kCounterBytes;
    *data_bytes = kScratchBytes - kCounterBytes;
    return hipSuccess;
}

}  // namespace sv
