// noalloc.hip -- the device array behind kv_decode_step_noalloc (api.cpp):
// the decode step's workspace (the attention kernels' split partials and
// schedule prefix sums) for callers that cannot allocate (code under graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The array is a static __device__ object: every device the library runs on
// holds its own copy, at its own address, until the process ends. In host code
// its name is only a host-side stand-in, so its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and only
// that address is ever handed to the kernels. Nothing here allocates.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace kvc {

namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) static unsigned char scratch[kNoallocScratchBytes];

std::mutex g_lock;
void *g_ptr[kMaxDevices];  // device address of `scratch` per device (null until looked up)

}  // namespace

void *noalloc_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_lock);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace kvc
