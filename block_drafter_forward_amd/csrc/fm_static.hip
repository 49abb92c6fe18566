// fm_static.hip — the library's static device scratch, for the entry point that allocates nothing.
//
// Callers that cannot allocate device memory at the call site (code under HIP graph capture, tight serving loops)
// call fm_lm_argmax_static, which takes its scratch -- the 16 argmax keys and the activation fragments of up to 16
// rows of width <= 8192 -- from this file-scope array instead of the handle's workspace. Each GPU the library runs
// on holds its own copy until the process ends. In host code `scratch` names a host-side stand-in, not device
// memory, so its device address is looked up once per device with hipGetSymbolAddress (with that device current)
// and only that address is ever handed to kernels or copies.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fm_kernels.h"

static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES];   // scratch's device address on each device, once looked up
}  // namespace

void* static_scratch(hipError_t* err) {
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= MAX_DEVICES) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_ptr[dev] = p;
    }
    *err = hipSuccess;
    return g_ptr[dev];
}
