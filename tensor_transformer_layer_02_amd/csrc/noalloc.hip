// Static device scratch of the no-allocation FFN backward (tp_mlp_shard_bwd_noalloc).
//
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid it), the backward's scratch (dU and
// the column-sum partials) lives in a file-scope device array of fixed size
// instead of a caller-provided work buffer.  Each device that loads the library's
// code holds its own copy of the array until the process ends.  In host code the
// array's name is only a host-side handle: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is handed to
// kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tp_kernels.h"

namespace tp {

namespace {

static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int SCRATCH_DEVICES = 64;
void* g_scratch[SCRATCH_DEVICES] = {};  // device address of `scratch` on each device
std::mutex g_scratch_mu;

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= SCRATCH_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch[dev]) {  // first use on this device (it is the current one)
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace tp
