// static_scratch.hip -- device memory the library owns, for the entry point
// that must not allocate (conv2d_fwd_bf16_noalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, from the first use until the process ends.  In host code the
// name is only a shadow symbol, not a device address, so host code never
// passes it anywhere; it asks the runtime for the address on the current
// device once (hipGetSymbolAddress) and from then on hands out that pointer.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "conv_internal.h"

static __device__ __align__(256) unsigned char scratch[convfwd::kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_init_mu;                               // serialises the first lookup per device
std::atomic<void *> g_scratch_ptr[kMaxDevices];    // device address of `scratch`, per device

}  // namespace

namespace convfwd {

hipError_t static_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_init_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            // `dev` is current here, so this is that device's copy.
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace convfwd
