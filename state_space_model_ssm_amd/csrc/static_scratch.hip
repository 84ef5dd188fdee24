// A fixed device array that stands in for the prefill workspace in
// mamba2_prefill_fwd_noalloc, for callers that cannot allocate. One copy per GPU,
// from the time the library's code is loaded on that GPU until the process ends.
//
// Host code never uses the array's name as a device address (on the host it is only
// a stand-in symbol): static_scratch() looks the array's address up once per device
// with hipGetSymbolAddress, with that device current, and every later use goes
// through that address.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/mamba2.h"
#include "kernels.hpp"

namespace m2 {

static __device__ __align__(256) unsigned char scratch[MAMBA2_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t static_scratch(void **ptr, size_t *bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    *bytes = MAMBA2_STATIC_SCRATCH_BYTES;
    return hipSuccess;
}

}  // namespace m2
