// noalloc.hip -- kda_prefill_noalloc: kda_prefill for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). Its workspace is a fixed-size array in the
// library's own device memory instead of a caller buffer.
#include "../../include/kda.h"

#include <atomic>

#include "kda_launch.h"

namespace kda {
namespace {

// The prefill workspace of every call of kda_prefill_noalloc on one GPU. Each
// GPU that loads the library holds its own copy until the process ends.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

}  // namespace

// Device address of `scratch` on the current device, looked up once per
// device with that device current. In host code the name `scratch` is only a
// host-side stand-in, never a device address, so kernels and copies must be
// given this pointer. Concurrent first calls may both look it up; they store
// the same value.
hipError_t noalloc_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace kda
