// noalloc.hip -- the fixed scratch buffer of the allocation-free entry point
// (gemv_q2_batched_noalloc in api.hip).
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) cannot bring the
// workspace that gemv_q2_batched_ws takes.  For them the partial sums of
// sliced rows go to one file-scope device array instead, SCRATCH_BYTES per
// GPU, which every GPU the library runs on holds until the process ends.
//
// In host code the array's name is only a host-side handle: its device
// address comes from hipGetSymbolAddress, asked once per device with that
// device current (each GPU holds its own copy at its own address), and only
// that address is ever passed to a kernel.  Every call on a GPU shares that
// GPU's array, so calls that overlap on one GPU (other streams, other
// threads) race.  The partial sums need no clearing: each launch writes every
// value it reads.
#include <hip/hip_runtime.h>

#include <atomic>

#include "kernels.hpp"

namespace gg {
namespace {

static __device__ __align__(256) float scratch[SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<float *> g_scratch[kMaxDevices];   // device address per device, once known

}  // namespace

float *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    float *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p != nullptr) return p;
    // first use on this device (the current one): its copy of the array
    void *addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
        return nullptr;
    p = static_cast<float *>(addr);
    g_scratch[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace gg
