// Physics probes for the benchmark's context figures; not part of the
// library.
//
//  * probe_empty launches a kernel that does nothing with a given grid and
//    workgroup size.  Launched back to back, it gives the queue's per-launch
//    floor for that launch shape: what any single call of that shape costs
//    before it touches memory.
//  * probe_chase has one lane follow a chain of indices, each load waiting
//    for the one before.  The time per link is the load-to-use latency of
//    the level of the memory hierarchy that holds the chain: a chain of
//    random links over a few MiB stays in the L2 cache, one over several
//    GiB goes to HBM.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ void empty_kernel() {}

__global__ __launch_bounds__(64) void chase_kernel(const uint32_t *__restrict__ next, uint32_t start,
                                                   int links, uint32_t *__restrict__ out) {
    if (threadIdx.x != 0) return;
    uint32_t i = start;
    for (int s = 0; s < links; ++s) {
        // keep the index in a vector register, so each link is a vector
        // memory load through the L2 cache
        asm volatile("" : "+v"(i));
        i = next[i];
    }
    out[0] = i;
}

}  // namespace

extern "C" {

// Launches the empty kernel on `stream`: `grid` workgroups of `block` lanes
// (1..1024).  Returns the launch's hipError_t, or hipErrorInvalidValue
// (without launching) for sizes out of range.
int probe_empty(int grid, int block, hipStream_t stream) {
    if (grid < 1 || block < 1 || block > 1024) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(block), 0, stream);
    return (int)hipGetLastError();
}

// Follows `links` links of the chain in `next` from index `start` and writes
// the last index to out[0].  `next` is a device array of `n` indices, each
// below `n`; the caller builds it.  Returns the launch's hipError_t, or
// hipErrorInvalidValue (without launching) when start >= n or links < 0.
int probe_chase(const uint32_t *next, uint64_t n, uint32_t start, int links, uint32_t *out,
                hipStream_t stream) {
    if (start >= n || links < 0 || n > 0xffffffffull) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(chase_kernel, dim3(1), dim3(64), 0, stream, next, start, links, out);
    return (int)hipGetLastError();
}

}  // extern "C"
