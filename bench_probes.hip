// Physics probes for the benchmark's context figures; not part of the
// library.
//
//  * probe_empty launches a kernel that does nothing with a given grid and
//    workgroup size.  Launched back to back, it gives the queue's per-launch
//    floor for that launch shape: what any single call of that shape costs
//    before it touches memory.
//  * probe_mfma runs fp32 MFMAs back to back on every SIMD with 1, 2 or 4
//    independent accumulators per wave: the rate the matrix cores reach
//    with no memory traffic, for 32 x 32 x 2 and 16 x 16 x 4 blocks.
//  * probe_chase has one lane follow a chain of indices, each load waiting
//    for the one before.  The time per link is the load-to-use latency of
//    the level of the memory hierarchy that holds the chain: a chain of
//    random links over a few MiB stays in the L2 cache, one over several
//    GiB goes to HBM.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// NACC independent accumulators, each taking `iters` fp32 MFMAs in turn
// (32 x 32 x 2 when BIG, else 16 x 16 x 4); each lane's sum of its
// accumulators goes to out[global lane], so that nothing is dead code.
template <bool BIG, int NACC>
__global__ __launch_bounds__(1024) void mfma_kernel(float a, float b, int iters,
                                                    float *__restrict__ out) {
    using V = typename std::conditional<BIG, v16f, v4f>::type;
    constexpr int R = BIG ? 16 : 4;
    V acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[j][r] = 0.f;
    const float av = a + (float)threadIdx.x, bv = b;
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int j = 0; j < NACC; ++j) {
            if constexpr (BIG)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc[j], 0, 0, 0);
            else
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[j], 0, 0, 0);
        }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
        for (int r = 0; r < R; ++r) s += acc[j][r];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
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

// Launches `grid` workgroups of `block` lanes (a multiple of 64, at most
// 1024), each lane running `iters` rounds of `nacc` (1, 2 or 4) independent
// fp32 MFMAs of shape 32 x 32 x 2 (shape 32) or 16 x 16 x 4 (shape 16).
// `out` holds grid * block floats.  Flops per launch:
// grid * block / 64 * iters * nacc * (4,096 or 2,048).  Returns the launch's
// hipError_t, or hipErrorInvalidValue (without launching) for other values.
int probe_mfma(int shape, int nacc, int grid, int block, int iters, float *out,
               hipStream_t stream) {
    if ((shape != 32 && shape != 16) || grid < 1 || block < 64 || block > 1024 ||
        block % 64 != 0 || iters < 0)
        return (int)hipErrorInvalidValue;
    void (*k)(float, float, int, float *) = nullptr;
    if (shape == 32)
        k = nacc == 1 ? mfma_kernel<true, 1> : nacc == 2 ? mfma_kernel<true, 2>
            : nacc == 4 ? mfma_kernel<true, 4> : nullptr;
    else
        k = nacc == 1 ? mfma_kernel<false, 1> : nacc == 2 ? mfma_kernel<false, 2>
            : nacc == 4 ? mfma_kernel<false, 4> : nullptr;
    if (!k) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k, dim3(grid), dim3(block), 0, stream, 1.0f, 1e-3f, iters, out);
    return (int)hipGetLastError();
}

}  // extern "C"
