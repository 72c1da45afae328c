// kernels.hpp -- launch functions exported by the kernel translation units to
// the C entry points (api.hip).  Internal to libgemvgemm.so.
//
// Each launcher assumes its arguments were validated by the caller: sizes in
// [0, 2^31), non-null aligned pointers for non-empty operands, leading
// dimensions at least the row width, output not aliasing an input.  It only
// picks a compile-time specialisation and a grid, and launches.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace gg {

// Launches kernel<<<grid, block, 0, s>>>(args...) and returns that launch's
// own status from hipLaunchKernel, so an error left pending by an earlier,
// unrelated HIP call is neither reported as ours nor cleared.  The arguments
// are converted to the kernel's parameter types first.
template <typename... P, size_t... I>
hipError_t launch_args(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s,
                       std::tuple<P...> &args, std::index_sequence<I...>) {
    void *ptrs[sizeof...(P) + 1] = {static_cast<void *>(&std::get<I>(args))..., nullptr};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, 0, s);
}

template <typename... P, typename... A>
hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s, A &&...a) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    std::tuple<P...> args(std::forward<A>(a)...);
    return launch_args(kernel, grid, block, s, args, std::index_sequence_for<P...>{});
}

// C = alpha * op(A).op(B) + beta * C (C not read when beta == 0).
// ax: A stored M x K (else K x M, i.e. op(A) = A^T); bx: B stored N x K
// (op(B) = B^T, else K x N).  num_cus is the device's compute-unit count (it
// picks the tile shape).  K = 0 writes beta * C (zeros for beta = 0).
hipError_t launch_gemm(bool ax, bool bx, int M, int N, int K, float alpha, const float *A,
                       int64_t lda, const float *B, int64_t ldb, float beta, float *C,
                       int64_t ldc, int num_cus, hipStream_t stream);

// y_b = W_b.x_b for b < count, fp32; the pointer arrays are host arrays of
// device pointers.  More than F32_MAX_BATCH products take several launches
// in order; if one of them is rejected the earlier ones stay queued.
constexpr int F32_MAX_BATCH = 64;
hipError_t launch_gemv_f32(int count, int M, int K, const float *const *W, int64_t ldw,
                           const float *const *x, float *const *y, hipStream_t stream);

// y_b = W_b.x_b for b < count, W_b as 2-bit (q2) or 4-bit (q4) codes with
// one binary16 scale per 64 columns; the pointer arrays are host arrays of
// device pointers.  More than PACKED_MAX_BATCH products take several
// launches in order; if one of them is rejected the earlier ones stay
// queued.
constexpr int PACKED_MAX_BATCH = 64;
// ws: NULL, or a workspace of gemv_q2_workspace_floats(count, M, K) floats
// that batches of long rows use for partial sums (rows cut into slices);
// without it they take a kernel that needs none.
hipError_t launch_gemv_q2(int count, int M, int K, const uint8_t *const *Q, int64_t ldq,
                          const uint16_t *const *S, int64_t lds, const float *const *x,
                          float *const *y, float *ws, hipStream_t stream);
// Batches of 2-bit products whose rows are long cut them into slices of
// SLICE_K columns, each written to the workspace as partial row sums, when
// a workspace is given: rows of 4 to SLICED_MAX slices, at least
// SLICED_MIN_COUNT products (at 1,536 x 12,288, µs per product sliced
// against whole: 4 products 2.46 / 2.39, 8: 1.67 / 1.77, 16: 1.32 / 1.49,
// 40: 1.08 / 1.33).  Slices of
// SLICE_K/512 waves each, as the integer-dot kernel is tuned for.
constexpr int SLICE_K = 1536;
constexpr int SLICED_MIN_COUNT = 8;
constexpr int SLICED_MAX = 1024;

// Slices per row for a batch of this shape, 0 where it is not cut.
inline int64_t sliced_count(int64_t count, int64_t M, int64_t K) {
    if (count < SLICED_MIN_COUNT || M < 1 || K % SLICE_K != 0) return 0;
    const int64_t n = K / SLICE_K;
    return n >= 4 && n <= SLICED_MAX ? n : 0;
}

// The fixed per-device scratch buffer of the allocation-free entry point
// (noalloc.hip): its size, and its device address on the current device
// (found on first use there), or NULL if it cannot be had.
constexpr int64_t SCRATCH_BYTES = int64_t(4) << 20;
float *device_scratch();

// Floats of workspace a 2-bit batch of this shape uses, 0 if none: one
// launch's partial sums (the next launch of a batch over PACKED_MAX_BATCH
// products reuses them).
inline int64_t gemv_q2_workspace_floats(int64_t count, int64_t M, int64_t K) {
    const int64_t n = sliced_count(count, M, K);
    return n ? (count < PACKED_MAX_BATCH ? count : PACKED_MAX_BATCH) * n * M : 0;
}
hipError_t launch_gemv_q4(int count, int M, int K, const uint8_t *const *Q, int64_t ldq,
                          const uint16_t *const *S, int64_t lds, const float *const *x,
                          float *const *y, hipStream_t stream);

}  // namespace gg
