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

namespace gg {

// C = alpha * op(A).op(B) + beta * C (C not read when beta == 0).
// ax: A stored M x K (else K x M, i.e. op(A) = A^T); bx: B stored N x K
// (op(B) = B^T, else K x N).  num_cus is the device's compute-unit count (it
// picks the tile shape).  K = 0 writes beta * C (zeros for beta = 0).
hipError_t launch_gemm(bool ax, bool bx, int M, int N, int K, float alpha, const float *A,
                       int64_t lda, const float *B, int64_t ldb, float beta, float *C,
                       int64_t ldc, int num_cus, hipStream_t stream);

// y = W.x, fp32.
hipError_t launch_gemv_f32(int M, int K, const float *W, int64_t ldw,
                           const float *x, float *y, hipStream_t stream);

// y_b = W_b.x_b for b < count, W_b as 2-bit (q2) or 4-bit (q4) codes with
// one binary16 scale per 64 columns; the pointer arrays are host arrays of
// device pointers.
constexpr int PACKED_MAX_BATCH = 64;
hipError_t launch_gemv_q2(int count, int M, int K, const uint8_t *const *Q, int64_t ldq,
                          const uint16_t *const *S, int64_t lds, const float *const *x,
                          float *const *y, hipStream_t stream);
hipError_t launch_gemv_q4(int count, int M, int K, const uint8_t *const *Q, int64_t ldq,
                          const uint16_t *const *S, int64_t lds, const float *const *x,
                          float *const *y, hipStream_t stream);

}  // namespace gg
