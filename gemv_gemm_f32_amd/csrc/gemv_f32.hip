// gemv_f32.hip -- fp32 y = W.x, bound by streaming W from HBM.
//
// The one-row matrix-vector path of "More Stumbling, This Time in the
// Browser" (section "Four answers per worker") at the 12,288 x 1,536 shape of
// "Kernel 0112" (section "What is being measured").  That page finds that the
// original kernel launched too few threads to keep enough reads in flight and
// that splitting each dot product over more threads paid (sections "What is
// being measured" and "The four variants").  On CDNA4 the split is a whole
// wave64 per row:
//
//  * Lane l reads the 16-byte chunks l, l+64, l+128, ... of a row, so each
//    load instruction covers 1 KiB of contiguous row.  Each wave owns R
//    consecutive rows and issues all R x U chunk loads of a pass before using
//    any of them, which keeps R x U KiB per wave in flight.  One row per wave
//    (12,288 waves at 12,288 rows) streamed faster than 2, 4 or 8.
//  * W is read once and never again, so its loads are non-temporal: they do
//    not displace x or other data from the caches (12.5 against 13.9 us per
//    12,288 x 1,536 call).
//  * The matching chunks of x are loaded once per pass and reused for the R
//    rows; x is 6 KiB and stays in L2/L1.
//  * A row's 64 partial sums are added with the DPP/swizzle tree of wave.hpp;
//    lane 0 writes y.
//  * Scalar-load specialisation of the same kernel for K, ldw or a base that
//    is not a multiple of 4 floats.
//  * Batches: the same kernel runs up to 64 products of one shape per launch,
//    blockIdx.y picking the product, whose W, x and y pointers travel in the
//    kernel arguments.  The page counts 40 of these products per generated
//    token; one launch each pays the fixed dispatch cost 40 times.  Every
//    product's arithmetic is the single call's, so the two agree bit for bit.
#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "wave.hpp"

namespace gg {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int THREADS = 256;
constexpr int WAVES = THREADS / 64;

// The pointers of NB products (kernel arguments; entries past the launch's
// product count repeat product 0 and are never used).
template <int NB>
struct F32Ptrs {
    const float *W[NB];
    const float *x[NB];
    float *y[NB];
};

template <int R, int U, bool VEC, int NB>
__global__ __launch_bounds__(THREADS) void gemv_f32_kernel(int M, int K, int64_t ldw,
                                                           F32Ptrs<NB> p) {
    const int b = NB == 1 ? 0 : (int)blockIdx.y;
    const float *__restrict__ W = p.W[b];
    const float *__restrict__ x = p.x[b];
    float *__restrict__ y = p.y[b];
    const int lane = threadIdx.x & 63;
    const int row0 = (blockIdx.x * WAVES + (threadIdx.x >> 6)) * R;
    if (row0 >= M) return;   // uniform per wave

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;

    // Loads are unconditional, from clamped (in-bounds) indices, so a pass
    // issues all of them back to back; rows past M are computed on the last
    // row and not stored, chunks past K are zeroed after a scheduling barrier.
    const int rl = M - 1;
    if (VEC) {
        const int nv = K >> 2;                       // 16-byte chunks per row
        const v4f *x4 = reinterpret_cast<const v4f *>(x);
        for (int c0 = 0; c0 < nv; c0 += 64 * U) {
            v4f xv[U];
            v4f wv[R][U];
#pragma unroll
            for (int u = 0; u < U; ++u) xv[u] = x4[min(c0 + lane + 64 * u, nv - 1)];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const v4f *wr = reinterpret_cast<const v4f *>(W + (int64_t)min(row0 + r, rl) * ldw);
#pragma unroll
                for (int u = 0; u < U; ++u)
                    wv[r][u] = __builtin_nontemporal_load(wr + min(c0 + lane + 64 * u, nv - 1));
            }
            __builtin_amdgcn_sched_barrier(0);
            if (c0 + 64 * U > nv) {                  // uniform: a partial pass
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const bool live = c0 + lane + 64 * u < nv;
                    xv[u] = live ? xv[u] : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        wv[r][u] = live ? wv[r][u] : v4f{0.f, 0.f, 0.f, 0.f};
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    acc[r] = __builtin_fmaf(wv[r][u].x, xv[u].x, acc[r]);
                    acc[r] = __builtin_fmaf(wv[r][u].y, xv[u].y, acc[r]);
                    acc[r] = __builtin_fmaf(wv[r][u].z, xv[u].z, acc[r]);
                    acc[r] = __builtin_fmaf(wv[r][u].w, xv[u].w, acc[r]);
                }
        }
    } else {
        for (int k0 = 0; k0 < K; k0 += 64 * U) {
            float xv[U];
            float wv[R][U];
#pragma unroll
            for (int u = 0; u < U; ++u) xv[u] = x[min(k0 + lane + 64 * u, K - 1)];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int u = 0; u < U; ++u)
                    wv[r][u] = __builtin_nontemporal_load(
                        W + (int64_t)min(row0 + r, rl) * ldw + min(k0 + lane + 64 * u, K - 1));
            __builtin_amdgcn_sched_barrier(0);
            if (k0 + 64 * U > K) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const bool live = k0 + lane + 64 * u < K;
                    xv[u] = live ? xv[u] : 0.f;
#pragma unroll
                    for (int r = 0; r < R; ++r) wv[r][u] = live ? wv[r][u] : 0.f;
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int u = 0; u < U; ++u) acc[r] = __builtin_fmaf(wv[r][u], xv[u], acc[r]);
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float s = wave64_sum(acc[r]);
        if (lane == 0 && row0 + r < M) y[row0 + r] = s;
    }
}

template <int NB>
hipError_t launch_f32(int count, int M, int K, const float *const *W, int64_t ldw,
                      const float *const *x, float *const *y, hipStream_t s) {
    constexpr int R = 1;
    const int waves = (M + R - 1) / R;
    const dim3 grid((waves + WAVES - 1) / WAVES, count);
    F32Ptrs<NB> p;
    bool vec = ldw % 4 == 0 && K % 4 == 0;
    for (int b = 0; b < NB; ++b) {
        const int i = b < count ? b : 0;
        p.W[b] = W[i];
        p.x[b] = x[i];
        p.y[b] = y[i];
        vec = vec && reinterpret_cast<uintptr_t>(W[i]) % 16 == 0 &&
              reinterpret_cast<uintptr_t>(x[i]) % 16 == 0;
    }
    if (vec) return launch(gemv_f32_kernel<R, 6, true, NB>, grid, dim3(THREADS), s, M, K, ldw, p);
    return launch(gemv_f32_kernel<R, 8, false, NB>, grid, dim3(THREADS), s, M, K, ldw, p);
}

}  // namespace

hipError_t launch_gemv_f32(int count, int M, int K, const float *const *W, int64_t ldw,
                           const float *const *x, float *const *y, hipStream_t s) {
    if (count == 1) return launch_f32<1>(1, M, K, W, ldw, x, y, s);
    for (int b0 = 0; b0 < count; b0 += F32_MAX_BATCH) {
        const int n = count - b0 < F32_MAX_BATCH ? count - b0 : F32_MAX_BATCH;
        const hipError_t e = launch_f32<F32_MAX_BATCH>(n, M, K, W + b0, ldw, x + b0, y + b0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gg
