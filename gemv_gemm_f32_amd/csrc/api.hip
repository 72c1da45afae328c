// api.hip -- the C entry points of libgemvgemm.so (declared in gemvgemm.h).
//
// Each entry point validates its arguments before any HIP call and before
// anything is written, checks once per device that the current device is a
// gfx950, launches one kernel on the caller's stream, and maps a rejected
// launch to a status.  No exception or abort leaves this file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/gemvgemm.h"
#include "kernels.hpp"

namespace {

constexpr int64_t kMaxDim = INT32_MAX;   // sizes must be below 2^31
constexpr int kMaxDevices = 64;

// Per-device cache: 0 unknown, else 1 + compute-unit count for a gfx950 and
// -1 for any other device.  Filled without a lock; a race only repeats the
// query and stores the same answer.
std::atomic<int> g_device_info[kMaxDevices];

// GG_OK and the current device's CU count, or an error status.
int check_device(int *num_cus) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GG_ERR_NO_DEVICE;
    if (dev < kMaxDevices) {
        const int known = g_device_info[dev].load(std::memory_order_relaxed);
        if (known > 0) {
            *num_cus = known - 1;
            return GG_OK;
        }
        if (known < 0) return GG_ERR_NO_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GG_ERR_NO_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    const int cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
    if (dev < kMaxDevices) g_device_info[dev].store(ok ? 1 + cus : -1, std::memory_order_relaxed);
    *num_cus = cus;
    return ok ? GG_OK : GG_ERR_NO_DEVICE;
}

// Byte range [lo, hi) of a rows x cols matrix with leading dimension ld.
struct Span {
    uintptr_t lo, hi;
};

// Bytes from p to the end of the matrix's last element (sizes below 2^31,
// so the product fits in 128 bits).
unsigned __int128 extent_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t elem) {
    if (rows <= 0 || cols <= 0) return 0;
    return ((unsigned __int128)(rows - 1) * (uint64_t)ld + (uint64_t)cols) * (uint64_t)elem;
}

// A matrix whose bytes would run past the end of the address space.
bool wraps(const void *p, int64_t rows, int64_t cols, int64_t ld, int64_t elem) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    return extent_bytes(rows, cols, ld, elem) > (unsigned __int128)(UINTPTR_MAX - b);
}

// Only for matrices that do not wrap.
Span span(const void *p, int64_t rows, int64_t cols, int64_t ld, int64_t elem) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    return {b, b + (uintptr_t)extent_bytes(rows, cols, ld, elem)};
}

bool overlaps(Span a, Span b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool bad_ptr(const void *p, int64_t align) {
    return p == nullptr || (reinterpret_cast<uintptr_t>(p) % (uintptr_t)align) != 0;
}

int launch_status(hipError_t e) { return e == hipSuccess ? GG_OK : GG_ERR_LAUNCH; }

// The byte range of one operand of a batch, and whether it is an output.
struct Iv {
    Span s;
    bool out;
};

// True when every output is disjoint from every input and from every other
// output (inputs may overlap each other, e.g. a shared x).  Sorted sweep: an
// interval overlaps an earlier one exactly when its start lies below the
// largest end seen so far.
bool outputs_disjoint(std::vector<Iv> &iv) {
    std::sort(iv.begin(), iv.end(), [](const Iv &a, const Iv &b) { return a.s.lo < b.s.lo; });
    uintptr_t end_all = 0, end_out = 0;
    for (const Iv &v : iv) {
        if (v.s.lo >= v.s.hi) continue;
        if (v.out ? end_all > v.s.lo : end_out > v.s.lo) return false;
        end_all = end_all > v.s.hi ? end_all : v.s.hi;
        if (v.out) end_out = end_out > v.s.hi ? end_out : v.s.hi;
    }
    return true;
}

// The checks and launch shared by gemv_f32 and gemv_f32_batched.
int f32_batched(int64_t count, int64_t M, int64_t K, const float *const *W, int64_t ldw,
                const float *const *x, float *const *y, gg_stream_t stream) {
    if (count < 0 || count > kMaxDim || M < 0 || K < 0 || M > kMaxDim || K > kMaxDim)
        return GG_ERR_INVALID_ARG;
    if (count == 0 || M == 0) return GG_OK;
    if (W == nullptr || x == nullptr || y == nullptr) return GG_ERR_INVALID_ARG;
    if (K > 0 && (ldw < K || ldw > kMaxDim)) return GG_ERR_INVALID_ARG;
    for (int64_t b = 0; b < count; ++b) {
        if (bad_ptr(y[b], 4) || wraps(y[b], 1, M, M, 4)) return GG_ERR_INVALID_ARG;
        if (K > 0 && (bad_ptr(W[b], 4) || bad_ptr(x[b], 4) || wraps(W[b], M, K, ldw, 4) ||
                      wraps(x[b], 1, K, K, 4)))
            return GG_ERR_INVALID_ARG;
    }
    if (K > 0 || count > 1) {
        std::vector<Iv> iv;
        iv.reserve((size_t)count * 3);
        for (int64_t b = 0; b < count; ++b) {
            iv.push_back({span(y[b], 1, M, M, 4), true});
            if (K > 0) {
                iv.push_back({span(W[b], M, K, ldw, 4), false});
                iv.push_back({span(x[b], 1, K, K, 4), false});
            }
        }
        if (!outputs_disjoint(iv)) return GG_ERR_ALIAS;
    }
    int cus = 0;
    if (int st = check_device(&cus)) return st;
    return launch_status(gg::launch_gemv_f32((int)count, (int)M, (int)K, W, ldw, x, y,
                                             reinterpret_cast<hipStream_t>(stream)));
}

// op(A) = A^T when ta (A stored K x M), op(B) = B^T when tb (B stored N x K).
int gemm_common(bool ta, bool tb, int64_t M, int64_t N, int64_t K, float alpha, const float *A,
                int64_t lda, const float *B, int64_t ldb, float beta, float *C, int64_t ldc,
                gg_stream_t stream) {
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return GG_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return GG_OK;
    // A and B are read only when the product term is present.
    const bool use_ab = K > 0 && alpha != 0.f;
    const int64_t a_rows = ta ? K : M, a_cols = ta ? M : K;
    const int64_t b_rows = tb ? N : K, b_cols = tb ? K : N;
    if (bad_ptr(C, 4)) return GG_ERR_INVALID_ARG;
    if (use_ab && (bad_ptr(A, 4) || bad_ptr(B, 4))) return GG_ERR_INVALID_ARG;
    if (ldc < N || ldc > kMaxDim) return GG_ERR_INVALID_ARG;
    if (use_ab && (lda < a_cols || ldb < b_cols || lda > kMaxDim || ldb > kMaxDim))
        return GG_ERR_INVALID_ARG;
    if (wraps(C, M, N, ldc, 4) ||
        (use_ab && (wraps(A, a_rows, a_cols, lda, 4) || wraps(B, b_rows, b_cols, ldb, 4))))
        return GG_ERR_INVALID_ARG;
    const Span c = span(C, M, N, ldc, 4);
    if (use_ab && (overlaps(c, span(A, a_rows, a_cols, lda, 4)) ||
                   overlaps(c, span(B, b_rows, b_cols, ldb, 4))))
        return GG_ERR_ALIAS;
    int cus = 0;
    if (int st = check_device(&cus)) return st;
    return launch_status(gg::launch_gemm(!ta, tb, (int)M, (int)N, use_ab ? (int)K : 0, alpha,
                                         A, lda, B, ldb, beta, C, ldc, cus,
                                         reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int gemm_f32(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
             int64_t ldb, float *C, int64_t ldc, gg_stream_t stream) {
    return gemm_common(false, false, M, N, K, 1.f, A, lda, B, ldb, 0.f, C, ldc, stream);
}

int gemm_f32_tn(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                int64_t ldb, float *C, int64_t ldc, gg_stream_t stream) {
    return gemm_common(true, false, M, N, K, 1.f, A, lda, B, ldb, 0.f, C, ldc, stream);
}

int gemm_f32_nt(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                int64_t ldb, float *C, int64_t ldc, gg_stream_t stream) {
    return gemm_common(false, true, M, N, K, 1.f, A, lda, B, ldb, 0.f, C, ldc, stream);
}

int gemm_f32_ex(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, float alpha,
                const float *A, int64_t lda, const float *B, int64_t ldb, float beta, float *C,
                int64_t ldc, gg_stream_t stream) {
    if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1))
        return GG_ERR_INVALID_ARG;
    return gemm_common(trans_a == 1, trans_b == 1, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                       stream);
}

int gemv_f32(int64_t M, int64_t K, const float *W, int64_t ldw, const float *x, float *y,
             gg_stream_t stream) {
    if (M < 0 || K < 0 || M > kMaxDim || K > kMaxDim) return GG_ERR_INVALID_ARG;
    if (M == 0) return GG_OK;
    // one product of the batched entry point (same checks, same kernel)
    return f32_batched(1, M, K, &W, ldw, &x, &y, stream);
}

int gemv_f32_batched(int64_t count, int64_t M, int64_t K, const float *const *W, int64_t ldw,
                     const float *const *x, float *const *y, gg_stream_t stream) {
    return f32_batched(count, M, K, W, ldw, x, y, stream);
}

}  // extern "C"

namespace {

// A caller's workspace (scratch false), or the library's fixed per-device
// scratch buffer (scratch true: found after the device check).
struct Workspace {
    void *p;
    int64_t bytes;
    bool scratch;
};

// The checks and launch shared by the 2-bit and 4-bit entry points.  With a
// workspace (2-bit only) a batch of long rows may cut them into slices whose
// partial sums go there.
int packed_batched(int bits, int64_t count, int64_t M, int64_t K, const uint8_t *const *Q,
                   int64_t ldq, const uint16_t *const *S, int64_t lds, const float *const *x,
                   float *const *y, const Workspace *ws, gg_stream_t stream) {
    if (count < 0 || count > kMaxDim || M < 0 || K < 0 || M > kMaxDim || K > kMaxDim)
        return GG_ERR_INVALID_ARG;
    if (count == 0 || M == 0) return GG_OK;
    if (Q == nullptr || S == nullptr || x == nullptr || y == nullptr) return GG_ERR_INVALID_ARG;
    const int64_t per_byte = 8 / bits;
    const int64_t qcols = (K + per_byte - 1) / per_byte, scols = (K + 63) / 64;
    if (K > 0 && (ldq < qcols || lds < scols || ldq > kMaxDim || lds > kMaxDim))
        return GG_ERR_INVALID_ARG;
    for (int64_t b = 0; b < count; ++b) {
        if (bad_ptr(y[b], 4) || wraps(y[b], 1, M, M, 4)) return GG_ERR_INVALID_ARG;
        if (K > 0 && (bad_ptr(Q[b], 1) || bad_ptr(S[b], 2) || bad_ptr(x[b], 4) ||
                      wraps(Q[b], M, qcols, ldq, 1) || wraps(S[b], M, scols, lds, 2) ||
                      wraps(x[b], 1, K, K, 4)))
            return GG_ERR_INVALID_ARG;
    }
    // The workspace this batch uses, if any: 16-byte aligned, large enough,
    // and written like an output.
    const int64_t ws_floats = (ws && bits == 2) ? gg::gemv_q2_workspace_floats(count, M, K) : 0;
    if (ws_floats > 0 && ws->scratch && ws_floats * 4 > gg::SCRATCH_BYTES) return GG_ERR_SCRATCH;
    if (ws_floats > 0 && !ws->scratch) {
        if (ws->bytes < ws_floats * 4 || bad_ptr(ws->p, 16) || wraps(ws->p, 1, ws_floats, ws_floats, 4))
            return GG_ERR_INVALID_ARG;
    }
    // Every output must be disjoint from every input and from every other
    // output, across the whole batch.
    if (K > 0 || count > 1 || ws_floats > 0) {
        std::vector<Iv> iv;
        iv.reserve((size_t)count * 4 + 1);
        for (int64_t b = 0; b < count; ++b) {
            iv.push_back({span(y[b], 1, M, M, 4), true});
            if (K > 0) {
                iv.push_back({span(Q[b], M, qcols, ldq, 1), false});
                iv.push_back({span(S[b], M, scols, lds, 2), false});
                iv.push_back({span(x[b], 1, K, K, 4), false});
            }
        }
        if (ws_floats > 0 && !ws->scratch)
            iv.push_back({span(ws->p, 1, ws_floats, ws_floats, 4), true});
        if (!outputs_disjoint(iv)) return GG_ERR_ALIAS;
    }
    int cus = 0;
    if (int st = check_device(&cus)) return st;
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    float *wsp = nullptr;
    if (ws_floats > 0) {
        wsp = ws->scratch ? gg::device_scratch() : static_cast<float *>(ws->p);
        if (wsp == nullptr) return GG_ERR_SCRATCH;
    }
    return launch_status(bits == 2 ? gg::launch_gemv_q2((int)count, (int)M, (int)K, Q, ldq, S,
                                                        lds, x, y, wsp, hs)
                                   : gg::launch_gemv_q4((int)count, (int)M, (int)K, Q, ldq, S,
                                                        lds, x, y, hs));
}

}  // namespace

extern "C" {

int gemv_q2_batched(int64_t count, int64_t M, int64_t K, const uint8_t *const *Q, int64_t ldq,
                    const uint16_t *const *S, int64_t lds, const float *const *x,
                    float *const *y, gg_stream_t stream) {
    return packed_batched(2, count, M, K, Q, ldq, S, lds, x, y, nullptr, stream);
}

int64_t gemv_q2_batched_ws_size(int64_t count, int64_t M, int64_t K) {
    if (count < 0 || count > kMaxDim || M < 0 || K < 0 || M > kMaxDim || K > kMaxDim)
        return GG_ERR_INVALID_ARG;
    return 4 * gg::gemv_q2_workspace_floats(count, M, K);
}

int gemv_q2_batched_ws(int64_t count, int64_t M, int64_t K, const uint8_t *const *Q,
                       int64_t ldq, const uint16_t *const *S, int64_t lds, const float *const *x,
                       float *const *y, void *workspace, int64_t workspace_bytes,
                       gg_stream_t stream) {
    const Workspace ws{workspace, workspace_bytes, false};
    return packed_batched(2, count, M, K, Q, ldq, S, lds, x, y, &ws, stream);
}

int gemv_q2_batched_noalloc(int64_t count, int64_t M, int64_t K, const uint8_t *const *Q,
                            int64_t ldq, const uint16_t *const *S, int64_t lds,
                            const float *const *x, float *const *y, gg_stream_t stream) {
    const Workspace ws{nullptr, 0, true};
    return packed_batched(2, count, M, K, Q, ldq, S, lds, x, y, &ws, stream);
}

int gemv_q2(int64_t M, int64_t K, const uint8_t *Q, int64_t ldq, const uint16_t *S,
            int64_t lds, const float *x, float *y, gg_stream_t stream) {
    if (M < 0 || K < 0 || M > kMaxDim || K > kMaxDim) return GG_ERR_INVALID_ARG;
    if (M == 0) return GG_OK;
    // one product of the batched entry point (same checks, same kernel)
    return packed_batched(2, 1, M, K, &Q, ldq, &S, lds, &x, &y, nullptr, stream);
}

int gemv_q4_batched(int64_t count, int64_t M, int64_t K, const uint8_t *const *Q, int64_t ldq,
                    const uint16_t *const *S, int64_t lds, const float *const *x,
                    float *const *y, gg_stream_t stream) {
    return packed_batched(4, count, M, K, Q, ldq, S, lds, x, y, nullptr, stream);
}

int gemv_q4(int64_t M, int64_t K, const uint8_t *Q, int64_t ldq, const uint16_t *S,
            int64_t lds, const float *x, float *y, gg_stream_t stream) {
    if (M < 0 || K < 0 || M > kMaxDim || K > kMaxDim) return GG_ERR_INVALID_ARG;
    if (M == 0) return GG_OK;
    return packed_batched(4, 1, M, K, &Q, ldq, &S, lds, &x, &y, nullptr, stream);
}

const char *gg_strerror(int status) {
    switch (status) {
        case GG_OK: return "success";
        case GG_ERR_INVALID_ARG:
            return "invalid argument: negative or oversized size, null or misaligned "
                   "pointer, or leading dimension smaller than the row width";
        case GG_ERR_ALIAS: return "output overlaps an input";
        case GG_ERR_NO_DEVICE: return "no current HIP device, or it is not a gfx950 (MI355X)";
        case GG_ERR_LAUNCH: return "kernel launch failed";
        case GG_ERR_SCRATCH:
            return "the batch needs more than the library's fixed scratch buffer holds (4 MiB "
                   "per GPU), or that buffer could not be located on the current device";
        default: return "unknown status";
    }
}

}  // extern "C"
