/*
 * gemvgemm.h -- C interface of libgemvgemm.so: fp32 matrix products, the fp32
 * matrix-vector product, and the 2-bit and 4-bit packed-weight matrix-vector
 * products, as hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every matrix is row-major with an explicit leading dimension (the stride,
 *    in elements, between the starts of consecutive rows).
 *  - Every data pointer is a DEVICE pointer on the calling thread's current
 *    HIP device.  The caller owns all memory; the library allocates nothing and
 *    keeps no pointer after a call returns.
 *  - Calls are asynchronous: work is queued on `stream` (NULL = the legacy
 *    default stream) and results are valid once the caller has synchronised
 *    that stream.  A fault inside a kernel surfaces at that synchronisation,
 *    as with any HIP launch.
 *  - The output is overwritten (no accumulation into it).  With K = 0 the
 *    output is written with zeros, the empty sum.
 *  - Each call returns a status.  Arguments are checked before any HIP call
 *    and before anything is written: a non-zero status means nothing was
 *    launched.  Checks, in order: sizes non-negative and below 2^31; an empty
 *    output returns GG_OK at once; non-null pointers, aligned to their element
 *    size, for every operand of non-zero extent; leading dimensions at least
 *    the row width; no operand's byte range running past the end of the
 *    address space; the output's byte range disjoint from every input's; the
 *    current device is a gfx950.  No exception or abort crosses this
 *    interface.  GG_ERR_LAUNCH reports the status of this call's own
 *    launch; an error left pending by an earlier HIP call is neither
 *    reported nor cleared.  (The one exception to "nothing was launched":
 *    a batch of more than 64 products takes several launches, and if a
 *    later one is rejected the earlier ones stay queued.)
 *  - Results are reproducible bit for bit from run to run on the same shapes
 *    (fixed reduction trees, no floating-point atomics).  They agree with the
 *    exact sum to |c - c_exact| <= 1e-4 * sum_k |a_ik * b_kj| per element for
 *    finite inputs whose partial sums stay in the normal fp32 range (for the
 *    packed products: the largest |x_k| in [2^-100, 2^100]; see there); fp32
 *    operands are used as IEEE fp32 (no reduced-precision inputs).
 *  - Non-finite inputs: the fp32 products follow IEEE arithmetic, so a NaN
 *    operand makes exactly the outputs whose sums contain it NaN, and an
 *    infinity gives +-inf there (NaN where it meets a zero or an opposite
 *    infinity).  The packed products do not: they apply the zero point
 *    through sums of x (or round x to integers), so a NaN or an infinity
 *    anywhere in x makes EVERY output NaN, where the exact sum would give
 *    +-inf in rows that meet an infinity; a NaN scale makes its own row NaN.
 *  - Thread safety: the only global state is a per-device property cache
 *    filled once; every entry point may be called from several threads.
 *    The one exception is gemv_q2_batched_noalloc, whose calls share one
 *    scratch buffer per GPU: calls of it that overlap on one GPU race.
 */
#ifndef GEMVGEMM_H
#define GEMVGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t, declared here so C callers need no HIP headers. */
typedef struct ihipStream_t *gg_stream_t;

enum gg_status {
    GG_OK = 0,
    GG_ERR_INVALID_ARG = -1, /* negative/oversized size, null or misaligned
                                pointer, leading dimension too small        */
    GG_ERR_ALIAS = -2,       /* output overlaps an input                     */
    GG_ERR_NO_DEVICE = -3,   /* no current HIP device, or it is not gfx950   */
    GG_ERR_LAUNCH = -4,      /* the kernel launch itself was rejected        */
    GG_ERR_SCRATCH = -5      /* gemv_q2_batched_noalloc: the batch needs more
                                than the fixed scratch buffer holds           */
};

/*
 * C[M x N] = A[M x K] . B[K x N]
 *
 * The dense matrix product: each output cell walks the inner dimension,
 * multiplying an activation by its weight and adding the products ("More
 * Stumbling, This Time in the Browser", section "Four answers per worker";
 * the square sizes of "I built a GPT-2 in the browser, then made it
 * 2.6x-12.1x faster", section "The kernel sweep").
 *   A[i*lda + k], lda >= K;  B[k*ldb + j], ldb >= N;  C[i*ldc + j], ldc >= N.
 * M = 1 is legal here and runs the same kernel (gemv_f32 is the one-row path).
 */
int gemm_f32(int64_t M, int64_t N, int64_t K,
             const float *A, int64_t lda,
             const float *B, int64_t ldb,
             float *C, int64_t ldc, gg_stream_t stream);

/*
 * C[M x N] = A^T . B with A stored K x M.
 *
 * The weight-gradient product of a hand-derived backward pass, dW = X^T.dY
 * ("I built a GPT-2 in the browser, then made it 2.6x-12.1x faster",
 * section "The architecture in 60 seconds").
 *   A[k*lda + i], lda >= M;  B[k*ldb + j], ldb >= N;  C[i*ldc + j], ldc >= N.
 */
int gemm_f32_tn(int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda,
                const float *B, int64_t ldb,
                float *C, int64_t ldc, gg_stream_t stream);

/*
 * C[M x N] = A . B^T with B stored N x K.
 *
 * The input-gradient product of a hand-derived backward pass, dX = dY.W^T
 * (same page and section as gemm_f32_tn).
 *   A[i*lda + k], lda >= K;  B[j*ldb + k], ldb >= K;  C[i*ldc + j], ldc >= N.
 */
int gemm_f32_nt(int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda,
                const float *B, int64_t ldb,
                float *C, int64_t ldc, gg_stream_t stream);

/*
 * C[M x N] = alpha * op(A) . op(B) + beta * C
 *
 * The scaled, accumulating form of the three products above, for gradient
 * accumulation (dW += X^T.dY) in the hand-derived backward pass and AdamW
 * training loop of "I built a GPT-2 in the browser, then made it
 * 2.6x-12.1x faster", section "The architecture in 60 seconds".  The pages
 * give no formula; this library reads it the BLAS way:
 *   op(A) = A (stored M x K, A[i*lda + k], lda >= K)       if trans_a == 0,
 *           A^T (stored K x M, A[k*lda + i], lda >= M)     if trans_a == 1;
 *   op(B) = B (stored K x N, B[k*ldb + j], ldb >= N)       if trans_b == 0,
 *           B^T (stored N x K, B[j*ldb + k], ldb >= K)     if trans_b == 1;
 *   C[i*ldc + j], ldc >= N, read and written in place.
 * beta == 0: C is not read (it may hold NaN).  alpha == 0 or K == 0: A and B
 * are not read (they may be NULL) and C becomes beta * C.  trans flags other
 * than 0 or 1 give GG_ERR_INVALID_ARG; C may not overlap A or B.  With
 * alpha = 1 and beta = 0 the results equal gemm_f32 / _tn / _nt bit for bit.
 */
int gemm_f32_ex(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                float alpha, const float *A, int64_t lda,
                const float *B, int64_t ldb, float beta,
                float *C, int64_t ldc, gg_stream_t stream);

/*
 * y[M] = W[M x K] . x[K]
 *
 * The single-row matrix-vector path kept beside the dense product ("More
 * Stumbling, This Time in the Browser", section "Four answers per worker"),
 * at the 12,288 x 1,536 shape of "Kernel 0112", section "What is being
 * measured".
 *   W[i*ldw + k], ldw >= K;  x and y contiguous.
 */
int gemv_f32(int64_t M, int64_t K, const float *W, int64_t ldw,
             const float *x, float *y, gg_stream_t stream);

/*
 * y_b = W_b . x_b for b = 0 .. count-1: count independent fp32 products of
 * one shape (M, K, ldw), each exactly as gemv_f32 defines it, in as few
 * launches as possible (up to 64 products per launch).  "Kernel 0112",
 * section "What is being measured", counts 40 matrix-vector products per
 * generated token; one launch per product pays a fixed dispatch cost each
 * time.
 *   W, x, y: HOST arrays of count DEVICE pointers (W[b], x[b], y[b] as in
 *   gemv_f32).  The arrays are read during the call and not kept.
 *   Every y[b] must be disjoint from every input and from every other y[c]
 *   (else GG_ERR_ALIAS); inputs may be shared (for example one x for all).
 *   Products 64 at a time share a launch, in order; GG_ERR_LAUNCH from a
 *   batch of more than 64 may leave the products of earlier launches queued.
 * Each product runs gemv_f32's arithmetic, so a batch equals count separate
 * gemv_f32 calls bit for bit.
 */
int gemv_f32_batched(int64_t count, int64_t M, int64_t K,
                     const float *const *W, int64_t ldw,
                     const float *const *x, float *const *y, gg_stream_t stream);

/*
 * y[M] = W[M x K] . x[K] with W held as 2-bit codes and binary16 scales.
 *
 * The 2-bit weight matrix times an input vector of "Kernel 0112", sections
 * "What is being measured" (12,288 x 1,536 weights, 1,536 inputs, 12,288
 * outputs) and "The kernel" (2-bit fields unpacked to floating point).  The
 * pages do not fix the packing; this library reads it as:
 *   code(i,k) = (Q[i*ldq + k/4] >> (2*(k%4))) & 3     (least significant first)
 *   s(i,k)    = binary16 S[i*lds + k/64]             (one scale per 64 columns)
 *   w(i,k)    = (code(i,k) - 1.5) * s(i,k)
 *   y[i]      = sum_k w(i,k) * x[k]
 *   Q: ldq >= ceil(K/4) bytes per row;  S: lds >= ceil(K/64) halves per row,
 *   holding IEEE binary16 bit patterns;  x (fp32) and y (fp32) contiguous.
 * Bits of Q for columns k >= K and scales past ceil(K/64) are never used.
 * Accuracy: |y_i - exact| <= 1e-4 * sum_k |w(i,k) x_k| for finite x whose
 * largest |x_k| lies in [2^-100, 2^100] and finite scales whose products
 * with x keep y finite; entries of x far below the largest may underflow in
 * partial products, which moves y by far less than the bound.  Any NaN or
 * infinity in x makes every y NaN; a NaN scale makes its own row NaN.
 */
int gemv_q2(int64_t M, int64_t K, const uint8_t *Q, int64_t ldq,
            const uint16_t *S, int64_t lds,
            const float *x, float *y, gg_stream_t stream);

/*
 * y_b = W_b . x_b for b = 0 .. count-1: count independent 2-bit products of
 * one shape (M, K, ldq, lds), each exactly as gemv_q2 defines it, in as few
 * launches as possible (up to 64 products per launch).  "Kernel 0112",
 * section "What is being measured", runs this product 40 times per generated
 * token; one launch per product pays a fixed dispatch cost each time, which
 * at this size is as large as the product itself.
 *   Q, S, x, y: HOST arrays of count DEVICE pointers (Q[b], S[b], x[b], y[b]
 *   as in gemv_q2).  The arrays are read during the call and not kept.
 *   Every y[b] must be disjoint from every input and from every other y[c]
 *   (else GG_ERR_ALIAS); inputs may be shared (for example one x for all).
 *   Products 64 at a time share a launch, in order; GG_ERR_LAUNCH from a
 *   batch of more than 64 may leave the products of earlier launches queued.
 * A batch meets gemv_q2's accuracy and non-finite behaviour and is
 * reproducible run to run, but it may take a different kernel from a gemv_q2
 * call (on the configurations' shapes it rounds x to 24-bit integers per 64
 * columns and multiplies with integer dot products), so the two need not
 * agree bit for bit.
 */
int gemv_q2_batched(int64_t count, int64_t M, int64_t K,
                    const uint8_t *const *Q, int64_t ldq,
                    const uint16_t *const *S, int64_t lds,
                    const float *const *x, float *const *y, gg_stream_t stream);

/*
 * gemv_q2_batched with a caller-owned device workspace, for batches whose
 * rows are long: "Kernel 0112", section "What is being measured", names the
 * same 2-bit product on the transposed shape (12,288 inputs -> 1,536
 * outputs), and section "What the kernel costs in a whole token" shows such
 * long rows need a deeper split than short ones.  With the workspace, a
 * batch of at least 8 products whose K is a multiple of 1,536 and at least
 * 6,144 cuts each row into K/1,536 slices handled by separate workgroups,
 * writes their partial row sums to the workspace, and adds each row's
 * partials in slice order (deterministic).  Other batches run exactly as
 * gemv_q2_batched and do not touch the workspace.
 *   workspace: DEVICE memory of at least gemv_q2_batched_ws_size(count, M,
 *   K) bytes, 16-byte aligned, disjoint from every input and output (else
 *   GG_ERR_INVALID_ARG, or GG_ERR_ALIAS for an overlap); it may be NULL
 *   when that size is 0.  Its contents on entry do not matter and on return
 *   are unspecified; it must not be used by other work until this call's
 *   work on `stream` has finished.  Calls on different streams need
 *   different workspaces.
 * Other arguments, accuracy, non-finite behaviour and launch splitting as
 * gemv_q2_batched; results are reproducible run to run, and within the
 * accuracy bound of (not bit-equal to) gemv_q2_batched's.
 */
int gemv_q2_batched_ws(int64_t count, int64_t M, int64_t K,
                       const uint8_t *const *Q, int64_t ldq,
                       const uint16_t *const *S, int64_t lds,
                       const float *const *x, float *const *y,
                       void *workspace, int64_t workspace_bytes, gg_stream_t stream);

/*
 * Bytes of workspace gemv_q2_batched_ws needs for count products of M x K
 * (0 when the batch does not cut its rows), or GG_ERR_INVALID_ARG for a
 * negative or oversized size.  It depends on the sizes only.
 */
int64_t gemv_q2_batched_ws_size(int64_t count, int64_t M, int64_t K);

/*
 * gemv_q2_batched_ws for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the partial sums go to a scratch buffer of 4 MiB that the
 * library holds on each GPU it runs on (a static device array, kept until
 * the process ends) instead of a caller's workspace.  The call allocates
 * nothing.  A batch whose workspace (gemv_q2_batched_ws_size) would exceed
 * 4 MiB is rejected with GG_ERR_SCRATCH before anything runs.  One launch's
 * partial sums are reused by the next, so that size stops growing at 64
 * products (at 1,536 x 12,288: 64 x 8 slices x 1,536 rows x 4 bytes =
 * 3 MiB).  Every call on a GPU
 * shares that GPU's buffer, which keeps the last call's partial sums (no
 * call needs it cleared): calls that overlap on one GPU, from other streams
 * or threads, race and must not be made.  Arguments and results as
 * gemv_q2_batched_ws, which it equals bit for bit.
 */
int gemv_q2_batched_noalloc(int64_t count, int64_t M, int64_t K,
                            const uint8_t *const *Q, int64_t ldq,
                            const uint16_t *const *S, int64_t lds,
                            const float *const *x, float *const *y, gg_stream_t stream);

/*
 * y[M] = W[M x K] . x[K] with W held as 4-bit codes and binary16 scales.
 *
 * 4-bit weight matrices sit beside the 2-bit one on the same path: two of the
 * kernels patched with "Kernel 0112" are 4-bit (section "What is being
 * measured"), and "More Stumbling, This Time in the Browser" has a packed
 * 4-bit (NF4) path.  No page fixes the format; this library reads it like the
 * 2-bit one:
 *   code(i,k) = (Q[i*ldq + k/2] >> (4*(k%2))) & 15   (least significant first)
 *   s(i,k)    = binary16 S[i*lds + k/64]             (one scale per 64 columns)
 *   w(i,k)    = (code(i,k) - 7.5) * s(i,k)
 *   y[i]      = sum_k w(i,k) * x[k]
 *   Q: ldq >= ceil(K/2) bytes per row;  S: lds >= ceil(K/64) halves per row;
 *   x (fp32) and y (fp32) contiguous.
 * Bits of Q for columns k >= K and scales past ceil(K/64) are never used.
 * A non-uniform codebook such as NF4 is not this format.  Accuracy and
 * non-finite inputs as for gemv_q2.
 */
int gemv_q4(int64_t M, int64_t K, const uint8_t *Q, int64_t ldq,
            const uint16_t *S, int64_t lds,
            const float *x, float *y, gg_stream_t stream);

/*
 * y_b = W_b . x_b for b = 0 .. count-1: count independent 4-bit products of
 * one shape, each exactly as gemv_q4 defines it, in as few launches as
 * possible (up to 64 products per launch).  Arguments, aliasing rules and
 * result guarantees are those of gemv_q2_batched.
 */
int gemv_q4_batched(int64_t count, int64_t M, int64_t K,
                    const uint8_t *const *Q, int64_t ldq,
                    const uint16_t *const *S, int64_t lds,
                    const float *const *x, float *const *y, gg_stream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *gg_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* GEMVGEMM_H */
