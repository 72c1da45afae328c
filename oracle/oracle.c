/*
 * oracle.c -- plain CPU oracle for the dense fp32 matrix product, its
 * one-row case, and the 2-bit and 4-bit packed-weight matrix-vector
 * products.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or helper with the HIP
 * library; the two meet only in the seeded input generators.
 *
 * Every sum is taken in IEEE binary64, in the plain order k = 0, 1, ..., K-1,
 * with one output cell at a time in the sense of the definition (the loops are
 * ordered i, k, j over a row of fp64 accumulators, which leaves each cell's
 * own sum order untouched).  A product of two fp32 values is exact in fp64
 * (24 + 24 significant bits <= 53), so each result carries only the rounding
 * of the fp64 additions.  Beside each result the oracle returns the bound
 * sum_k |a_ik * b_kj|, the scale against which the GPU result is judged.
 *
 * Sources (the pages):
 *  - "More Stumbling, This Time in the Browser", section "Four answers per
 *    worker": a dense-layer output cell is the walk along the inner dimension,
 *    multiplying an activation by its weight and adding the products; the
 *    single-row matrix-vector path is kept beside it.
 *  - "I built a GPT-2 in the browser, then made it 2.6x-12.1x faster",
 *    sections "The architecture in 60 seconds" and "The kernel sweep": matmul
 *    with hand-derived backward passes, which for Y = X.W need dX = dY.W^T and
 *    dW = X^T.dY (the transposed products below).  The same training loop
 *    (forward, backward, AdamW) accumulates gradients; the scaled and
 *    accumulating form C = alpha * op(A).op(B) + beta * C is read from that
 *    (the pages give no formula for it; beta = 0 means C is not read).
 *  - "Kernel 0112", section "What is being measured": a 12,288 x 1,536 matrix
 *    of 2-bit weights times a vector of 1,536 inputs, 12,288 outputs; section
 *    "The kernel": the 2-bit fields are unpacked to floating point before the
 *    multiply.  The pages do not fix the bit order, the code-to-value map or
 *    the scale layout; the readings taken here are: column 4q+t of a row sits
 *    in bits 2t..2t+1 of byte q (least significant first), the weight is
 *    (code - 1.5) * s, and s is the IEEE binary16 scale of columns
 *    [64g, 64g+64) stored at S[i*lds + g].
 *  - "Kernel 0112", sections "What is being measured" (two of the kernels
 *    patched beside it, 0099 and 0105, are 4-bit) and "More Stumbling, This
 *    Time in the Browser" (a packed NF4 path): 4-bit weight matrices also sit
 *    on this path, with no format given.  The reading taken for them follows
 *    the 2-bit one: column 2q+t of a row sits in bits 4t..4t+3 of byte q
 *    (least significant first), the weight is (code - 7.5) * s (16 levels
 *    symmetric about zero), and s is the binary16 scale of columns
 *    [64g, 64g+64) at S[i*lds + g].
 *
 * Pins: every function here is checked against something other than itself in
 * tests/test_oracle.py (hand-worked cases, numpy's float64 product, exact
 * integer arithmetic, exhaustive binary16 decode against numpy, identities).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

/* ---------------------------------------------------------------- dense -- */

/* C = A.B with A row-major M x K (A[i*lda+k]) and B row-major K x N
 * (B[k*ldb+j]).  C and bound are row-major M x N doubles with stride ldc. */
void oracle_gemm_nn(int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda, const float *B, int64_t ldb,
                    double *C, double *bound, int64_t ldc)
{
    for (int64_t i = 0; i < M; ++i) {
        double *c = C + i * ldc, *b = bound + i * ldc;
        for (int64_t j = 0; j < N; ++j) { c[j] = 0.0; b[j] = 0.0; }
        for (int64_t k = 0; k < K; ++k) {
            double a = (double)A[i * lda + k];
            const float *brow = B + k * ldb;
            for (int64_t j = 0; j < N; ++j) {
                double p = a * (double)brow[j];
                c[j] += p;
                b[j] += fabs(p);
            }
        }
    }
}

/* C = A^T.B where A is stored K x M (A[k*lda+i]); B as in oracle_gemm_nn. */
void oracle_gemm_tn(int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda, const float *B, int64_t ldb,
                    double *C, double *bound, int64_t ldc)
{
    for (int64_t i = 0; i < M; ++i) {
        double *c = C + i * ldc, *b = bound + i * ldc;
        for (int64_t j = 0; j < N; ++j) { c[j] = 0.0; b[j] = 0.0; }
        for (int64_t k = 0; k < K; ++k) {
            double a = (double)A[k * lda + i];
            const float *brow = B + k * ldb;
            for (int64_t j = 0; j < N; ++j) {
                double p = a * (double)brow[j];
                c[j] += p;
                b[j] += fabs(p);
            }
        }
    }
}

/* C = A.B^T where B is stored N x K (B[j*ldb+k]); A as in oracle_gemm_nn.
 * Here the natural loop is the plain dot product per cell. */
void oracle_gemm_nt(int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda, const float *B, int64_t ldb,
                    double *C, double *bound, int64_t ldc)
{
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double s = 0.0, t = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = (double)A[i * lda + k] * (double)B[j * ldb + k];
                s += p;
                t += fabs(p);
            }
            C[i * ldc + j] = s;
            bound[i * ldc + j] = t;
        }
    }
}

/* Selected cells of op(A).op(B), one dot product each, for checking a few
 * outputs of a product too large to form whole.  trans_a / trans_b = 1 means
 * the operand is stored transposed (A as K x M, B as N x K). */
void oracle_gemm_cells(int trans_a, int trans_b, int64_t K,
                       const float *A, int64_t lda, const float *B, int64_t ldb,
                       int64_t n_cells, const int64_t *rows, const int64_t *cols,
                       double *c_out, double *bound_out)
{
    for (int64_t q = 0; q < n_cells; ++q) {
        int64_t i = rows[q], j = cols[q];
        double s = 0.0, t = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = trans_a ? (double)A[k * lda + i] : (double)A[i * lda + k];
            double b = trans_b ? (double)B[j * ldb + k] : (double)B[k * ldb + j];
            double p = a * b;
            s += p;
            t += fabs(p);
        }
        c_out[q] = s;
        bound_out[q] = t;
    }
}

/* ----------------------------------------------------------------- gemv -- */

/* C_out = alpha * op(A).op(B) + beta * C_in, one cell at a time:
 *   s  = sum_k opA(i,k) * opB(k,j), k = 0, 1, ..., K-1 (fp64)
 *   c  = alpha * s + beta * C_in[i*ldc + j]   (the C_in term only if beta != 0,
 *        so C_in is not read when beta == 0 and may hold anything; likewise
 *        the product term only if alpha != 0 and K > 0, so A and B are then
 *        not read)
 * with opA(i,k) = A[k*lda + i] if trans_a else A[i*lda + k] and
 *      opB(k,j) = B[j*ldb + k] if trans_b else B[k*ldb + j].
 * bound = |alpha| * sum_k |opA * opB| + |beta * C_in|.  C_out and bound are
 * M x N doubles with stride N. */
void oracle_gemm_ex(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                    double alpha, const float *A, int64_t lda,
                    const float *B, int64_t ldb, double beta,
                    const float *C_in, int64_t ldc, double *C_out, double *bound)
{
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double s = 0.0, t = 0.0;
            for (int64_t k = 0; alpha != 0.0 && k < K; ++k) {
                double a = trans_a ? (double)A[k * lda + i] : (double)A[i * lda + k];
                double b = trans_b ? (double)B[j * ldb + k] : (double)B[k * ldb + j];
                s += a * b;
                t += fabs(a * b);
            }
            double c = alpha != 0.0 ? alpha * s : 0.0, u = fabs(alpha) * t;
            if (beta != 0.0) {
                double cin = beta * (double)C_in[i * ldc + j];
                c += cin;
                u += fabs(cin);
            }
            C_out[i * N + j] = c;
            bound[i * N + j] = u;
        }
}

/* y = W.x with W row-major M x K (W[i*ldw+k]). */
void oracle_gemv(int64_t M, int64_t K, const float *W, int64_t ldw,
                 const float *x, double *y, double *bound)
{
    for (int64_t i = 0; i < M; ++i) {
        double s = 0.0, t = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = (double)W[i * ldw + k] * (double)x[k];
            s += p;
            t += fabs(p);
        }
        y[i] = s;
        bound[i] = t;
    }
}

/* ------------------------------------------------------------- binary16 -- */

/* IEEE 754 binary16 bit pattern to double, from the format's definition:
 * 1 sign bit, 5 exponent bits with bias 15, 10 fraction bits.  Exponent 0
 * holds zero and the subnormals (fraction * 2^-24); exponent 31 holds the
 * infinities (fraction 0) and NaN (fraction != 0). */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + (double)f, e - 25);   /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* --------------------------------------------------------- 2-bit gemv -- */

/* Unpack row i of a 2-bit matrix into fp64 weights w[0..K).
 *   byte  = Q[i*ldq + k/4]
 *   code  = (byte >> 2*(k%4)) & 3
 *   s     = binary16 S[i*lds + k/64]
 *   w[k]  = (code - 1.5) * s                                             */
void oracle_q2_unpack_row(int64_t i, int64_t K, const uint8_t *Q, int64_t ldq,
                          const uint16_t *S, int64_t lds, double *w)
{
    for (int64_t k = 0; k < K; ++k) {
        unsigned byte = Q[i * ldq + k / 4];
        unsigned code = (byte >> (2 * (k % 4))) & 3u;
        double s = oracle_half_to_double(S[i * lds + k / 64]);
        w[k] = ((double)code - 1.5) * s;
    }
}

/* y = W.x for the 2-bit matrix, unpacking each row whole (into the caller's
 * scratch w of K doubles) and then taking the plain dot product. */
void oracle_gemv_q2(int64_t M, int64_t K, const uint8_t *Q, int64_t ldq,
                    const uint16_t *S, int64_t lds, const float *x,
                    double *y, double *bound, double *w)
{
    for (int64_t i = 0; i < M; ++i) {
        oracle_q2_unpack_row(i, K, Q, ldq, S, lds, w);
        double s = 0.0, t = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = w[k] * (double)x[k];
            s += p;
            t += fabs(p);
        }
        y[i] = s;
        bound[i] = t;
    }
}

/* --------------------------------------------------------- 4-bit gemv -- */

/* Unpack row i of a 4-bit matrix into fp64 weights w[0..K).
 *   byte  = Q[i*ldq + k/2]
 *   code  = (byte >> 4*(k%2)) & 15
 *   s     = binary16 S[i*lds + k/64]
 *   w[k]  = (code - 7.5) * s                                             */
void oracle_q4_unpack_row(int64_t i, int64_t K, const uint8_t *Q, int64_t ldq,
                          const uint16_t *S, int64_t lds, double *w)
{
    for (int64_t k = 0; k < K; ++k) {
        unsigned byte = Q[i * ldq + k / 2];
        unsigned code = (byte >> (4 * (k % 2))) & 15u;
        double s = oracle_half_to_double(S[i * lds + k / 64]);
        w[k] = ((double)code - 7.5) * s;
    }
}

/* y = W.x for the 4-bit matrix: unpack each row whole into the caller's
 * scratch w (K doubles), then the plain dot product. */
void oracle_gemv_q4(int64_t M, int64_t K, const uint8_t *Q, int64_t ldq,
                    const uint16_t *S, int64_t lds, const float *x,
                    double *y, double *bound, double *w)
{
    for (int64_t i = 0; i < M; ++i) {
        oracle_q4_unpack_row(i, K, Q, ldq, S, lds, w);
        double s = 0.0, t = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = w[k] * (double)x[k];
            s += p;
            t += fabs(p);
        }
        y[i] = s;
        bound[i] = t;
    }
}
