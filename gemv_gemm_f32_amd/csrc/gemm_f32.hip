// gemm_f32.hip -- fp32 C = op(A).op(B) on gfx950 matrix cores.
//
// The operation is the dense-layer product of "More Stumbling, This Time in
// the Browser" (section "Four answers per worker") and the matmul of "I built
// a GPT-2 in the browser, then made it 2.6x-12.1x faster" (sections "The
// kernel sweep", "Step 1" and "Step 2"), including its backward transposes
// (section "The architecture in 60 seconds").  Those pages tile for WebGPU
// (16 x 16 workgroup tiles, 4 x 4 register blocks); here the tile is shaped
// for CDNA4 instead:
//
//  * One workgroup of 256 lanes (4 wave64s) owns a 128 x 128 tile of C.  Each
//    wave owns a 64 x 64 quarter as 2 x 2 blocks of v_mfma_f32_32x32x2_f32,
//    whose 64 fp32 accumulators per lane stay in registers for the whole K
//    walk.  The matrix core takes IEEE fp32 operands (no reduced-precision
//    inputs) and accumulates in fp32.
//  * Operands are staged global -> registers -> LDS in k-slabs of BK = 16,
//    double-buffered: slab k+1 is fetched from global memory while the
//    MFMAs consume slab k from LDS, with one barrier per slab.
//  * LDS holds both operands k-major (one row per k, the M or N index
//    contiguous, rows padded to 160 floats).  An MFMA step reads, per lane,
//    one A value and one B value with ds_read_b32: half-wave h reads row
//    k0 + h, 32 consecutive words, which is conflict-free.  So the three
//    layouts differ only in how a slab is copied in: an operand whose global
//    rows run along M or N is copied row for row with 16-byte writes; one
//    whose global rows run along K is transposed on the way in.
//  * Edges: loads outside the matrix write zeros into LDS (this also pads the
//    K tail), and stores outside C are skipped.  The 16-byte load path is a
//    compile-time specialisation taken when pointers, leading dimensions and
//    the contiguous extent are multiples of 4; otherwise the same kernel is
//    instantiated with scalar loads.
//  * Tile order: workgroups are handed to the 8 XCDs round-robin, so the grid
//    index is remapped to give each XCD a contiguous run of tiles, ordered in
//    groups of 4 tile rows so that a run shares A row panels and B column
//    panels in that XCD's L2.
//  * Every output cell is one fixed sequence of MFMA accumulations over k,
//    independent of timing, so results are reproducible bit for bit.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace gg {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 128;            // tile rows (M)
constexpr int BN = 128;            // tile columns (N)
constexpr int BK = 16;             // k-slab depth
constexpr int LDS_STRIDE = 160;    // floats per LDS row (128 + 32 pad)
constexpr int THREADS = 256;
constexpr int GROUP_M = 4;         // tile rows per ordering group

// One operand slab: BK rows (k) of 128 contiguous floats (m or n) in LDS.
// Global layout per operand:
//   KMAJOR = true : element (k, x) at P[k*ld + x]   (rows along x = m or n)
//   KMAJOR = false: element (k, x) at P[x*ld + k]   (rows along k)
// Each thread moves 8 elements per slab, as two groups of 4.
template <bool KMAJOR, int VEC>
struct SlabLoader {
    v4f r[2];

    __device__ __forceinline__ void load(const float *__restrict__ P, int64_t ld,
                                         int x0, int k0, int X, int K, int tid) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int idx = tid + THREADS * p;
            if (KMAJOR) {
                // 16 rows of k x 32 groups of 4 consecutive x
                const int k = k0 + idx / 32;
                const int x = x0 + (idx % 32) * 4;
                if (VEC == 4) {
                    v4f v = {0.f, 0.f, 0.f, 0.f};
                    if (k < K && x < X)
                        v = *reinterpret_cast<const v4f *>(P + (int64_t)k * ld + x);
                    r[p] = v;
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        r[p][c] = (k < K && x + c < X) ? P[(int64_t)k * ld + x + c] : 0.f;
                }
            } else {
                // 4 groups of 4 consecutive k x 128 values of x; a wave covers
                // 64 consecutive x so the transposed LDS writes are conflict-free
                const int x = x0 + idx % 128;
                const int k = k0 + (idx / 128) * 4;
                if (VEC == 4) {
                    v4f v = {0.f, 0.f, 0.f, 0.f};
                    if (x < X && k < K)
                        v = *reinterpret_cast<const v4f *>(P + (int64_t)x * ld + k);
                    r[p] = v;
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        r[p][c] = (x < X && k + c < K) ? P[(int64_t)x * ld + k + c] : 0.f;
                }
            }
        }
    }

    __device__ __forceinline__ void store(float *lds, int tid) const {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int idx = tid + THREADS * p;
            if (KMAJOR) {
                const int k = idx / 32, x = (idx % 32) * 4;
                *reinterpret_cast<v4f *>(lds + k * LDS_STRIDE + x) = r[p];
            } else {
                const int x = idx % 128, k = (idx / 128) * 4;
#pragma unroll
                for (int c = 0; c < 4; ++c) lds[(k + c) * LDS_STRIDE + x] = r[p][c];
            }
        }
    }
};

// Grid index -> (tile row, tile column).
__device__ __forceinline__ void tile_of(int bid, int nwg, int tiles_m, int tiles_n,
                                        int &tm, int &tn) {
    int t = bid;
    if ((nwg & 7) == 0) t = (bid & 7) * (nwg >> 3) + (bid >> 3);   // XCD runs
    const int per_group = GROUP_M * tiles_n;
    const int group = t / per_group;
    const int first_m = group * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int in_group = t - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// TA: A stored K x M (A^T.B).  TB: B stored N x K (A.B^T).
template <bool TA, bool TB, int VA, int VB>
__global__ __launch_bounds__(THREADS) void gemm_f32_kernel(
    int M, int N, int K, const float *__restrict__ A, int64_t lda,
    const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(16))) float As[2][BK * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * LDS_STRIDE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;   // wave quarter
    const int h = lane >> 5;          // k row within an MFMA step
    const int l32 = lane & 31;

    // A is k-major in global memory when stored K x M; B when stored K x N.
    SlabLoader<TA, VA> la;
    SlabLoader<!TB, VB> lb;

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        la.load(A, lda, m0, 0, M, K, tid);
        lb.load(B, ldb, n0, 0, N, K, tid);
        la.store(As[0], tid);
        lb.store(Bs[0], tid);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            la.load(A, lda, m0, (kt + 1) * BK, M, K, tid);
            lb.load(B, ldb, n0, (kt + 1) * BK, N, K, tid);
        }
        const float *as = As[buf] + h * LDS_STRIDE + wm + l32;
        const float *bs = Bs[buf] + h * LDS_STRIDE + wn + l32;
#pragma unroll
        for (int kk = 0; kk < BK; kk += 2) {
            const float a0 = as[kk * LDS_STRIDE];
            const float a1 = as[kk * LDS_STRIDE + 32];
            const float b0 = bs[kk * LDS_STRIDE];
            const float b1 = bs[kk * LDS_STRIDE + 32];
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
        }
        if (more) {
            la.store(As[buf ^ 1], tid);
            lb.store(Bs[buf ^ 1], tid);
        }
        __syncthreads();
    }

    // Accumulator layout of a 32 x 32 block: register r of lane l holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn + 32 * j + l32;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < M) C[(int64_t)row * ldc + col] = acc[i][j][r];
            }
        }
}

template <bool TA, bool TB, int VA, int VB>
hipError_t launch_t(int M, int N, int K, const float *A, int64_t lda, const float *B,
                    int64_t ldb, float *C, int64_t ldc, hipStream_t s) {
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int nwg = tiles_m * tiles_n;
    hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, VA, VB>), dim3(nwg), dim3(THREADS), 0, s,
                       M, N, K, A, lda, B, ldb, C, ldc, tiles_m, tiles_n);
    return hipGetLastError();
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_gemm(GemmLayout layout, int M, int N, int K, const float *A, int64_t lda,
                       const float *B, int64_t ldb, float *C, int64_t ldc, hipStream_t s) {
    // 16-byte loads need the operand's contiguous extent, its leading
    // dimension and its base all to be multiples of 4 floats.
    const bool ta = layout == GemmLayout::TN, tb = layout == GemmLayout::NT;
    const int a_contig = ta ? M : K;
    const int b_contig = tb ? K : N;
    const bool va = aligned16(A) && (lda % 4 == 0) && (a_contig % 4 == 0);
    const bool vb = aligned16(B) && (ldb % 4 == 0) && (b_contig % 4 == 0);
#define GG_GEMM_CASE(TA_, TB_)                                                          \
    if (va && vb) return launch_t<TA_, TB_, 4, 4>(M, N, K, A, lda, B, ldb, C, ldc, s); \
    if (va) return launch_t<TA_, TB_, 4, 1>(M, N, K, A, lda, B, ldb, C, ldc, s);       \
    if (vb) return launch_t<TA_, TB_, 1, 4>(M, N, K, A, lda, B, ldb, C, ldc, s);       \
    return launch_t<TA_, TB_, 1, 1>(M, N, K, A, lda, B, ldb, C, ldc, s);
    switch (layout) {
        case GemmLayout::NN: { GG_GEMM_CASE(false, false) }
        case GemmLayout::TN: { GG_GEMM_CASE(true, false) }
        case GemmLayout::NT: { GG_GEMM_CASE(false, true) }
    }
#undef GG_GEMM_CASE
    return hipErrorInvalidValue;
}

}  // namespace gg
