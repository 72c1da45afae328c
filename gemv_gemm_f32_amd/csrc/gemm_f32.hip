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
//  * Operands are staged global -> registers -> LDS in k-slabs of BK,
//    double-buffered: slab k+1 is fetched from global memory while the
//    MFMAs consume slab k from LDS, with one barrier per slab.
//  * No operand is ever transposed.  Each operand tile is copied into LDS in
//    the orientation it has in global memory, with 16-byte loads and writes:
//      x-major  ([x][k], rows along k): an operand stored M x K or N x K;
//      k-major  ([k][x], rows along x): an operand stored K x M or K x N.
//    The sum over k may be taken in any order, so the MFMA steps walk k in
//    groups of 8 with step t (0..3) of a group taking, in half-wave h, the
//    column k = 8g + 4h + t.  An x-major operand then feeds 4 steps from one
//    ds_read_b128 per lane (4 consecutive k); a k-major operand feeds each
//    step from one ds_read_b32 (row 8g + 4h + t, 32 consecutive x per
//    half-wave).  Row strides (BK + 4 words x-major, 136 words k-major) keep
//    both reads free of LDS bank conflicts.  The next group's operands are
//    read before the current group's MFMAs are issued.
//  * Edges: loads are clamped into the matrix; entries past the K edge are
//    zeroed before they reach LDS, and stores outside C are skipped.  The
//    16-byte load path is a compile-time specialisation taken when pointers,
//    leading dimensions and the contiguous extent are multiples of 4;
//    otherwise the same kernel is instantiated with scalar loads.
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
constexpr int THREADS = 256;
constexpr int GROUP_M = 4;         // tile rows per ordering group
constexpr int KSTRIDE = 136;       // words per LDS row, k-major operand

// LDS words per row of an x-major operand tile.
template <int BK>
constexpr int xstride() { return BK + 4; }

// LDS words of one operand tile (128 x BK) in either orientation.
template <int BK, bool XMAJOR>
constexpr int tile_words() { return XMAJOR ? 128 * xstride<BK>() : BK * KSTRIDE; }

// One operand tile of a k-slab: 128 values of x (m or n) by BK values of k.
//   XMAJOR: element (x, k) at P[x*ld + k]; LDS [x][k], row stride BK + 4.
//   else  : element (x, k) at P[k*ld + x]; LDS [k][x], row stride KSTRIDE.
// Each thread moves NL groups of 4 consecutive elements per slab.
//
// Loads are unconditional, from indices clamped into the matrix, so they
// issue back to back without branches.  A value fetched for an index x past
// the matrix edge only ever meets rows or columns of C that are not stored;
// values for k past K would enter real sums and are zeroed in store(), which
// runs after the MFMAs of the current slab.
template <int BK, bool XMAJOR, int VEC>
struct Operand {
    static constexpr int NL = BK / 8;
    v4f r[NL];

    __device__ __forceinline__ void load(const float *__restrict__ P, int64_t ld, int x0,
                                         int k0, int X, int K, int tid) {
#pragma unroll
        for (int p = 0; p < NL; ++p) {
            const int idx = tid + THREADS * p;
            if (XMAJOR) {
                const int x = min(x0 + idx / (BK / 4), X - 1);
                const int k = k0 + (idx % (BK / 4)) * 4;
                const float *row = P + (int64_t)x * ld;
                if (VEC == 4) {
                    r[p] = *reinterpret_cast<const v4f *>(row + min(k, K - 4));
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c) r[p][c] = row[min(k + c, K - 1)];
                }
            } else {
                const int k = min(k0 + idx / 32, K - 1);
                const int x = x0 + (idx % 32) * 4;
                const float *row = P + (int64_t)k * ld;
                if (VEC == 4) {
                    r[p] = *reinterpret_cast<const v4f *>(row + min(x, X - 4));
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c) r[p][c] = row[min(x + c, X - 1)];
                }
            }
        }
    }

    __device__ __forceinline__ void store(float *lds, int tid, int k0, int K) const {
        const bool tail = k0 + BK > K;     // uniform: only the last slab
#pragma unroll
        for (int p = 0; p < NL; ++p) {
            const int idx = tid + THREADS * p;
            v4f v = r[p];
            if (XMAJOR) {
                const int x = idx / (BK / 4), k = (idx % (BK / 4)) * 4;
                if (tail) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) v[c] = k0 + k + c < K ? v[c] : 0.f;
                }
                *reinterpret_cast<v4f *>(lds + x * xstride<BK>() + k) = v;
            } else {
                const int k = idx / 32, x = (idx % 32) * 4;
                if (tail && k0 + k >= K) v = v4f{0.f, 0.f, 0.f, 0.f};
                *reinterpret_cast<v4f *>(lds + k * KSTRIDE + x) = v;
            }
        }
    }

    // The 4 MFMA-step operands of k-group g for the 32-row block starting at
    // x = xb (lane: x = xb + l32, half-wave h).
    __device__ __forceinline__ static v4f frag(const float *lds, int g, int xb, int l32, int h) {
        if (XMAJOR) {
            return *reinterpret_cast<const v4f *>(lds + (xb + l32) * xstride<BK>() + 8 * g + 4 * h);
        } else {
            const float *p = lds + (8 * g + 4 * h) * KSTRIDE + xb + l32;
            return v4f{p[0], p[KSTRIDE], p[2 * KSTRIDE], p[3 * KSTRIDE]};
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

// AX: A is stored M x K (x-major tiles); otherwise K x M.
// BX: B is stored N x K (x-major tiles); otherwise K x N.
template <int BK, bool AX, bool BX, int VA, int VB>
__global__ __launch_bounds__(THREADS) void gemm_f32_kernel(
    int M, int N, int K, const float *__restrict__ A, int64_t lda,
    const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n) {
    static_assert(BK % 8 == 0, "k walks in groups of 8");
    constexpr int AW = tile_words<BK, AX>(), BW = tile_words<BK, BX>();
    __shared__ __attribute__((aligned(16))) float As[2][AW];
    __shared__ __attribute__((aligned(16))) float Bs[2][BW];
    using OpA = Operand<BK, AX, VA>;
    using OpB = Operand<BK, BX, VB>;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;   // wave quarter
    const int h = lane >> 5;
    const int l32 = lane & 31;

    OpA la;
    OpB lb;

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
        la.store(As[0], tid, 0, K);
        lb.store(Bs[0], tid, 0, K);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            la.load(A, lda, m0, (kt + 1) * BK, M, K, tid);
            lb.load(B, ldb, n0, (kt + 1) * BK, N, K, tid);
        }
        const float *as = As[buf];
        const float *bs = Bs[buf];
        v4f fa0 = OpA::frag(as, 0, wm, l32, h), fa1 = OpA::frag(as, 0, wm + 32, l32, h);
        v4f fb0 = OpB::frag(bs, 0, wn, l32, h), fb1 = OpB::frag(bs, 0, wn + 32, l32, h);
#pragma unroll
        for (int g = 0; g < BK / 8; ++g) {
            v4f na0 = fa0, na1 = fa1, nb0 = fb0, nb1 = fb1;
            if (g + 1 < BK / 8) {
                na0 = OpA::frag(as, g + 1, wm, l32, h);
                na1 = OpA::frag(as, g + 1, wm + 32, l32, h);
                nb0 = OpB::frag(bs, g + 1, wn, l32, h);
                nb1 = OpB::frag(bs, g + 1, wn + 32, l32, h);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa0[t], fb0[t], acc[0][0], 0, 0, 0);
                acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa0[t], fb1[t], acc[0][1], 0, 0, 0);
                acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa1[t], fb0[t], acc[1][0], 0, 0, 0);
                acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa1[t], fb1[t], acc[1][1], 0, 0, 0);
            }
            fa0 = na0; fa1 = na1; fb0 = nb0; fb1 = nb1;
        }
        if (more) {
            la.store(As[buf ^ 1], tid, (kt + 1) * BK, K);
            lb.store(Bs[buf ^ 1], tid, (kt + 1) * BK, K);
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

constexpr int PROD_BK = 32;

template <bool AX, bool BX, int VA, int VB, int BK = PROD_BK>
hipError_t launch_t(int M, int N, int K, const float *A, int64_t lda, const float *B,
                    int64_t ldb, float *C, int64_t ldc, hipStream_t s) {
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int nwg = tiles_m * tiles_n;
    hipLaunchKernelGGL((gemm_f32_kernel<BK, AX, BX, VA, VB>), dim3(nwg), dim3(THREADS), 0, s,
                       M, N, K, A, lda, B, ldb, C, ldc, tiles_m, tiles_n);
    return hipGetLastError();
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_gemm(GemmLayout layout, int M, int N, int K, const float *A, int64_t lda,
                       const float *B, int64_t ldb, float *C, int64_t ldc, hipStream_t s) {
    // 16-byte loads need the operand's contiguous extent, its leading
    // dimension and its base all to be multiples of 4 floats.
    const bool ax = layout != GemmLayout::TN;     // A stored M x K
    const bool bx = layout == GemmLayout::NT;     // B stored N x K
    const int a_contig = ax ? K : M;
    const int b_contig = bx ? K : N;
    const bool va = aligned16(A) && (lda % 4 == 0) && (a_contig % 4 == 0);
    const bool vb = aligned16(B) && (ldb % 4 == 0) && (b_contig % 4 == 0);
#define GG_GEMM_CASE(AX_, BX_)                                                          \
    if (va && vb) return launch_t<AX_, BX_, 4, 4>(M, N, K, A, lda, B, ldb, C, ldc, s); \
    if (va) return launch_t<AX_, BX_, 4, 1>(M, N, K, A, lda, B, ldb, C, ldc, s);       \
    if (vb) return launch_t<AX_, BX_, 1, 4>(M, N, K, A, lda, B, ldb, C, ldc, s);       \
    return launch_t<AX_, BX_, 1, 1>(M, N, K, A, lda, B, ldb, C, ldc, s);
    switch (layout) {
        case GemmLayout::NN: { GG_GEMM_CASE(true, false) }
        case GemmLayout::TN: { GG_GEMM_CASE(false, false) }
        case GemmLayout::NT: { GG_GEMM_CASE(true, true) }
    }
#undef GG_GEMM_CASE
    return hipErrorInvalidValue;
}

}  // namespace gg
