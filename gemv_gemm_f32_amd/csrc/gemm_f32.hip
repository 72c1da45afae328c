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
//  * A group of 4 wave64s owns a BM x BN tile of C (64 x 64 on the direct path;
//    128 x 64 or 64 x 64 on the staged path, picked per call from the grid
//    size).  Each wave owns a quarter as 32 x 32 blocks of
//    v_mfma_f32_32x32x2_f32, whose fp32 accumulators stay in registers for
//    the whole K walk.
//  * Split K inside the workgroup (direct path): a workgroup holds KS = 1, 2
//    or 4 such groups on one tile, group g taking k-slabs g, g + KS, ...
//    through its own LDS stages; groups 1 .. KS-1 then hand their sums to
//    group 0 through LDS, which adds them in group order.  Products with few
//    output tiles (the K-heavy backward products, small squares) get 8 or 16
//    waves per tile instead of 4, without a workspace or atomics.  The matrix core
//    takes IEEE fp32 operands (no reduced-precision inputs) and accumulates
//    in fp32.
//  * Operand tiles are staged in LDS in k-slabs of BK = 32, double-buffered:
//    slab k+1 is fetched while the MFMAs consume slab k, with one barrier per
//    slab.  The sum over k may be taken in any order, so the MFMA steps walk k
//    in groups of 8 with step t (0..3) of a group taking, in half-wave h, the
//    column k = 8g + 4h + t.  An x-major operand ([x][k], stored M x K or
//    N x K) then feeds 4 steps from one ds_read_b128 per lane (4 consecutive
//    k); a k-major operand ([k][x], stored K x M or K x N) feeds each step
//    from one ds_read_b32 (row 8g + 4h + t, 32 consecutive x per half-wave).
//    No operand is ever transposed.  The next group's operands are read
//    before the current group's MFMAs are issued.
//  * Direct path (16-byte aligned operands whose byte extent fits 32-bit
//    offsets): slabs move global -> LDS with buffer_load_dwordx4 ... lds, so
//    the data never passes through registers and advancing a slab costs one
//    scalar offset.  Each such instruction writes 1 KB of LDS in lane order;
//    which global 16-byte chunk a lane fetches is chosen so that the chunks
//    land XOR-swizzled (x-major rows: chunk c of row r at slot
//    c ^ ((r ^ r/8) mod 8); k-major rows: c ^ 8 on every other group of 4
//    rows), which keeps the fragment reads free of bank conflicts without
//    padding.  Reads past the end of an operand return zero (range-checked
//    buffer), and k past K is zeroed by the lane that fetched it once its
//    load has landed, before the barrier that publishes the slab.
//  * Staged path (any other operand): slabs move global -> registers -> LDS
//    with loads clamped into the matrix, into padded rows (BK + 4 words
//    x-major, tile width + 8 k-major) that are free of bank conflicts; k past
//    K is zeroed on the way in.  16-byte loads are a compile-time
//    specialisation taken when pointers, leading dimensions and the
//    contiguous extent are multiples of 4 floats; otherwise scalar loads.
//  * Edges: rows and columns past M or N are fetched clamped into the matrix
//    and their results are never stored.
//  * Epilogue: C = alpha * acc, plus beta * C when beta != 0 (C is not read
//    otherwise).  With alpha = 1 and beta = 0 the stored value is the
//    accumulator itself.
//  * Tile order: workgroups are handed to the 8 XCDs round-robin, so the grid
//    index is remapped to give each XCD a contiguous run of tiles, ordered in
//    groups of 8 tile rows so that a run shares A row panels and B column
//    panels in that XCD's L2.
//  * Every output cell is one fixed sequence of MFMA accumulations over k,
//    independent of timing and of the path taken, so results are
//    reproducible bit for bit.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kernels.hpp"

namespace gg {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int THREADS = 256;
constexpr int GROUP_M = 8;         // tile rows per ordering group

// ---------------------------------------------------------------------------
// Staged path.

// LDS words per row of an operand tile of TX values of x by BK values of k:
// x-major rows hold BK words plus 4 of padding (16 consecutive rows then
// cover all banks for a 16-byte read); k-major rows hold TX plus 8 (so rows
// 4 apart, read by the two half-waves, fall 32 banks apart).
template <int BK>
constexpr int xstride() { return BK + 4; }
template <int TX>
constexpr int kstride() { return TX + 8; }

template <int TX, int BK, bool XMAJOR>
constexpr int tile_words() { return XMAJOR ? TX * xstride<BK>() : BK * kstride<TX>(); }

// One operand tile of a k-slab: TX values of x (m or n) by BK values of k.
//   XMAJOR: element (x, k) at P[x*ld + k]; LDS [x][k].
//   else  : element (x, k) at P[k*ld + x]; LDS [k][x].
// Each thread moves NL groups of 4 consecutive elements per slab.
//
// Loads are unconditional, from indices clamped into the matrix, so they
// issue back to back without branches.  A value fetched for an index x past
// the matrix edge only ever meets rows or columns of C that are not stored;
// values for k past K would enter real sums and are zeroed in store(), which
// runs after the MFMAs of the current slab.
template <int TX, int BK, bool XMAJOR, int VEC>
struct Operand {
    static constexpr int NL = TX * BK / 4 / THREADS;
    static constexpr int KS = kstride<TX>();
    static_assert(NL >= 1 && NL * 4 * THREADS == TX * BK, "tile must split evenly");
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
                const int k = min(k0 + idx / (TX / 4), K - 1);
                const int x = x0 + (idx % (TX / 4)) * 4;
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
                const int k = idx / (TX / 4), x = (idx % (TX / 4)) * 4;
                if (tail && k0 + k >= K) v = v4f{0.f, 0.f, 0.f, 0.f};
                *reinterpret_cast<v4f *>(lds + k * KS + x) = v;
            }
        }
    }

    // The 4 MFMA-step operands of k-group g for the 32-row block starting at
    // x = xb (lane: x = xb + l32, half-wave h).
    __device__ __forceinline__ static v4f frag(const float *lds, int g, int xb, int l32, int h) {
        if (XMAJOR) {
            return *reinterpret_cast<const v4f *>(lds + (xb + l32) * xstride<BK>() + 8 * g + 4 * h);
        } else {
            const float *p = lds + (8 * g + 4 * h) * KS + xb + l32;
            return v4f{p[0], p[KS], p[2 * KS], p[3 * KS]};
        }
    }
};

// One output cell: alpha * acc, plus beta * C when beta != 0.
__device__ __forceinline__ void store_c(float *c, float acc, float alpha, float beta) {
    float v = alpha * acc;
    if (beta != 0.f) v = __builtin_fmaf(beta, *c, v);
    *c = v;
}

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
// BM x BN tile per workgroup; 2 x 2 waves of (BM/2) x (BN/2), each as
// (BM/64) x (BN/64) blocks of 32 x 32.
template <int BM, int BN, int BK, bool AX, bool BX, int VA, int VB, bool FENCE = true>
__global__ __launch_bounds__(THREADS) void gemm_f32_kernel(
    int M, int N, int K, float alpha, const float *__restrict__ A, int64_t lda,
    const float *__restrict__ B, int64_t ldb, float beta, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n) {
    static_assert(BK % 8 == 0, "k walks in groups of 8");
    constexpr int WM = BM / 2, WN = BN / 2;        // wave tile
    constexpr int IB = WM / 32, JB = WN / 32;      // 32 x 32 blocks per wave
    constexpr int AW = tile_words<BM, BK, AX>(), BW = tile_words<BN, BK, BX>();
    __shared__ __attribute__((aligned(16))) float As[2][AW];
    __shared__ __attribute__((aligned(16))) float Bs[2][BW];
    using OpA = Operand<BM, BK, AX, VA>;
    using OpB = Operand<BN, BK, BX, VB>;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;   // wave quarter
    const int h = lane >> 5;
    const int l32 = lane & 31;

    OpA la;
    OpB lb;

    v16f acc[IB][JB];
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
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
        v4f fa[IB], fb[JB];
#pragma unroll
        for (int i = 0; i < IB; ++i) fa[i] = OpA::frag(as, 0, wm + 32 * i, l32, h);
#pragma unroll
        for (int j = 0; j < JB; ++j) fb[j] = OpB::frag(bs, 0, wn + 32 * j, l32, h);
#pragma unroll
        for (int g = 0; g < BK / 8; ++g) {
            v4f na[IB], nb[JB];
#pragma unroll
            for (int i = 0; i < IB; ++i)
                na[i] = g + 1 < BK / 8 ? OpA::frag(as, g + 1, wm + 32 * i, l32, h) : fa[i];
#pragma unroll
            for (int j = 0; j < JB; ++j)
                nb[j] = g + 1 < BK / 8 ? OpB::frag(bs, g + 1, wn + 32 * j, l32, h) : fb[j];
            // Keep the next group's LDS reads ahead of this group's MFMAs:
            // left alone, the scheduler sinks each read to just before its
            // use and the MFMA pipe waits on LDS latency.
            if (FENCE) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < IB; ++i)
#pragma unroll
                    for (int j = 0; j < JB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][t], fb[j][t],
                                                                        acc[i][j], 0, 0, 0);
            if (FENCE) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < IB; ++i) fa[i] = na[i];
#pragma unroll
            for (int j = 0; j < JB; ++j) fb[j] = nb[j];
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
    for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            const int col = n0 + wn + 32 * j + l32;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < M) store_c(C + (int64_t)row * ldc + col, acc[i][j][r], alpha, beta);
            }
        }
}

// ---------------------------------------------------------------------------
// Direct path.

typedef __attribute__((address_space(3))) void lds_void;

// chunk slot of x-major row r (8 chunks of 16 B per row of BK = 32 floats)
__device__ __forceinline__ int xswz(int r) { return (r ^ (r >> 3)) & 7; }

// One operand's k-slab (TX values of x by 32 of k) as NBLK buffer loads of
// 1 KB, spread over the WPG waves of a group: instruction j of wave w fills
// block WPG*j + w of the stage (when the blocks do not split evenly, the
// last round of instructions is issued by the first waves only).
//   XMAJOR: element (x, k) at P[x*ld + k]; the stage holds TX rows of 128 B.
//   else  : element (x, k) at P[k*ld + x]; the stage holds 32 rows of TX*4 B.
// KT: K is not a multiple of 4, so an x-major chunk can straddle K.
// MF: the MFMA block the fragments feed, 32 (32 x 32 x 2) or 16 (16 x 16 x 4).
template <int TX, bool XMAJOR, int WPG = 4, bool KT = false, int MF = 32>
struct DirectOperand {
    static constexpr int BK = 32;
    static constexpr int STAGE = TX * BK * 4;     // bytes per stage
    static constexpr int NBLK = STAGE / 1024;     // 1 KB load instructions per slab
    static constexpr int NI = (NBLK + WPG - 1) / WPG;   // per wave, at most
    static_assert(NBLK >= WPG && NBLK * 1024 == STAGE, "tile must split over the waves");
    // k-major rows of CPR 16-byte chunks are rotated so that the lane groups
    // of a fragment read, which read rows 4 apart, use different banks: by 8
    // chunks (128 bytes) on every other group of four rows for 32 x 32
    // blocks (two half-waves), and by 4 chunks (64 bytes) per group of four
    // rows, cycling over four groups, for 16 x 16 blocks (four quarter-waves).
    // Rows of 32 floats have no second half and take 2-way conflicts instead.
    static constexpr int CPR = TX / 4;
    static_assert(XMAJOR || CPR % (MF == 32 ? 8 : 16) == 0,
                  "k-major tiles are a multiple of 32 (64 for 16 x 16 blocks) wide");
    static __device__ __forceinline__ int krot(int row) {
        return MF == 32 ? 8 * ((row >> 2) & 1) : 4 * ((row >> 2) & 3);
    }
    static __device__ __forceinline__ int kslot(int c, int row) { return (c + krot(row)) % CPR; }
    // whether this wave issues instruction j
    static __device__ __forceinline__ bool has(int j, int wave) {
        if constexpr (NBLK % WPG == 0) return true;
        return WPG * j + wave < NBLK;
    }
    unsigned voff[NI];   // byte offset of this lane's chunk at k = 0
    int kof[NI];         // k of this lane's chunk (x-major) or row (k-major) in the slab

    __device__ __forceinline__ void init(int64_t ld, int x0, int X, int lane, int wave) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int blk = has(j, wave) ? WPG * j + wave : 0;
            if (XMAJOR) {
                const int row = 8 * blk + lane / 8;
                const int c = (lane % 8) ^ xswz(row);
                voff[j] = (unsigned)(((int64_t)min(x0 + row, X - 1) * ld + 4 * c) * 4);
                kof[j] = 4 * c;
            } else {
                // the lane writes LDS chunk q of the stage (row q / CPR, slot
                // q % CPR), so it fetches the chunk of that row whose slot it is
                const int q = 64 * blk + lane;
                const int row = q / CPR;
                const int c = (q % CPR + CPR - krot(row) % CPR) % CPR;
                // chunks past the row's last one load that one (their columns
                // are never stored); the last one may run past X into the next
                // row, or past the operand's end, which reads zeros
                voff[j] = (unsigned)(((int64_t)row * ld + min(x0 + 4 * c, (X - 1) & ~3)) * 4);
                kof[j] = row;
            }
        }
    }
    // bytes from P to the end of the operand's last element
    static __device__ __forceinline__ int extent(int64_t ld, int X, int K) {
        return (int)(XMAJOR ? ((int64_t)(X - 1) * ld + K) * 4 : ((int64_t)(K - 1) * ld + X) * 4);
    }
    __device__ __forceinline__ void issue(char *stage, const float *P, int ext, int64_t ld, int k0,
                                          int wave) const {
        // The buffer builtins exist only in the device compilation.
#if defined(__HIP_DEVICE_COMPILE__)
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void *)P, (short)0, ext, 0x00020000);
        const unsigned so = (unsigned)((XMAJOR ? (int64_t)k0 : k0 * ld) * 4);
#pragma unroll
        for (int j = 0; j < NI; ++j)
            if (has(j, wave))
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc, (lds_void *)(stage + (WPG * j + wave) * 1024), 16, voff[j], so, 0, 0);
#endif
    }
    // after this wave's loads of the slab at k0 have landed: zero what lies at
    // k >= K (whole chunks, and in x-major rows the part of a chunk past K
    // when K is not a multiple of 4)
    __device__ __forceinline__ void zero_tail(char *stage, int k0, int K, int wave, int lane) const {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            if (!has(j, wave)) continue;
            float *p = reinterpret_cast<float *>(stage + (WPG * j + wave) * 1024 + lane * 16);
            const int k = k0 + kof[j];
            if (k >= K) {
                *reinterpret_cast<v4f *>(p) = v4f{0.f, 0.f, 0.f, 0.f};
            } else if (XMAJOR && KT && k + 4 > K) {
                for (int e = K - k; e < 4; ++e) p[e] = 0.f;
            }
        }
    }
    // byte offset, within a stage, of a lane's operand of k-group g for the
    // MF-block at x = xb.  32 x 32 x 2: half-wave h = lane / 32 takes x =
    // xb + lane % 32 at k = 8g + 4h + t in step t.  16 x 16 x 4: quarter-wave
    // q = lane / 16 takes x = xb + lane % 16 at k = 16g + 4q + t.  Either
    // way an x-major lane reads the 4 k of its step from one 16-byte chunk.
    static __device__ __forceinline__ int frag_offset(int xb, int lane, int g) {
        const int x = xb + (lane & (MF - 1));
        const int part = lane / MF;               // h or q
        const int krow = (64 / MF) * 4 * g + 4 * part;
        if (XMAJOR) return x * 128 + ((((64 / MF) * g + part) ^ xswz(x)) * 16);
        return krow * TX * 4 + kslot(x >> 2, 4 * part) * 16 + (x & 3) * 4;
    }
    static __device__ __forceinline__ v4f frag(const char *stage, int off) {
        if (XMAJOR) return *reinterpret_cast<const v4f *>(stage + off);
        const float *p = reinterpret_cast<const float *>(stage + off);
        return v4f{p[0], p[TX], p[2 * TX], p[3 * TX]};
    }
};

// KS groups of WPG waves split the k-slabs of one output tile: group g takes
// slabs g, g + KS, g + 2 KS, ... through its own double-buffered stages.  At
// the end groups 1 .. KS-1 hand their accumulators to group 0 through LDS,
// which adds them in group order, so the sum is fixed for a given KS.  With
// 32 x 32 MFMA blocks (MF = 32) the WPG waves of a group lay out as 2 x 2
// (WPG = 4), 1 x 2 or 2 x 1 (WPG = 2, along the longer side of the tile) or
// 1 x 1 over the tile; with 16 x 16 blocks (MF = 16) they stack along M,
// each wave holding a row of BN / 16 blocks (64 x 48 tiles: 16 x 48 per
// wave, three independent accumulators).
template <int BM, int BN, bool AX, bool BX, int KS, int WPG = 4, bool KT = false, int MF = 32>
__global__ __launch_bounds__(64 * WPG * KS) void gemm_f32_direct(
    int M, int N, int K, float alpha, const float *__restrict__ A, int64_t lda,
    const float *__restrict__ B, int64_t ldb, float beta, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n) {
    constexpr int BK = 32;
    constexpr int WC = MF == 16 ? 1 : (WPG == 4 ? 2 : (WPG == 2 && BN >= BM ? 2 : 1));   // wave columns
    constexpr int WR = WPG / WC;                  // wave rows
    constexpr int WM = BM / WR, WN = BN / WC;
    constexpr int IB = WM / MF, JB = WN / MF;
    static_assert(IB * MF == WM && JB * MF == WN && WR * WC == WPG, "tile must split into MF-blocks");
    // 16 x 16 blocks: a k-major B tile 48 wide is staged 64 wide (the next
    // 16 columns ride along unused) so that its rows keep the conflict-free
    // rotation of 64-float rows
    constexpr int TB = (MF == 16 && !BX && BN == 48) ? 64 : BN;
    using OA = DirectOperand<BM, AX, WPG, KT, MF>;
    using OB = DirectOperand<TB, BX, WPG, KT, MF>;
    using Acc = typename std::conditional<MF == 32, v16f, v4f>::type;
    constexpr int AR = MF == 32 ? 16 : 4;         // accumulator words per block
    constexpr int NG = MF == 32 ? 4 : 2;          // k-groups of 4 steps per slab
    // Narrow and 32 x 32 tiles (one or two waves per k-group), and 64 x 64
    // tiles in four k-groups, issue the next slab's loads after the first
    // k-group's MFMAs rather than before them: 1024 x 2304 x 768 40.3 -> 36.5
    // us, 768 x 3072 x 1024 50.6 -> 46.9, 500 x 500 x 2000 14.8 -> 13.5,
    // 1024 x 1024 x 4096 69.6 -> 65.9.  64 x 64 tiles in two k-groups (two
    // workgroups per CU) and the 64 x 48 tiles keep the early issue: late,
    // 2048^3 took 129.2 us against 127.5 and 1024 x 768 x 3072 46.3 against
    // 44.8.
    constexpr bool LATE = WPG <= 2 || (KS == 4 && MF == 32);
    constexpr int STAGE = OA::STAGE + OB::STAGE;
    constexpr int ACCW = IB * JB * AR;            // accumulator words per lane
    static_assert(KS == 1 || (KS - 1) * 64 * WPG * ACCW * 4 <= KS * 2 * STAGE,
                  "the hand-over of partial sums must fit in the stages");
    __shared__ __attribute__((aligned(1024))) char smem[KS * 2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave / WPG, wq = wave % WPG;  // k-group, wave within the group
    const int h = lane >> 5;
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int wm = (wq / WC) * WM, wn = (wq % WC) * WN;

    OA oa;
    OB ob;
    oa.init(lda, m0, M, lane, wq);
    ob.init(ldb, n0, N, lane, wq);
    const int exta = OA::extent(lda, M, K), extb = OB::extent(ldb, N, K);
    char *const gsmem = smem + grp * 2 * STAGE;
    auto stage_a = [&](int b) { return gsmem + b * STAGE; };
    auto stage_b = [&](int b) { return gsmem + b * STAGE + OA::STAGE; };
    int aoff[IB][NG], boff[JB][NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
        for (int i = 0; i < IB; ++i) aoff[i][g] = OA::frag_offset(wm + MF * i, lane, g);
#pragma unroll
        for (int j = 0; j < JB; ++j) boff[j][g] = OB::frag_offset(wn + MF * j, lane, g);
    }

    Acc acc[IB][JB];
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
            for (int r = 0; r < AR; ++r) acc[i][j][r] = 0.f;

    const int nk = (K + BK - 1) / BK;
    const int rounds = (nk + KS - 1) / KS;        // the same for every group
    if (rounds > 0) {
        if (grp < nk) {
            oa.issue(stage_a(0), A, exta, lda, grp * BK, wq);
            ob.issue(stage_b(0), B, extb, ldb, grp * BK, wq);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            if (grp * BK + BK > K) {
                oa.zero_tail(stage_a(0), grp * BK, K, wq, lane);
                ob.zero_tail(stage_b(0), grp * BK, K, wq, lane);
            }
        }
        __syncthreads();
    }
    for (int r = 0; r < rounds; ++r) {
        const int buf = r & 1;
        const int kt = r * KS + grp;              // this group's slab in round r
        const int kn = kt + KS;                   // and in round r + 1
        const int k1 = kn * BK;
        const bool more = r + 1 < rounds;
        // slab kn goes to the stage last read in round r-1, whose reads all
        // finished before the previous barrier
        if (!LATE && more && kn < nk) {
            oa.issue(stage_a(buf ^ 1), A, exta, lda, k1, wq);
            ob.issue(stage_b(buf ^ 1), B, extb, ldb, k1, wq);
        }
        if (kt < nk) {
            const char *as = stage_a(buf), *bs = stage_b(buf);
            v4f fa[IB], fb[JB];
#pragma unroll
            for (int i = 0; i < IB; ++i) fa[i] = OA::frag(as, aoff[i][0]);
#pragma unroll
            for (int j = 0; j < JB; ++j) fb[j] = OB::frag(bs, boff[j][0]);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                v4f na[IB], nb[JB];
#pragma unroll
                for (int i = 0; i < IB; ++i)
                    na[i] = g + 1 < NG ? OA::frag(as, aoff[i][g + 1]) : fa[i];
#pragma unroll
                for (int j = 0; j < JB; ++j)
                    nb[j] = g + 1 < NG ? OB::frag(bs, boff[j][g + 1]) : fb[j];
                // The next group's LDS reads and this group's MFMAs, interleaved
                // by the pattern below: each MFMA is followed by up to two of
                // the reads (one in narrow tiles).  Same box, against all reads
                // ahead of the MFMAs: 2048^3 126.8 -> 125.7 us, the GPT-2
                // products 1-3.5% faster.
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int i = 0; i < IB; ++i)
#pragma unroll
                        for (int j = 0; j < JB; ++j) {
                            if constexpr (MF == 32)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                    fa[i][t], fb[j][t], acc[i][j], 0, 0, 0);
                            else
                                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                    fa[i][t], fb[j][t], acc[i][j], 0, 0, 0);
                        }
                // 64 x 64 tiles in two k-groups over an x-major A raise the
                // wave's priority for a slab's MFMAs (2048^3 127.9 -> 127.0 us,
                // 1024 x 3072 x 768 42.4 -> 41.9); over a k-major A it cost 8%
                // (768 x 2304 x 1024 TN), and on the other tiles up to 13%.
                if constexpr (KS == 2 && WPG == 4 && AX) {
                    if (g == 0) __builtin_amdgcn_s_setprio(1);
                    if (g == NG - 1) __builtin_amdgcn_s_setprio(0);
                }
#pragma unroll
                for (int t = 0; t < 4 * IB * JB; ++t) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    // two LDS reads (one in narrow tiles: 1280 x 2048 x 1024
                    // 53.1 -> 45.6 us, the others within 1%)
                    __builtin_amdgcn_sched_group_barrier(0x100, WPG == 2 ? 1 : 2, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (LATE && g == 0 && more && kn < nk) {
                    oa.issue(stage_a(buf ^ 1), A, exta, lda, k1, wq);
                    ob.issue(stage_b(buf ^ 1), B, extb, ldb, k1, wq);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int i = 0; i < IB; ++i) fa[i] = na[i];
#pragma unroll
                for (int j = 0; j < JB; ++j) fb[j] = nb[j];
            }
        }
        if (more) {
            // the loads into LDS are tracked by vmcnt; the compiler does not
            // wait for them, so wait here before publishing the slab
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            if (kn < nk && k1 + BK > K) {
                oa.zero_tail(stage_a(buf ^ 1), k1, K, wq, lane);
                ob.zero_tail(stage_b(buf ^ 1), k1, K, wq, lane);
            }
            // A k-group of one wave reads only the stages it fills itself:
            // its own wait above publishes the slab to it, and its reads of
            // a stage are done before it issues loads into that stage again,
            // so the groups run on without a workgroup barrier per slab
            // (32 x 32 tiles: 500 x 500 x 2000 12.9 -> 12.1 us, 128 x 768 x
            // 3072 16.6 -> 15.6, 64 x 1024 x 4096 20.8 -> 19.2).  They meet
            // again at the barrier before the hand-over.
            if constexpr (WPG > 1) __syncthreads();
        }
    }

    // The k-groups' sums meet in LDS.  With four or more k-groups, group g
    // finishes about a KS-th of a lane's accumulator words (split below):
    // every group writes the words the others finish, and after a
    // barrier each adds, for its own words, all groups' values in group
    // order and stores them, so every wave takes part in the hand-over and
    // the stores (500 x 500 x 2000 13.7 -> 13.0 us, 1024^3 20.2 -> 19.8,
    // 256^3 4.9 -> 4.35; with 6 groups on narrow tiles 346 x 768 x 1536
    // 16.9 -> 16.3, 400 x 1024 x 2048 20.8 -> 20.1).  With two k-groups,
    // where the other workgroup on the CU keeps the matrix cores busy
    // meanwhile, group 1 hands its words to group 0, which adds them and
    // stores the tile (split, the narrow tiles ran 1.5-2.5% slower and
    // 1024 x 3072 x 768 NT 4%).  Either way each output is
    // ((g0 + g1) + g2) + ..., fixed for a given KS.
    // Word e of a lane goes to group e * KS / ACCW: ACCW / KS words each,
    // one more for some groups when KS does not divide ACCW (16 words over
    // 6 groups: 3, 3, 2, 3, 3, 2).
    constexpr bool SPLIT_OUT = KS >= 4 && ACCW >= KS;
    const auto owner = [](int e) { return e * KS / ACCW; };
    if constexpr (KS > 1) {
        float *red = reinterpret_cast<float *>(smem);
        __syncthreads();                          // every stage read is done
        if constexpr (SPLIT_OUT) {
            static_assert(KS * WPG * ACCW * 64 * 4 <= KS * 2 * STAGE,
                          "the hand-over of partial sums must fit in the stages");
            // word e of lane l of wave wq of group g at (g*WPG + wq)*ACCW*64 + e*64 + l
            float *dst = red + (grp * WPG + wq) * ACCW * 64 + lane;
#pragma unroll
            for (int i = 0; i < IB; ++i)
#pragma unroll
                for (int j = 0; j < JB; ++j)
#pragma unroll
                    for (int r = 0; r < AR; ++r) {
                        const int e = (i * JB + j) * AR + r;
                        if (owner(e) != grp) dst[e * 64] = acc[i][j][r];
                    }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < IB; ++i)
#pragma unroll
                for (int j = 0; j < JB; ++j)
#pragma unroll
                    for (int r = 0; r < AR; ++r) {
                        const int e = (i * JB + j) * AR + r;
                        if (owner(e) != grp) continue;
                        float v = 0.f;
#pragma unroll
                        for (int g = 0; g < KS; ++g) {
                            const float x =
                                g == grp ? acc[i][j][r] : red[(g * WPG + wq) * ACCW * 64 + e * 64 + lane];
                            v = g == 0 ? x : v + x;
                        }
                        acc[i][j][r] = v;
                    }
        } else {
            // word e of lane l of wave wq of group g at ((g-1)*WPG + wq)*ACCW*64 + e*64 + l
            if (grp > 0) {
                float *dst = red + ((grp - 1) * WPG + wq) * ACCW * 64 + lane;
#pragma unroll
                for (int i = 0; i < IB; ++i)
#pragma unroll
                    for (int j = 0; j < JB; ++j)
#pragma unroll
                        for (int r = 0; r < AR; ++r) dst[((i * JB + j) * AR + r) * 64] = acc[i][j][r];
            }
            __syncthreads();
            if (grp > 0) return;
#pragma unroll
            for (int g = 1; g < KS; ++g) {
                const float *src = red + ((g - 1) * WPG + wq) * ACCW * 64 + lane;
#pragma unroll
                for (int i = 0; i < IB; ++i)
#pragma unroll
                    for (int j = 0; j < JB; ++j)
#pragma unroll
                        for (int r = 0; r < AR; ++r) acc[i][j][r] += src[((i * JB + j) * AR + r) * 64];
            }
        }
    }

    // Accumulator layouts: register r of lane l holds, in a 32 x 32 block,
    // row 8*(r/4) + 4*(l/32) + r%4 and column l%32; in a 16 x 16 block, row
    // 4*(l/16) + r and column l%16.
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            const int col = n0 + wn + MF * j + (lane & (MF - 1));
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < AR; ++r) {
                if (SPLIT_OUT && owner((i * JB + j) * AR + r) != grp) continue;
                const int row = m0 + wm + MF * i +
                                (MF == 32 ? 8 * (r >> 2) + 4 * h + (r & 3) : 4 * (lane >> 4) + r);
                if (row < M) store_c(C + (int64_t)row * ldc + col, acc[i][j][r], alpha, beta);
            }
        }
}

template <bool AX, bool BX, int BM, int BN, int KS = 1, int WPG = 4, bool KT = false, int MF = 32>
hipError_t launch_direct(int M, int N, int K, float alpha, const float *A, int64_t lda,
                         const float *B, int64_t ldb, float beta, float *C, int64_t ldc,
                         hipStream_t s) {
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    return launch(gemm_f32_direct<BM, BN, AX, BX, KS, WPG, KT, MF>, dim3(tiles_m * tiles_n),
                  dim3(64 * WPG * KS), s, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tiles_m,
                  tiles_n);
}

// Narrow tiles, 64 x 32 (TALL) or 32 x 64, with two waves per k-group and
// KS k-groups (6 fill 144 KiB of LDS).
template <bool AX, bool BX, bool TALL, bool KT>
hipError_t launch_half(int ks, int M, int N, int K, float alpha, const float *A, int64_t lda,
                       const float *B, int64_t ldb, float beta, float *C, int64_t ldc,
                       hipStream_t s) {
    constexpr int BM = TALL ? 64 : 32, BN = TALL ? 32 : 64;
    switch (ks) {
    case 6: return launch_direct<AX, BX, BM, BN, 6, 2, KT>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s);
    case 4: return launch_direct<AX, BX, BM, BN, 4, 2, KT>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s);
    case 2: return launch_direct<AX, BX, BM, BN, 2, 2, KT>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s);
    default: return launch_direct<AX, BX, BM, BN, 1, 2, KT>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s);
    }
}

// Quarter tiles: 32 x 32, one wave per k-group, KS k-groups (8 fill 128 KiB
// of LDS).
template <bool AX, bool BX, bool KT>
hipError_t launch_quarter(int ks, int M, int N, int K, float alpha, const float *A, int64_t lda,
                          const float *B, int64_t ldb, float beta, float *C, int64_t ldc,
                          hipStream_t s) {
    switch (ks) {
    case 8: return launch_direct<AX, BX, 32, 32, 8, 1, KT>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s);
    case 4: return launch_direct<AX, BX, 32, 32, 4, 1, KT>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s);
    case 2: return launch_direct<AX, BX, 32, 32, 2, 1, KT>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s);
    default: return launch_direct<AX, BX, 32, 32, 1, 1, KT>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s);
    }
}

// The direct kernel for a tile choice made by launch_gemm.
template <bool AX, bool BX, bool KT>
hipError_t launch_pick(bool quarter, bool half, bool tall, bool t48, int ksq, int ksh, int ks,
                       int M, int N, int K, float alpha, const float *A, int64_t lda,
                       const float *B, int64_t ldb, float beta, float *C, int64_t ldc,
                       hipStream_t s) {
    if (quarter) return launch_quarter<AX, BX, KT>(ksq, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s);
    if (t48) return launch_direct<AX, BX, 64, 48, 4, 4, KT, 16>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s);
    if (half)
        return tall ? launch_half<AX, BX, true, KT>(ksh, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s)
                    : launch_half<AX, BX, false, KT>(ksh, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s);
    return ks == 4 ? launch_direct<AX, BX, 64, 64, 4, 4, KT>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s)
           : ks == 2 ? launch_direct<AX, BX, 64, 64, 2, 4, KT>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s)
                     : launch_direct<AX, BX, 64, 64, 1, 4, KT>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s);
}

constexpr int PROD_BK = 32;

template <bool AX, bool BX, int VA, int VB, int BM = 128, int BN = 128, int BK = PROD_BK,
          bool FENCE = true>
hipError_t launch_t(int M, int N, int K, float alpha, const float *A, int64_t lda,
                    const float *B, int64_t ldb, float beta, float *C, int64_t ldc,
                    hipStream_t s) {
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int nwg = tiles_m * tiles_n;
    return launch(gemm_f32_kernel<BM, BN, BK, AX, BX, VA, VB, FENCE>, dim3(nwg), dim3(THREADS),
                  s, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tiles_m, tiles_n);
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_gemm(bool ax, bool bx, int M, int N, int K, float alpha, const float *A,
                       int64_t lda, const float *B, int64_t ldb, float beta, float *C,
                       int64_t ldc, int num_cus, hipStream_t s) {
    // The staged path's 16-byte register loads need the operand's contiguous
    // extent, its leading dimension and its base all to be multiples of 4
    // floats; otherwise it loads floats one by one.
    const int a_contig = ax ? K : M;
    const int b_contig = bx ? K : N;
    const bool va = aligned16(A) && (lda % 4 == 0) && (a_contig % 4 == 0);
    const bool vb = aligned16(B) && (ldb % 4 == 0) && (b_contig % 4 == 0);
    // The direct path addresses each operand with 32-bit byte offsets.
    auto extent = [](bool xmajor, int X, int64_t ld, int K) {
        return xmajor ? ((int64_t)(X - 1) * ld + K) * 4 : ((int64_t)(K - 1) * ld + X) * 4;
    };
    // Its 16-byte loads need only 4-byte aligned addresses (rows of any
    // width and leading dimension), and the buffer range check is per dword,
    // so a chunk that runs past an operand's last element reads zeros there.
    const bool direct = K > 0 && extent(ax, M, lda, K) < (int64_t(1) << 31) &&
                        extent(bx, N, ldb, K) < (int64_t(1) << 31);
    // Staged path: 128 x 64 tiles when that grid still gives every CU two
    // tiles to interleave; otherwise 64 x 64, which keeps small and K-heavy
    // products (few output tiles) spread over the CUs.
    // Grids are at most 2^31 - 1 workgroups of the smallest tile (32 x 32);
    // no product that fits in memory comes near that.
    if ((int64_t)((M + 31) / 32) * ((N + 31) / 32) > INT32_MAX) return hipErrorInvalidValue;
    const int64_t tiles_128x64 = (int64_t)((M + 127) / 128) * ((N + 63) / 64);
    const bool big = tiles_128x64 >= 2 * (int64_t)num_cus;
    // Direct path: 64 x 64 tiles with the k-slabs split over KS groups of 4
    // waves, 4 when there are no more tiles than CUs (each CU then runs one
    // tile with 16 waves), else 2; fewer when K has too few slabs to share.
    const int64_t tiles_64 = (int64_t)((M + 63) / 64) * ((N + 63) / 64);
    const int slabs = (K + 31) / 32;
    const int ks = tiles_64 <= (int64_t)num_cus && slabs >= 8 ? 4 : (slabs >= 4 ? 2 : 1);
    // Smaller tiles where 64 x 64 balances badly over the CUs.  The largest
    // per-CU share of tiles is ceil(tiles / CUs); a narrow tile (64 x 32 or
    // 32 x 64) costs about half a 64 x 64 one, a little more than half on a
    // busy CU.  Of the two narrow shapes the one whose grid pads M and N
    // less is taken, on a tie 64 x 32 when A is x-major (A . B, A . B^T)
    // and 32 x 64 otherwise.
    //  - Small grids (64 x 64 tiles for fewer than half the CUs): 32 x 32
    //    tiles when those still fit one per CU, else narrow tiles.  The
    //    k-slabs split over 8 groups for 32 x 32 tiles, as many as the LDS
    //    holds (500 x 500 x 2000: 24.0 us with 64 x 32 tiles, 18.4 with
    //    32 x 32 in 4 groups, 15.3 in 8; 4 groups ran 5-19% slower from 8
    //    to 63 slabs).  Narrow tiles take 6 groups, which the LDS also
    //    holds, from 40 slabs on and 4 below (346 x 768 x 768: 9.2 us in 4,
    //    9.5 in 6; 346 x 768 x 1536 16.9 in 4, 16.3 in 6): with fewer
    //    slabs per group, filling and draining each group's pipeline costs
    //    more than the extra waves gain.
    //  - More tiles than CUs: narrow tiles when the share of 64 x 64 tiles
    //    is at least 1.2 times that of narrow ones in 64 x 64 units, i.e. a
    //    last round of 64 x 64 tiles that would leave most CUs idle.  On
    //    1024 x 2304 x 768 (576 tiles) 43.1 -> 40.6 us and on 1024 x 1216 x
    //    1024 (304 tiles) 35.1 -> 31.2 us; 432, 700, 768 and 1024 tiles
    //    stay on 64 x 64, where narrow tiles measured 6-24% slower.
    const int64_t tiles_32 = (int64_t)((M + 31) / 32) * ((N + 31) / 32);
    const int64_t pad_tall = (int64_t)((M + 63) / 64) * ((N + 31) / 32) * 2;   // in 32 x 32 units
    const int64_t pad_wide = (int64_t)((M + 31) / 32) * ((N + 63) / 64) * 2;
    const bool tall = pad_tall < pad_wide || (pad_tall == pad_wide && ax);
    const int64_t tiles_h = (tall ? pad_tall : pad_wide) / 2;
    const auto share = [num_cus](int64_t t) { return (t + num_cus - 1) / num_cus; };
    const bool small = tiles_64 * 2 < (int64_t)num_cus;
    const bool quarter = small && tiles_32 <= (int64_t)num_cus;
    const bool half = small ? !quarter
                            : tiles_64 > (int64_t)num_cus && 10 * share(tiles_64) >= 6 * share(tiles_h);
    // Between half the CUs and all of them, where 64 x 64 tiles leave CUs
    // idle: 64 x 48 tiles of 16 x 16 MFMA blocks in four k-groups when their
    // grid still fits one tile per CU (1024 x 768 outputs: 256 tiles for 256
    // CUs instead of 192; 1024 x 768 x 3072 53.7 -> 44.8 us).  With more
    // tiles than CUs, 64 x 48 tiles in two k-groups ran slower than narrow
    // tiles on 1024 x 2304 x 768 and 768 x 3072 x 1024 (41.5 against 39.7
    // us, 53.4 against 50.8), so they serve only this case.
    const int64_t tiles_48 = (int64_t)((M + 63) / 64) * ((N + 47) / 48);
    const bool t48 = !small && ks == 4 && tiles_48 <= (int64_t)num_cus && tiles_48 > tiles_64;
    const int ksq = slabs >= 8 ? 8 : (slabs >= 4 ? 4 : (slabs >= 2 ? 2 : 1));
    const int ksh = !small ? ks : (slabs >= 40 ? 6 : (slabs >= 8 ? 4 : (slabs >= 4 ? 2 : 1)));
#define GG_ARGS M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s
#define GG_GEMM_DIRECT(AX_, BX_)                                                     \
    if (K % 4 != 0 && (AX_ || BX_))                                                  \
        return launch_pick<AX_, BX_, true>(quarter, half, tall, t48, ksq, ksh, ks, GG_ARGS); \
    return launch_pick<AX_, BX_, false>(quarter, half, tall, t48, ksq, ksh, ks, GG_ARGS);
#define GG_GEMM_SHAPE(AX_, BX_, VA_, VB_)                                     \
    return big ? launch_t<AX_, BX_, VA_, VB_, 128, 64>(GG_ARGS)            \
               : launch_t<AX_, BX_, VA_, VB_, 64, 64>(GG_ARGS);
#define GG_GEMM_CASE(AX_, BX_)                      \
    if (direct) { GG_GEMM_DIRECT(AX_, BX_) }        \
    if (va && vb) { GG_GEMM_SHAPE(AX_, BX_, 4, 4) } \
    if (va) { GG_GEMM_SHAPE(AX_, BX_, 4, 1) }       \
    if (vb) { GG_GEMM_SHAPE(AX_, BX_, 1, 4) }       \
    GG_GEMM_SHAPE(AX_, BX_, 1, 1)
    if (ax && !bx) { GG_GEMM_CASE(true, false) }     // A.B
    if (!ax && !bx) { GG_GEMM_CASE(false, false) }   // A^T.B
    if (ax && bx) { GG_GEMM_CASE(true, true) }       // A.B^T
    GG_GEMM_CASE(false, true)                        // A^T.B^T
#undef GG_GEMM_CASE
#undef GG_GEMM_SHAPE
#undef GG_GEMM_DIRECT
#undef GG_ARGS
}

}  // namespace gg
