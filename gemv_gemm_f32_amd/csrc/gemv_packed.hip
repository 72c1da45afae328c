// gemv_packed.hip -- y = W.x with W as 2-bit or 4-bit codes and binary16
// group scales.
//
// The 12,288 x 1,536 2-bit matrix-vector product of "Kernel 0112" (section
// "What is being measured"): the work is dominated by streaming the packed
// weights, the original kernel kept too few reads in flight, and splitting a
// row's dot product over 32 threads was the change that paid (sections "What
// is being measured" and "The four variants").  The same page patches two
// 4-bit kernels beside it, and "More Stumbling, This Time in the Browser" has
// a packed 4-bit path; the 4-bit product here uses the same kernel with
// wider codes.  That page's kernel unpacked the fields with floating-point
// floor arithmetic and reduced through shared memory with barriers (section
// "The kernel"); these are shaped for CDNA4.  Three kernels live here: the
// row-split kernel described first (any shape), the flat split (rows of 8 to
// 48 chunks of 16 bytes; single products and 4-bit batches), which share the
// multiply-add unpack below, and the integer-dot kernel for batches of 2-bit
// products on the configurations' shapes, described at its definition.
//
//  * Units: a row is read in units of 16 codes -- 4 bytes of 2-bit codes or
//    8 bytes of 4-bit codes -- and 4 units make one 64-column scale group.
//  * Split: a row belongs to SPLIT lanes.  Lane j of those takes units j,
//    j+SPLIT, j+2*SPLIT, ..., so each load instruction covers 128 (2-bit) or
//    256 (4-bit) contiguous bytes of a row per 32 lanes.  With SPLIT = 32 (half
//    a wave64) each half-wave owns RPL consecutive rows; with SPLIT = 256 the
//    workgroup's four waves share RPL rows, the deeper split that long rows
//    with few outputs need: the transposed 12,288 -> 1,536 shape, whose
//    kernel 0113 was patched from 2 x 32 to 1 x 256 threads per row in the
//    running model ("Kernel 0112", section "What the kernel costs in a whole
//    token").  Either way each group of lanes issues every code and scale
//    load of a pass before consuming any, so all bytes of a call are
//    requested up front.
//  * x: lane j keeps the 16 x values of each of its units in registers and
//    reuses them for all RPL rows; x is 6 KiB and read from L2/L1.
//  * Unpack: a code pair is masked out of its 32-bit word where it lies, one
//    code in each 16-bit half, and the result read as two binary16 numbers.
//    With the exponent field left at zero each half is a subnormal,
//    h = c * 2^(pos - 24) exactly, for a code c at fraction bit pos; codes
//    above bit 9 of a half are first shifted down by one shift per word.
//    That is one v_and_b32 per two weights.  The multiply-add reads h
//    directly as a binary16 operand of v_fma_mix_f32 (which converts
//    subnormal binary16 operands exactly: the library is built without
//    denormal flushing), with x and the accumulator in fp32.  Each x is
//    scaled once per pass by 2^(K0 - pos) for the position pos its codes
//    take, so every product is c * x * 2^(K0 - 24), formed from exact
//    operands; K0 is 8 for 2-bit codes and 4 for 4-bit ones.  With the zero
//    point z = (2^b - 1) / 2 of the code-to-weight map w = (c - z) * s,
//    per unit:
//        a = -z 2^(K0 - 24) X + sum h x' = 2^(K0 - 24) sum (c - z) x,
//    with X = sum x over the unit's columns, precomputed once per lane and
//    reused for every row.  The row sum is y = 2^(24 - K0) * sum over units
//    of s * a: about 1.6 instructions per weight, and one scale multiply
//    per 16 weights.
//  * Rounding: a partial sum of a unit's chain is
//    sum_{i<=n} (c_i - z) x_i - z sum_{i>n} x_i, within z sum|x|, and
//    |c - z| >= 1/2, so sum |w x| >= s sum|x| / 2 over a unit.  The 17
//    roundings of the chain and the 15 of X then keep the fp32 error below
//    64 z 2^-24 sum |w x|: 6e-6 for 2-bit codes and 3e-5 for 4-bit ones, for
//    any inputs whose scaled values and products stay normal fp32 numbers
//    (|x| between 2^-100 and 2^100).
//  * Reduction: the partial sums of a row are added within each wave with DPP
//    and ds_swizzle (wave.hpp), without LDS or atomics; with SPLIT = 256 the
//    four wave sums then meet in LDS and one lane adds them in wave order.
//    The tree is fixed, so results repeat bit for bit.
//  * A byte-load specialisation of the same kernel serves K not a multiple of
//    16, or Q rows not aligned to a unit; it masks columns k >= K.
//  * Batches: blockIdx.y picks one of up to 64 products of one shape whose
//    pointers travel in the kernel arguments, so a token's worth of products
//    costs one launch.
#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "wave.hpp"

namespace gg {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));

constexpr int THREADS = 256;
constexpr int WAVES = THREADS / 64;
constexpr int UPL = 3;                  // units of 16 codes per lane per pass

// Device pointers of up to NB products of one shape, passed by value in the
// kernel arguments (blockIdx.y selects the product).
template <int NB>
struct PackedPtrs {
    const uint8_t *Q[NB];
    const uint16_t *S[NB];
    const float *x[NB];
    float *y[NB];
};

// Per-width constants of the unpack.  Pair t of a word is code t of the low
// half and code t + HALF of the high half, at the same bit of each half.
template <int BITS>
struct Codes {
    static constexpr int UW = BITS / 2;              // 32-bit words per unit
    static constexpr int CPD = 32 / BITS;            // codes per word
    static constexpr int HALF = CPD / 2;             // code pairs per word
    static constexpr unsigned FIELD = (1u << BITS) - 1u;
    static constexpr int SH = BITS == 2 ? 6 : 8;     // shift for pairs above bit 9
    static constexpr int K0 = BITS == 2 ? 8 : 4;     // x scaled by 2^(K0 - pos)
    static constexpr float Z = (float)FIELD / 2.f;   // zero point
    static constexpr float OUT = (float)(1 << (24 - K0));
    // whether pair t is shifted down first, and its fraction bit after that
    static constexpr bool shifted(int t) { return BITS * (t + 1) > 10; }
    static constexpr int pos(int t) { return shifted(t) ? BITS * t - SH : BITS * t; }
    static constexpr unsigned mask(int t) { return (FIELD << pos(t)) | (FIELD << (pos(t) + 16)); }
};
// The unit of 16 codes at unit index u of a row, as UW words: the fast
// specialisation loads it whole; the generic one assembles it from bytes,
// zeroing columns at or beyond K.
template <int BITS, bool FAST>
__device__ __forceinline__ void load_unit(const uint8_t *__restrict__ Qrow, int u, int K,
                                          unsigned (&w)[Codes<BITS>::UW]) {
    constexpr int UW = Codes<BITS>::UW, CPB = 8 / BITS;   // codes per byte
    if (FAST) {
        if (UW == 1) {
            w[0] = reinterpret_cast<const unsigned *>(Qrow)[u];
        } else {
            const u2 v = reinterpret_cast<const u2 *>(Qrow)[u];
            w[0] = v.x;
            w[UW - 1] = v.y;
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < UW; ++i) {
        unsigned word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int k = u * 16 + (4 * i + b) * CPB;   // first column of this byte
            if (k < K) {
                unsigned byte = Qrow[k / CPB];
                const int live = K - k;                  // columns of this byte below K
                if (live < CPB) byte &= (1u << (BITS * live)) - 1u;
                word |= byte << (8 * b);
            }
        }
        w[i] = word;
    }
}

// SPLIT lanes per row (32 or 256); RPL rows per group of SPLIT lanes; FAST:
// unit loads and 32-bit offsets; FULL (with FAST): every group's rows and
// every pass's units exist, so no index is clamped; NB: number of products
// the pointer block holds (blockIdx.y picks one).
template <int BITS, int SPLIT, int RPL, bool FAST, bool FULL, int NB>
__global__ __launch_bounds__(THREADS) void gemv_packed_kernel(int M, int K, int64_t ldq,
                                                              int64_t lds, PackedPtrs<NB> ptrs) {
    static_assert(SPLIT == 32 || SPLIT == THREADS, "a row is split over 32 or 256 lanes");
    using C = Codes<BITS>;
    constexpr int UW = C::UW, UB = 4 * UW;         // words, bytes per unit
    constexpr int UNITS_PER_PASS = SPLIT * UPL;
    const int b = NB == 1 ? 0 : (int)blockIdx.y;
    const uint8_t *__restrict__ Q = ptrs.Q[b];
    const uint16_t *__restrict__ S = ptrs.S[b];
    const float *__restrict__ x = ptrs.x[b];
    float *__restrict__ y = ptrs.y[b];
    const int lane = threadIdx.x & 63;
    const int j = SPLIT == 32 ? lane & 31 : (int)threadIdx.x;   // lane within the row's group
    int row0;
    if (SPLIT == 32) {
        const int wave = blockIdx.x * WAVES + (threadIdx.x >> 6);
        row0 = wave * (2 * RPL) + (lane >> 5) * RPL;
        if (wave * (2 * RPL) >= M) return;    // uniform per wave
    } else {
        row0 = blockIdx.x * RPL;
        if (row0 >= M) return;                // uniform per workgroup
    }

    const int units = (K + 15) >> 4;      // units of 16 codes per row
    const int row_last = M - 1;
    float acc[RPL];
#pragma unroll
    for (int m = 0; m < RPL; ++m) acc[m] = 0.f;

    for (int u0 = 0; u0 < units; u0 += UNITS_PER_PASS) {
        // ---- Loads.  Every load of a pass is issued first, unconditionally,
        // from clamped (always in-bounds) addresses, unit by unit: a unit's x,
        // then its codes and scale in every row.  The multiply-adds below run
        // unit by unit across the rows too, so each unit's work can start as
        // soon as its own data has arrived.  Predicated loads, or selects right after each load,
        // make the compiler wait for each load before issuing the next.  The
        // fast path addresses with 32-bit byte offsets from the base pointer.
        v4f xraw[UPL][4];
        unsigned craw[RPL][UPL][UW];
        unsigned sraw[RPL][UPL];          // binary16 bits, zero-extended
        if (FULL) {
            // Every row and unit of this wave exists: one per-lane base and
            // compile-time offsets (row m adds m*ldq, unit q adds 32q units).
            const char *xb = reinterpret_cast<const char *>(x) + (unsigned)(u0 + j) * 64u;
            const unsigned qb = (unsigned)row0 * (unsigned)ldq + (unsigned)(u0 + j) * UB;
            const unsigned sb = ((unsigned)row0 * (unsigned)lds + (unsigned)((u0 + j) >> 2)) * 2u;
#pragma unroll
            for (int q = 0; q < UPL; ++q) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    xraw[q][c] = *reinterpret_cast<const v4f *>(xb + 64 * SPLIT * q + 16 * c);
#pragma unroll
                for (int m = 0; m < RPL; ++m) {
                    const char *qp = reinterpret_cast<const char *>(Q) + qb +
                                     (unsigned)m * (unsigned)ldq + (unsigned)(SPLIT * UB * q);
                    if (UW == 1) {
                        craw[m][q][0] = *reinterpret_cast<const unsigned *>(qp);
                    } else {
                        const u2 v = *reinterpret_cast<const u2 *>(qp);
                        craw[m][q][0] = v.x;
                        craw[m][q][UW - 1] = v.y;
                    }
                    sraw[m][q] = *reinterpret_cast<const uint16_t *>(
                        reinterpret_cast<const char *>(S) + sb + (unsigned)m * (unsigned)lds * 2u +
                        (unsigned)(SPLIT / 2 * q));
                }
                __builtin_amdgcn_sched_barrier(0);   // keep the unit order
            }
        } else {
#pragma unroll
            for (int q = 0; q < UPL; ++q) {
                const int ud = u0 + j + SPLIT * q;
                const int udc = ud < units ? ud : units - 1;
                if (FAST) {
                    const char *xb = reinterpret_cast<const char *>(x) + (unsigned)udc * 64u;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        xraw[q][c] = *reinterpret_cast<const v4f *>(xb + 16 * c);
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int k = udc * 16 + 4 * c + e;
                            xraw[q][c][e] = x[k < K ? k : K - 1];
                        }
                }
#pragma unroll
                for (int m = 0; m < RPL; ++m) {
                    const int row = row0 + m;
                    const int rowc = row < M ? row : row_last;
                    if (FAST) {
                        const unsigned qo = (unsigned)rowc * (unsigned)ldq;
                        const unsigned so =
                            ((unsigned)rowc * (unsigned)lds + (unsigned)(udc >> 2)) * 2u;
                        load_unit<BITS, true>(reinterpret_cast<const uint8_t *>(Q) + qo, udc, K,
                                              craw[m][q]);
                        sraw[m][q] = *reinterpret_cast<const uint16_t *>(
                            reinterpret_cast<const char *>(S) + so);
                    } else {
                        load_unit<BITS, false>(Q + (int64_t)rowc * ldq, udc, K, craw[m][q]);
                        sraw[m][q] = S[(int64_t)rowc * lds + (udc >> 2)];
                    }
                }
                __builtin_amdgcn_sched_barrier(0);   // keep the unit order
            }
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- Dead units (past the row's end, only in a last partial pass)
        // contribute nothing: their x and scale are zeroed.  Rows past M are
        // computed on a clamped row and never stored.
        float xv[UPL][16];
        unsigned sbits[RPL][UPL];
        if (FULL || (FAST && u0 + UNITS_PER_PASS <= units)) {
#pragma unroll
            for (int q = 0; q < UPL; ++q) {
#pragma unroll
                for (int p = 0; p < 16; ++p) xv[q][p] = xraw[q][p >> 2][p & 3];
#pragma unroll
                for (int m = 0; m < RPL; ++m) sbits[m][q] = sraw[m][q];
            }
        } else {
#pragma unroll
            for (int q = 0; q < UPL; ++q) {
                const int ud = u0 + j + SPLIT * q;
                const bool live = ud < units;
#pragma unroll
                for (int p = 0; p < 16; ++p)
                    xv[q][p] = (live && (FAST || ud * 16 + p < K)) ? xraw[q][p >> 2][p & 3] : 0.f;
#pragma unroll
                for (int m = 0; m < RPL; ++m) sbits[m][q] = live ? sraw[m][q] : 0u;
            }
        }

        // ---- Unit by unit, in the order the loads were issued: X = sum x
        // (unscaled) for the zero point, each x scaled for the bit position
        // its codes take, then one multiply-add chain per row; the RPL rows'
        // chains are independent and interleave.
#pragma unroll
        for (int q = 0; q < UPL; ++q) {
            float X = 0.f;
#pragma unroll
            for (int p = 0; p < 16; ++p) X += xv[q][p];
            const float init = (-C::Z / C::OUT) * X;
#pragma unroll
            for (int p = 0; p < 16; ++p)
                xv[q][p] *= (float)(1 << (C::K0 - C::pos((p % C::CPD) % C::HALF)));
#pragma unroll
            for (int m = 0; m < RPL; ++m) {
                float a = init;
#pragma unroll
                for (int i = 0; i < UW; ++i)
#pragma unroll
                    for (int t = 0; t < C::HALF; ++t) {
                        const unsigned d = craw[m][q][i];
                        const unsigned e = C::shifted(t) ? d >> C::SH : d;
                        const h2 hv = __builtin_bit_cast(h2, e & C::mask(t));
                        a = __builtin_fmaf((float)hv.x, xv[q][i * C::CPD + t], a);
                        a = __builtin_fmaf((float)hv.y, xv[q][i * C::CPD + t + C::HALF], a);
                    }
                const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sbits[m][q]);
                acc[m] = __builtin_fmaf(s, a, acc[m]);
            }
            // A single product runs one wave per SIMD: keep the units apart so
            // that each waits only for its own data.  (In a batch the scheduler
            // interleaves them within the register budget of three waves.)
            if (NB == 1) __builtin_amdgcn_sched_barrier(0);
        }
    }

    if (SPLIT == 32) {
#pragma unroll
        for (int m = 0; m < RPL; ++m) {
            const float t = half32_sum(acc[m]);
            if (j == 0 && row0 + m < M) y[row0 + m] = C::OUT * t;
        }
    } else {
        __shared__ float part[WAVES][RPL];
        const int wave = threadIdx.x >> 6;
#pragma unroll
        for (int m = 0; m < RPL; ++m) {
            const float t = wave64_sum(acc[m]);
            if (lane == 0) part[wave][m] = t;
        }
        __syncthreads();
        if (threadIdx.x < RPL && row0 + (int)threadIdx.x < M) {
            float t = part[0][threadIdx.x];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) t += part[w][threadIdx.x];
            y[row0 + threadIdx.x] = C::OUT * t;
        }
    }
}

// ---------------------------------------------------------------------------
// Flat split.  A workgroup of TH lanes (192 in a batch, 576 for a single
// product) reads a block of RPS consecutive rows per step, lane f taking
// 16-byte chunk f of the block.  When a row holds CPR chunks and CPR divides
// 192 (RPS = TH / CPR), lane f
// always lands on chunk f mod CPR of row f / CPR: its columns -- and the x
// values, position scales and unit sums that go with them -- are the same at
// every step, so they are set up once per workgroup.  Each load instruction
// then covers 1 KiB of weights, contiguous when rows are (ldq equal to the
// row width), and each scale load 128 contiguous bytes.  A chunk is one scale
// group of 2-bit codes or half a group of 4-bit codes, so a lane needs one
// scale per chunk.  Per chunk the lane forms the UPC unit chains of the
// unpack above, adds them in unit order and applies the scale; the CPR
// partial sums of a row meet in LDS, where one lane adds them in a fixed
// pairwise tree.  The order is fixed for a given shape, so results repeat bit
// for bit, and single and batched products agree bit for bit.
constexpr int FLAT_THREADS = 192;
// A single product takes nine-wave workgroups: a third as many workgroups
// read x and dispatch (2-bit 12,288 x 1,536: 3.94 -> 3.76 us; 4-bit 4.47 ->
// 4.28 us, same box; 384 lanes gave 3.91 and 4.29 us, 768 lanes 4.00 and
// 4.46 us).
constexpr int FLAT_SINGLE_THREADS = 576;
constexpr int FLAT_MIN_CPR = 8, FLAT_MAX_CPR = 48;

typedef unsigned u4 __attribute__((ext_vector_type(4)));

// Cache policy of the code loads: non-temporal (each code byte is read once).
[[maybe_unused]] constexpr int NT = 2;

// The per-lane pieces of the flat split, shared by the one-shot and the
// streaming kernels so that both form every row the same way.
template <int BITS>
struct Flat {
    using C = Codes<BITS>;
    static constexpr int CC = 128 / BITS;     // codes per 16-byte chunk
    static constexpr int UPC = CC / 16;       // units of 16 codes per chunk
    static constexpr int CPG = 64 / CC;       // chunks per 64-column scale group
    static constexpr int XP = CC + 4;         // LDS floats per chunk of scaled x (padded)

    struct Smem {
        float xs[FLAT_MAX_CPR * XP];
        float xi[FLAT_MAX_CPR * UPC];
    };

    // Set-up, one unit of 16 columns per lane: load_x fetches the unit's x
    // (lanes past the last unit fetch nothing: every workgroup reads x, so
    // its loads are a large share of the set-up's traffic); stage turns them
    // into the chain start -z 2^(K0-24) X and the x values scaled for their
    // codes' bit positions, in LDS, and after a barrier each lane takes those
    // of its chunk c.
    static __device__ __forceinline__ void load_x(const float *__restrict__ x, int cpr, int f,
                                                  float (&v)[16]) {
        if (f < cpr * UPC) {
            const v4f *xp = reinterpret_cast<const v4f *>(x) + 4 * f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const v4f t = xp[q];
                v[4 * q] = t.x;
                v[4 * q + 1] = t.y;
                v[4 * q + 2] = t.z;
                v[4 * q + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int p = 0; p < 16; ++p) v[p] = 0.f;
        }
    }
    static __device__ __forceinline__ void stage(const float (&v)[16], int cpr, int f, int c,
                                                 Smem &sm, float (&xv)[CC], float (&init)[UPC]) {
        if (f < cpr * UPC) {
            float X = 0.f;
#pragma unroll
            for (int p = 0; p < 16; ++p) X += v[p];
            sm.xi[f] = (-C::Z / C::OUT) * X;
            float *dst = sm.xs + (f / UPC) * XP + 16 * (f % UPC);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v4f t;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    t[e] = v[4 * q + e] *
                           (float)(1 << (C::K0 - C::pos(((4 * q + e) % C::CPD) % C::HALF)));
                *reinterpret_cast<v4f *>(dst + 4 * q) = t;
            }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < CC / 4; ++q) {
            const v4f t = *reinterpret_cast<const v4f *>(sm.xs + c * XP + 4 * q);
            xv[4 * q] = t.x;
            xv[4 * q + 1] = t.y;
            xv[4 * q + 2] = t.z;
            xv[4 * q + 3] = t.w;
        }
#pragma unroll
        for (int i = 0; i < UPC; ++i) init[i] = sm.xi[c * UPC + i];
    }

    // The lane's chunk of one step: the unit chains, their sum in unit
    // order, times the chunk's scale.
    static __device__ __forceinline__ float step(const unsigned (&w)[4], unsigned sbits,
                                                 const float (&xv)[CC], const float (&init)[UPC]) {
        float a[UPC];
#pragma unroll
        for (int i = 0; i < UPC; ++i) {
            a[i] = init[i];
#pragma unroll
            for (int k = 0; k < C::UW; ++k)
#pragma unroll
                for (int h = 0; h < C::HALF; ++h) {
                    const unsigned d = w[i * C::UW + k];
                    const unsigned e = C::shifted(h) ? d >> C::SH : d;
                    const h2 hv = __builtin_bit_cast(h2, e & C::mask(h));
                    a[i] = __builtin_fmaf((float)hv.x, xv[16 * i + k * C::CPD + h], a[i]);
                    a[i] = __builtin_fmaf((float)hv.y, xv[16 * i + k * C::CPD + h + C::HALF],
                                          a[i]);
                }
        }
        float p = a[0];
#pragma unroll
        for (int i = 1; i < UPC; ++i) p += a[i];
        const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sbits);
        return s * p;
    }

    // The NQ * 4 partial sums of a row: every read issued first, then a
    // pairwise tree in a fixed order (one LDS round trip and log2 levels of
    // adds on the workgroup's last step, instead of a chain through it).
    template <int NQ>
    static __device__ __forceinline__ float row_sum(const float *pr) {
        float v[4 * NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const v4f t = *reinterpret_cast<const v4f *>(pr + 4 * q);
            v[4 * q] = t.x;
            v[4 * q + 1] = t.y;
            v[4 * q + 2] = t.z;
            v[4 * q + 3] = t.w;
        }
#pragma unroll
        for (int w = 1; w < 4 * NQ; w *= 2)
#pragma unroll
            for (int i = 0; i + w < 4 * NQ; i += 2 * w) v[i] += v[i + w];
        return v[0];
    }

    // Rows [0, nrows) of a block of partial sums (ps floats per row, cpr
    // used), one lane per row; row r goes to y[r] when r < rows_valid.
    static __device__ __forceinline__ void rows(const float *part, int ps, int cpr, int nrows,
                                                int rows_valid, float *__restrict__ y, int f,
                                                int threads) {
        for (int r = f; r < nrows; r += threads) {
            if (r >= rows_valid) break;
            const float *pr = part + r * ps;
            float sum;
            switch (cpr) {   // the chunk counts the flat split takes
            case 8: sum = row_sum<2>(pr); break;
            case 12: sum = row_sum<3>(pr); break;
            case 16: sum = row_sum<4>(pr); break;
            case 24: sum = row_sum<6>(pr); break;
            case 32: sum = row_sum<8>(pr); break;
            default: sum = row_sum<12>(pr); break;   // 48
            }
            y[r] = C::OUT * sum;
        }
    }
};

// Code and scale loads of the workgroup's rows from row0 on: buffer
// resources that start at row0 and end at the matrix's last byte, so rows
// past M read zeros (they are never stored), and per-lane offsets.
struct FlatLoads {
#if defined(__HIP_DEVICE_COMPILE__)
    __amdgpu_buffer_rsrc_t rq, rs;
#endif
    unsigned vq, vs, sq, ss;

    __device__ __forceinline__ void init(const uint8_t *Q, const uint16_t *S, int M, int row0,
                                         int cpr, int cpg, int rps, int rin, int c, int64_t ldq,
                                         int64_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
        const int rows_left = M - row0;       // >= 1
        const int extq = (int)((int64_t)(rows_left - 1) * ldq + 16 * cpr);
        const int exts = (int)(((int64_t)(rows_left - 1) * lds + (cpr + cpg - 1) / cpg) * 2);
        rq = __builtin_amdgcn_make_buffer_rsrc((void *)(Q + (int64_t)row0 * ldq), (short)0, extq,
                                               0x00020000);
        rs = __builtin_amdgcn_make_buffer_rsrc((void *)(S + (int64_t)row0 * lds), (short)0, exts,
                                               0x00020000);
#endif
        vq = (unsigned)rin * (unsigned)ldq + 16u * (unsigned)c;
        vs = ((unsigned)rin * (unsigned)lds + (unsigned)(c / cpg)) * 2u;
        sq = (unsigned)rps * (unsigned)ldq;
        ss = (unsigned)rps * (unsigned)lds * 2u;
    }

    // Steps s0 .. s0 + T - 1, issued in step order.
    template <int T>
    __device__ __forceinline__ void issue(int s0, unsigned (&craw)[T][4], unsigned (&sraw)[T]) const {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const unsigned st = (unsigned)(s0 + t);
            const u4 v = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(vq + st * sq), 0, NT);
            craw[t][0] = v.x;
            craw[t][1] = v.y;
            craw[t][2] = v.z;
            craw[t][3] = v.w;
            sraw[t] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(vs + st * ss), 0, 0);
            __builtin_amdgcn_sched_barrier(0);   // keep the step order
        }
#else
        for (int t = 0; t < T; ++t) {
            craw[t][0] = craw[t][1] = craw[t][2] = craw[t][3] = sraw[t] = 0u * (unsigned)s0;
        }
#endif
    }
};

// T steps per workgroup; a batch asks for four waves per SIMD (at most 128
// VGPRs), which fits five three-wave workgroups on a compute unit.  EARLY:
// the code loads are issued between the x loads and the set-up arithmetic,
// so that their latency runs under the set-up (vector-memory loads retire
// in issue order, so the set-up's wait for x does not wait for them).
template <int BITS, int T, int NB, bool EARLY, int TH = FLAT_THREADS>
__global__ __launch_bounds__(TH) __attribute__((amdgpu_waves_per_eu(NB == 1 ? 1 : 4)))
void gemv_packed_flat(int M, int cpr, int rdiv, int64_t ldq, int64_t lds, PackedPtrs<NB> ptrs) {
    using F = Flat<BITS>;
    __shared__ __attribute__((aligned(16))) typename F::Smem sm;
    __shared__ __attribute__((aligned(16))) float part[T * (TH + 4 * (TH / FLAT_MIN_CPR))];

    const int b = NB == 1 ? 0 : (int)blockIdx.y;
    const int f = threadIdx.x;
    const int rps = TH / cpr;                 // rows per step
    const int rin = (f * rdiv) >> 16, c = f - rin * cpr;   // f / cpr (rdiv = ceil(2^16 / cpr))
    const int row0 = (int)blockIdx.x * rps * T;
    const int ps = cpr + 4;                   // LDS floats per row of partial sums

    // Every chunk and scale of the T steps is issued step by step before any
    // is used; then the steps run in the same order, into LDS.
    FlatLoads ld;
    ld.init(ptrs.Q[b], ptrs.S[b], M, row0, cpr, F::CPG, rps, rin, c, ldq, lds);
    unsigned craw[T][4], sraw[T];
    float xr[16], xv[F::CC], init[F::UPC];
    F::load_x(ptrs.x[b], cpr, f, xr);
    __builtin_amdgcn_sched_barrier(0);
    if (EARLY) ld.issue<T>(0, craw, sraw);
    F::stage(xr, cpr, f, c, sm, xv, init);
    if (!EARLY) ld.issue<T>(0, craw, sraw);
#pragma unroll
    for (int t = 0; t < T; ++t) {
        part[(t * rps + rin) * ps + c] = F::step(craw[t], sraw[t], xv, init);
        if (NB == 1) __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    F::rows(part, ps, cpr, rps * T, M - row0, ptrs.y[b] + row0, f, TH);
}

// Chunks per row for the flat split, or 0 where it does not apply: every row
// a whole number of 16-byte chunks (K a multiple of 64), between 8 and 48
// chunks dividing 192, chunk-aligned rows and bases, 16-byte aligned x, and
// byte offsets within 31 bits.
template <int BITS>
int flat_cpr(int count, int M, int K, const uint8_t *const *Q, int64_t ldq, int64_t lds,
             const float *const *x) {
    if (K % 64 != 0 || ldq % 16 != 0) return 0;
    const int cpr = K * BITS / 128;
    if (cpr < FLAT_MIN_CPR || cpr > FLAT_MAX_CPR || FLAT_THREADS % cpr != 0) return 0;
    if ((int64_t)M * ldq >= (int64_t(1) << 31) || (int64_t)M * lds * 2 >= (int64_t(1) << 31))
        return 0;
    for (int i = 0; i < count; ++i)
        if (reinterpret_cast<uintptr_t>(Q[i]) % 16 != 0 ||
            reinterpret_cast<uintptr_t>(x[i]) % 16 != 0)
            return 0;
    return cpr;
}

// Steps per workgroup.  A single product needs many workgroups to fill the
// chip: one step (2-bit) or two (4-bit, whose rows are twice as long).  A
// batch has workgroups to spare: eight steps.  (A sweep of 1, 2 and 4 steps
// for single products and 4 to 16 for batches of 40 at 12,288 x 1,536 put
// the best there.)
// The code loads go out before the x set-up's arithmetic (EARLY): 2% faster
// for single 2-bit products and for batches, and, since x is loaded once per
// unit, for single 4-bit products too (4.57 -> 4.45 us with two steps).
template <int BITS, int NB, int T = (NB == 1 ? (BITS == 2 ? 1 : 2) : 8), bool EARLY = true,
          int TH = (NB == 1 ? FLAT_SINGLE_THREADS : FLAT_THREADS)>
hipError_t launch_flat(int count, int M, int cpr, const uint8_t *const *Q, int64_t ldq,
                       const uint16_t *const *S, int64_t lds, const float *const *x,
                       float *const *y, hipStream_t s) {
    const int rows_per_wg = TH / cpr * T;
    const dim3 grid((M + rows_per_wg - 1) / rows_per_wg, count);
    PackedPtrs<NB> p;
    for (int b = 0; b < NB; ++b) {
        const int i = b < count ? b : 0;
        p.Q[b] = Q[i];
        p.S[b] = S[i];
        p.x[b] = x[i];
        p.y[b] = y[i];
    }
    // f / cpr as (f * rdiv) >> 16 is exact for f < 768 and cpr <= 48: the
    // rounding excess f * (rdiv - 2^16 / cpr) / 2^16 stays below 1 / cpr.
    const int rdiv = (65536 + cpr - 1) / cpr;
    return launch(gemv_packed_flat<BITS, T, NB, EARLY, TH>, grid, dim3(TH), s, M, cpr, rdiv, ldq,
                  lds, p);
}

// A single product needs every SIMD busy: 6 rows per group of lanes gives
// one wave per SIMD at 12,288 rows split 32 ways, or at 1,536 rows split 256
// ways.  A batch has waves to spare, so each lane takes more rows and reuses
// its x registers and unit sums longer: 12 for 2-bit codes, 8 for 4-bit ones
// (a sweep over 6..24 rows at 40 products of 12,288 x 1,536 put each width's
// best there: 1.54 and 2.00 us per product).
template <int BITS, int SPLIT, int NB, int RPL = (NB == 1 ? 6 : (BITS == 2 ? 12 : 8))>
hipError_t launch_chunk(int count, int M, int K, const uint8_t *const *Q, int64_t ldq,
                        const uint16_t *const *S, int64_t lds, const float *const *x,
                        float *const *y, hipStream_t s) {
    constexpr int UB = 2 * BITS;                   // bytes per unit of 16 codes
    constexpr int GROUPS = THREADS / SPLIT;        // row groups per workgroup
    const int rows_per_wg = GROUPS * RPL;
    const dim3 grid((M + rows_per_wg - 1) / rows_per_wg, count);
    PackedPtrs<NB> p;
    bool aligned = true;
    for (int b = 0; b < NB; ++b) {
        const int i = b < count ? b : 0;
        p.Q[b] = Q[i];
        p.S[b] = S[i];
        p.x[b] = x[i];
        p.y[b] = y[i];
        aligned = aligned && reinterpret_cast<uintptr_t>(Q[i]) % UB == 0 &&
                  reinterpret_cast<uintptr_t>(x[i]) % 16 == 0;
    }
    // unit loads, 16-byte x loads, and 32-bit byte offsets into Q and S
    const bool fast = aligned && (K % 16 == 0) && (ldq % UB == 0) &&
                      (int64_t)M * ldq < (int64_t(1) << 32) &&
                      (int64_t)M * lds * 2 < (int64_t(1) << 32);
    const bool full = fast && (K % (16 * SPLIT * UPL) == 0) &&
                      (M % (SPLIT == 32 ? 2 * RPL : RPL) == 0);
    if (full)
        return launch(gemv_packed_kernel<BITS, SPLIT, RPL, true, true, NB>, grid, dim3(THREADS),
                      s, M, K, ldq, lds, p);
    if (fast)
        return launch(gemv_packed_kernel<BITS, SPLIT, RPL, true, false, NB>, grid, dim3(THREADS),
                      s, M, K, ldq, lds, p);
    return launch(gemv_packed_kernel<BITS, SPLIT, RPL, false, false, NB>, grid, dim3(THREADS), s,
                  M, K, ldq, lds, p);
}

// ---------------------------------------------------------------------------
// 2-bit codes with integer dot products.  The multiply-add unpack above costs
// 16 v_fma_mix_f32 and 9 bit operations per 16 weights; a batch of 2-bit
// products is bound by that work, not by HBM.  v_dot8_i32_i4 multiplies 8
// pairs of signed nibbles and adds them to an int32, so with x held as
// integers the codes need no conversion at all:
//
//  * x as integers.  Per 64-column chunk (one scale group) let E be the
//    exponent of the chunk's largest |x| (max |x| < 2^E) and
//    q_k = rint(x_k 2^k) with k = 22 - E, so |q_k| <= 2^22 and
//    |x_k - q_k 2^-k| <= 2^(-k-1).  q + 0x888888 has six nibbles d_i + 8
//    with q = sum_i d_i 16^i and d_i in [-8, 7]; flipping bit 3 of each
//    nibble gives d_i as a signed nibble.  The rounding to an integer is done
//    by the fp32 add of 1.5 * 2^23, whose bit pattern then holds q + 2^22.
//  * Five digits where they suffice.  A chunk whose sum of |x| is at least
//    2^(E+3) takes k = 18 - E (|q| <= 2^18, top digit zero); the wave takes
//    six digits if any of its 8 chunks needs them, so the branch is uniform
//    over the wave.
//  * Lanes.  A wave reads 8 chunks of 8 rows per step: lane l takes chunk
//    8 * wave + (l & 7) of row l >> 3, so each load instruction covers eight
//    128-byte segments, and the 8 lanes that share a chunk sit in one wave.
//    Those 8 lanes split the chunk's set-up, lane j taking the even (j even)
//    or odd columns of unit j >> 1 (a unit is 16 columns, one code word):
//    they quantise their 8 columns and transpose the 8 x 6 nibbles into six
//    digit words (word i holds digit i of the 8 columns), and swap them
//    through LDS inside the wave, so every lane holds the 48 digit words of
//    its chunk.  The chunk's maximum, sum of |x| and sum of q meet by lane
//    shuffles.
//  * Steps.  For a code word w, w & 0x33333333 holds the codes of its even
//    columns in nibbles 0..7 and (w >> 2) & 0x33333333 those of its odd
//    columns.  One chain of v_dot8_i32_i4 walks the digits from the top one
//    down, shifting by one digit in between, and gives, exactly,
//        T = sum_i 16^i sum_k c_k d_ik = sum_k c_k q_k    (|T| < 2^30),
//        Z = 2 T - 3 sum_k q_k = 2 sum_k (c_k - 3/2) q_k   (|Z| < 2^31),
//    both in int32, and the chunk's share of the row is s 2^(-k-1) Z.  Per
//    16 weights: 10 or 12 dot products and 3 bit operations, against 25
//    instructions for the multiply-add unpack.
//  * Rounding.  Only x is rounded.  Over a chunk that moves the sum by at
//    most 64 * (3/2) s 2^(-k-1), while the chunk's share of the bound is
//    sum |w x| >= (s/2) sum |x|: at most 96 2^-k / sum |x|, which is
//    96 2^(E-22) / 2^(E-1) = 4.6e-5 with six digits (sum |x| >= max |x|) and
//    96 2^(E-18) / 2^(E+3) = 4.6e-5 with five.  Converting Z to fp32, the
//    scale product and the row's sum over chunks add at most
//    (3 + chunks) * 3 * 2^-24 of it: below 1e-5 for up to 48 chunks.  This
//    holds for every finite x and s for which no partial result overflows or
//    falls below the normal range.
//  * Non-finite x.  A NaN or an infinity in x makes every output NaN (its
//    chunk's quantised values leave the 24-bit range, which the set-up
//    detects); a non-finite scale makes its own row non-finite.
//  * Scales.  Lane l of a wave loads the 8 scales of its wave's chunks in
//    row l of the workgroup with one 16-byte load and the lanes trade them
//    through LDS, instead of one 2-byte load per lane and step.
//  * Reduction.  The row's partial sums meet in LDS after one barrier and one
//    lane per row adds them in a fixed pairwise tree: deterministic.
//  * Slices.  Rows longer than 48 chunks (the transposed 12,288 -> 1,536
//    shape) are cut into slices of 1,536 columns, each slice of each row
//    block a workgroup of its own.  The grid is row block x slice x
//    product (blockIdx.x, y, z), so a product's slices of the same rows are
//    read close together in time while 12 workgroups share each slice's x
//    (slices outermost ran 4% slower, the slices of each row block
//    interleaved 9%).  The kernel then reads the slice's codes, scales and
//    x from offsets of z slices and
//    writes its partial row sums, block z of M values per product, to a
//    workspace; gemv_slices_sum adds a row's partials in slice order.  A
//    slice is exactly the 24-chunk row the kernel is tuned for, with three
//    waves per workgroup, and the workgroups of all slices of all products
//    of a batch run in one launch.

template <int WAVES, int T>
struct IdotSmem {
    static constexpr int CPR = 8 * WAVES, ROWS = 8 * T, PS = CPR + 4;
    // per wave: 8 chunks x 8 lanes x 6 digit words, a chunk's 48 words padded
    // to DS = 52, so that the 8 chunks' 16-byte reads fall on distinct banks
    static constexpr int DS = 52;
    unsigned dig[WAVES][8 * DS];
    uint16_t scl[WAVES][ROWS * 8];        // per wave: row x its 8 chunks' scales
    float part[ROWS * PS];                // row x chunk partial sums
    int bad[WAVES];
};

// a * b over 8 signed nibble pairs, as the first product of a chain (the
// VOP3P form with an inline zero addend: no move of a zero into the
// accumulator first, as the accumulating VOP2 form needs)
__device__ __forceinline__ int dot8_first(int a, int b) {
    int r;
    asm("v_dot8_i32_i4 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// binary16 h (the low half of hb) times fp32 f, in one mixed-precision
// multiply-add with a zero addend
__device__ __forceinline__ float mul_half(unsigned hb, float f) {
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(hb), "v"(f));
    return r;
}

__device__ __forceinline__ unsigned nib_swap(unsigned a, unsigned b, bool hi) {
    // one output of the 4-bit stage of the transpose
    return hi ? (((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u))
              : ((a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u));
}

// Code chunks in flight per lane: the first IDOT_NBUF steps' chunks are
// issued up front, the rest one by one as steps finish with their slots.
constexpr int IDOT_NBUF = 8;

// The integer-dot kernel's buffer loads: resources that start at the
// workgroup's first row and end at the matrix's last byte, so rows past M
// read zeros (they are never stored).
struct IdotLoads {
#if defined(__HIP_DEVICE_COMPILE__)
    __amdgpu_buffer_rsrc_t rq, rs;
#endif
    unsigned vq, sq, vs, ss;

    __device__ __forceinline__ void init(const uint8_t *Q, const uint16_t *S, int M, int row0,
                                         int cpr, int64_t ldq, int64_t lds, int w, int l, int j,
                                         int c) {
#if defined(__HIP_DEVICE_COMPILE__)
        const int rows_left = M - row0;       // >= 1
        rq = __builtin_amdgcn_make_buffer_rsrc((void *)(Q + (int64_t)row0 * ldq), (short)0,
                                               (int)((int64_t)(rows_left - 1) * ldq + 16 * cpr),
                                               0x00020000);
        rs = __builtin_amdgcn_make_buffer_rsrc((void *)(S + (int64_t)row0 * lds), (short)0,
                                               (int)(((int64_t)(rows_left - 1) * lds + cpr) * 2),
                                               0x00020000);
#endif
        vq = (unsigned)j * (unsigned)ldq + 16u * (unsigned)c;   // row j of step 0, chunk c
        sq = 8u * (unsigned)ldq;                                // 8 rows per step
        vs = (unsigned)l * (unsigned)lds * 2u + 16u * (unsigned)w;  // row l, this wave's 8 scales
        ss = 64u * (unsigned)lds * 2u;                          // 64 rows per scale load
    }
    // Step t's 16-byte code chunk (non-temporal: each byte is read once).
    __device__ __forceinline__ void codes(int t, unsigned (&cw)[4]) const {
#if defined(__HIP_DEVICE_COMPILE__)
        const u4 v = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(vq + (unsigned)t * sq), 0, NT);
        cw[0] = v.x;
        cw[1] = v.y;
        cw[2] = v.z;
        cw[3] = v.w;
#else
        cw[0] = cw[1] = cw[2] = cw[3] = (unsigned)t * 0u;
#endif
    }
    // The 8 scales of this wave's chunks in row r of the workgroup (16 bytes);
    // r < 0 reads from past the resource, which gives zeros.
    __device__ __forceinline__ u4 scales(int r) const {
#if defined(__HIP_DEVICE_COMPILE__)
        const int off = r < 0 ? 0x7FFFFFF0 : (int)(vs + (unsigned)(r >> 6) * ss);
        return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
#else
        return u4{0u, 0u, 0u, (unsigned)r * 0u};
#endif
    }
};

// WAVES waves per workgroup (the row has 8 * WAVES chunks), T steps of 8
// rows, NB products per pointer block; SLICED: rows cut into slices
// (blockIdx.z), partial sums out.
constexpr int IDOT_WAVES_PER_SIMD = 4;   // occupancy asked for in a batch

template <int WAVES, int T, int NB, bool SLICED = false>
__global__ __launch_bounds__(64 * WAVES)
__attribute__((amdgpu_waves_per_eu(NB == 1 ? 1 : IDOT_WAVES_PER_SIMD)))
void gemv_q2_idot(int M, int64_t ldq, int64_t lds, PackedPtrs<NB> ptrs) {
    using Sm = IdotSmem<WAVES, T>;
    constexpr int CPR = Sm::CPR, ROWS = Sm::ROWS, PS = Sm::PS;
    constexpr int NBUF = T < IDOT_NBUF ? T : IDOT_NBUF;   // code chunks in flight per lane
    constexpr int SL = (ROWS + 63) / 64;                   // 16-byte scale loads per lane
    __shared__ __attribute__((aligned(16))) Sm sm;

    // sliced: blockIdx.y is the slice and blockIdx.z the product
    const int b = NB == 1 ? 0 : (int)(SLICED ? blockIdx.z : blockIdx.y);
    const int z = SLICED ? (int)blockIdx.y : 0;    // column slice
    const int w = (int)threadIdx.x >> 6, l = (int)threadIdx.x & 63;
    const int cl = l & 7, j = l >> 3, c = 8 * w + cl, u = j >> 1;
    const unsigned odd = 0u - (unsigned)(j & 1);   // all ones for the odd-column lanes
    const int row0 = (int)blockIdx.x * ROWS;

    // ---- Loads, in the order they are needed (vector-memory loads retire in
    // issue order): the unit's 16 x values, the 16-byte scale blocks, then
    // the code chunks of the first NBUF steps; each later step's chunk is
    // issued as soon as a slot frees up.
    v4f xr[4];
    {
        const v4f *xp =
            reinterpret_cast<const v4f *>(ptrs.x[b] + (size_t)z * (64 * CPR) + 64 * c + 16 * u);
#pragma unroll
        for (int q = 0; q < 4; ++q) xr[q] = xp[q];
    }
    __builtin_amdgcn_sched_barrier(0);
    IdotLoads ld;
    ld.init(ptrs.Q[b] + (size_t)z * (16 * CPR), ptrs.S[b] + (size_t)z * CPR, M, row0, CPR, ldq,
            lds, w, l, j, c);
    u4 sraw[SL];
#pragma unroll
    for (int q = 0; q < SL; ++q) sraw[q] = ld.scales(64 * q + l < ROWS ? 64 * q + l : -1);
    __builtin_amdgcn_sched_barrier(0);
    unsigned craw[NBUF][4];
#pragma unroll
    for (int t = 0; t < NBUF; ++t) ld.codes(t, craw[t]);
    __builtin_amdgcn_sched_barrier(0);

    // ---- Set-up: this lane's 8 columns of the chunk as digit words.
    float v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        v[4 * q] = xr[q].x;
        v[4 * q + 1] = xr[q].y;
        v[4 * q + 2] = xr[q].z;
        v[4 * q + 3] = xr[q].w;
    }
    float mx = 0.f;   // largest |x| of the unit (a NaN is skipped here, caught below)
#pragma unroll
    for (int q = 0; q < 16; ++q) mx = __builtin_fmaxf(mx, __builtin_fabsf(v[q]));
    // ... and of the chunk: the other units' lanes are l ^ 16 and l ^ 32
    mx = __builtin_fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(mx), 0x401F)));
    mx = __builtin_fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_bpermute((l ^ 32) << 2,
                                                                          __float_as_int(mx))));
    const int E = __builtin_amdgcn_frexp_expf(mx);   // max |x| < 2^E; 0 for 0 and non-finite
    float xv[8];
    float ax = 0.f;   // sum of |x| over this lane's 8 columns, then over the chunk
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        // the odd or even column, by a bit select (not an indexed load)
        xv[m] = __uint_as_float((__float_as_uint(v[2 * m + 1]) & odd) |
                                (__float_as_uint(v[2 * m]) & ~odd));
        ax += __builtin_fabsf(xv[m]);
    }
    ax += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ax), 0x128, 0xF, 0xF,
                                                     false));   // row_ror:8, lane l ^ 8
    ax += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(ax), 0x401F));
    ax += __int_as_float(__builtin_amdgcn_ds_bpermute((l ^ 32) << 2, __float_as_int(ax)));
    // Five digits (|q| <= 2^18) suffice for a chunk with sum |x| >= 2^(E+3);
    // the wave takes six if any of its 8 chunks needs them.
    const bool six = __builtin_amdgcn_ballot_w64(!(ax >= __builtin_amdgcn_ldexpf(1.f, E + 3))) != 0ull;
    const int k = (six ? 22 : 18) - E;
    unsigned uq[8];
    int qs = 0;
    unsigned orr = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float t = __builtin_amdgcn_ldexpf(xv[m], k) + 12582912.f;   // + 1.5 * 2^23
        uq[m] = __float_as_uint(t) - 0x4AB77778u;      // q + 0x888888
        orr |= uq[m];
        qs += (int)uq[m];
    }
    qs -= 8 * 0x888888;
    const bool bad = (orr >> 24) != 0u;                // a NaN or an infinity in x
    // the chunk's sum of q over its 8 lanes: l ^ 8, l ^ 16, l ^ 32
    qs += __builtin_amdgcn_update_dpp(0, qs, 0x128, 0xF, 0xF, false);   // row_ror:8
    qs += __builtin_amdgcn_ds_swizzle(qs, 0x401F);
    qs += __builtin_amdgcn_ds_bpermute((l ^ 32) << 2, qs);
    const unsigned neg3q = (unsigned)(-3 * qs);
    const int kz = -k - 1;                             // Z counts halves of 2^-k
    // transpose the 8 x 8 nibbles (digits 6, 7 are zero and dropped): halves,
    // then bytes, then nibbles
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const unsigned A = uq[r], B = uq[r + 4];
        uq[r] = __builtin_amdgcn_perm(B, A, 0x05040100u);
        uq[r + 4] = __builtin_amdgcn_perm(B, A, 0x07060302u);
    }
#pragma unroll
    for (int r = 0; r < 8; r += 4)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const unsigned A = uq[r + h], B = uq[r + h + 2];
            uq[r + h] = __builtin_amdgcn_perm(B, A, 0x06020400u);
            uq[r + h + 2] = __builtin_amdgcn_perm(B, A, 0x07030501u);
        }
    unsigned dg[6];
#pragma unroll
    for (int r = 0; r < 6; r += 2) {
        dg[r] = nib_swap(uq[r], uq[r + 1], false) ^ 0x88888888u;
        dg[r + 1] = nib_swap(uq[r], uq[r + 1], true) ^ 0x88888888u;
    }
    // ---- Swap digit words and scales inside the wave through LDS.
    {
        u2 *dst = reinterpret_cast<u2 *>(&sm.dig[w][cl * Sm::DS + j * 6]);
        dst[0] = u2{dg[0], dg[1]};
        dst[1] = u2{dg[2], dg[3]};
        dst[2] = u2{dg[4], dg[5]};
#pragma unroll
        for (int q = 0; q < SL; ++q)
            if (64 * q + l < ROWS) *reinterpret_cast<u4 *>(&sm.scl[w][(64 * q + l) * 8]) = sraw[q];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    unsigned D[48];
#pragma unroll
    for (int q = 0; q < 12; ++q) {
        const u4 t = *reinterpret_cast<const u4 *>(&sm.dig[w][cl * Sm::DS + 4 * q]);
        D[4 * q] = t.x;
        D[4 * q + 1] = t.y;
        D[4 * q + 2] = t.z;
        D[4 * q + 3] = t.w;
    }

    // ---- Steps: the chunk of row 8t + j.  One chain over the even and the odd
    // columns walks the digits from the top one down, shifting by one digit
    // in between (Horner's rule inside the chain):
    //     a = ((acc_top 16 + ...) 16 + acc_1) 16 + acc_0,
    // from digit 5 when the wave takes six digits, else from digit 4 (the
    // branch is uniform over the wave).  Integer sums are exact, so the
    // order of the dot products does not change the result.
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const unsigned sb = sm.scl[w][(8 * t + j) * 8 + cl];
        int ev[4], od[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const unsigned wd = craw[t % NBUF][q];
            ev[q] = (int)(wd & 0x33333333u);
            od[q] = (int)((wd >> 2) & 0x33333333u);
        }
        if (t + NBUF < T) ld.codes(t + NBUF, craw[t % NBUF]);
        int a;
        if (six) {
            a = dot8_first(ev[0], (int)D[5]);
            a = __builtin_amdgcn_sdot8(od[0], (int)D[6 + 5], a, false);
#pragma unroll
            for (int q = 1; q < 4; ++q) {
                a = __builtin_amdgcn_sdot8(ev[q], (int)D[12 * q + 5], a, false);
                a = __builtin_amdgcn_sdot8(od[q], (int)D[12 * q + 6 + 5], a, false);
            }
            a = (int)((unsigned)a << 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a = __builtin_amdgcn_sdot8(ev[q], (int)D[12 * q + 4], a, false);
                a = __builtin_amdgcn_sdot8(od[q], (int)D[12 * q + 6 + 4], a, false);
            }
        } else {
            a = dot8_first(ev[0], (int)D[4]);
            a = __builtin_amdgcn_sdot8(od[0], (int)D[6 + 4], a, false);
#pragma unroll
            for (int q = 1; q < 4; ++q) {
                a = __builtin_amdgcn_sdot8(ev[q], (int)D[12 * q + 4], a, false);
                a = __builtin_amdgcn_sdot8(od[q], (int)D[12 * q + 6 + 4], a, false);
            }
        }
#pragma unroll
        for (int d = 3; d >= 0; --d) {
            a = (int)((unsigned)a << 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a = __builtin_amdgcn_sdot8(ev[q], (int)D[12 * q + d], a, false);
                a = __builtin_amdgcn_sdot8(od[q], (int)D[12 * q + 6 + d], a, false);
            }
        }
        const int z = (int)(((unsigned)a << 1) + neg3q);
        sm.part[(8 * t + j) * PS + c] = __builtin_amdgcn_ldexpf(mul_half(sb, (float)z), kz);
        if (NB == 1) __builtin_amdgcn_sched_barrier(0);
    }
    const unsigned long long anybad = __builtin_amdgcn_ballot_w64(bad);
    if (l == 0) sm.bad[w] = anybad != 0ull;
    __syncthreads();
    bool nan_out = false;
#pragma unroll
    for (int q = 0; q < WAVES; ++q) nan_out = nan_out || sm.bad[q] != 0;
    float *__restrict__ y = ptrs.y[b] + (size_t)z * M + row0;
    for (int r = (int)threadIdx.x; r < ROWS; r += 64 * WAVES) {
        if (row0 + r >= M) break;
        const float sum = Flat<2>::template row_sum<CPR / 4>(sm.part + r * PS);
        y[r] = nan_out ? __builtin_nanf("") : sum;
    }
}

// The integer-dot kernel serves 2-bit rows of 8 to 48 chunks, a multiple of
// 8 (K = 512, 1024, 1536, 2048, 3072), with 16-byte aligned code rows, scale
// rows (lds a multiple of 8) and x, and byte offsets within 31 bits; 0 where
// it does not apply, else the number of waves per workgroup.
inline int idot_waves(int count, int M, int K, const uint8_t *const *Q, int64_t ldq,
                      const uint16_t *const *S, int64_t lds, const float *const *x) {
    if (K % 512 != 0 || K / 64 > FLAT_MAX_CPR || ldq % 16 != 0 || lds % 8 != 0) return 0;
    if ((int64_t)M * ldq >= (int64_t(1) << 31) || (int64_t)M * lds * 2 >= (int64_t(1) << 31))
        return 0;
    for (int i = 0; i < count; ++i)
        if (reinterpret_cast<uintptr_t>(Q[i]) % 16 != 0 ||
            reinterpret_cast<uintptr_t>(S[i]) % 16 != 0 ||
            reinterpret_cast<uintptr_t>(x[i]) % 16 != 0)
            return 0;
    return K / 512;
}

// Steps per workgroup: IDOT_BATCH_T in a batch, IDOT_SINGLE_T for a single
// product, which needs many workgroups to fill the chip.
constexpr int IDOT_SINGLE_T = 1;
constexpr int IDOT_BATCH_T = 16;

template <int NB, int T = (NB == 1 ? IDOT_SINGLE_T : IDOT_BATCH_T)>
hipError_t launch_idot(int waves, int count, int M, const uint8_t *const *Q, int64_t ldq,
                       const uint16_t *const *S, int64_t lds, const float *const *x,
                       float *const *y, hipStream_t s) {
    const dim3 grid((M + 8 * T - 1) / (8 * T), count);
    PackedPtrs<NB> p;
    for (int b = 0; b < NB; ++b) {
        const int i = b < count ? b : 0;
        p.Q[b] = Q[i];
        p.S[b] = S[i];
        p.x[b] = x[i];
        p.y[b] = y[i];
    }
    switch (waves) {
    case 1: return launch(gemv_q2_idot<1, T, NB>, grid, dim3(64), s, M, ldq, lds, p);
    case 2: return launch(gemv_q2_idot<2, T, NB>, grid, dim3(128), s, M, ldq, lds, p);
    case 3: return launch(gemv_q2_idot<3, T, NB>, grid, dim3(192), s, M, ldq, lds, p);
    case 4: return launch(gemv_q2_idot<4, T, NB>, grid, dim3(256), s, M, ldq, lds, p);
    default: return launch(gemv_q2_idot<6, T, NB>, grid, dim3(384), s, M, ldq, lds, p);
    }
}

// The row sums of sliced rows: y_b[r] = sum over slices s, in slice order,
// of part[(b * slices + s) * M + r].
template <int NB>
struct OutPtrs {
    float *y[NB];
};

template <int NB>
__global__ __launch_bounds__(256) void gemv_slices_sum(int M, int slices,
                                                       const float *__restrict__ part,
                                                       OutPtrs<NB> out) {
    const int b = (int)blockIdx.y;
    const int r = (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (r >= M) return;
    const float *p = part + (size_t)b * slices * M + r;
    // the loads of 8 slices at a time go out together, then the adds in order
    float v = 0.f;
    for (int q0 = 0; q0 < slices; q0 += 8) {
        float t[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) t[q] = q0 + q < slices ? p[(size_t)(q0 + q) * M] : 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (q0 + q < slices) v = q0 + q == 0 ? t[q] : v + t[q];
    }
    out.y[b][r] = v;
}

// Slices per row for this batch (sliced_count), or 0 where the integer-dot
// kernel's conditions fail on a slice: 16-byte aligned code rows, scale rows
// (lds a multiple of 8) and x, byte offsets within 31 bits.
inline int sliced_slices(int count, int M, int K, const uint8_t *const *Q, int64_t ldq,
                         const uint16_t *const *S, int64_t lds, const float *const *x) {
    const int n = (int)sliced_count(count, M, K);
    if (n == 0 || ldq % 16 != 0 || lds % 8 != 0) return 0;
    if ((int64_t)M * ldq >= (int64_t(1) << 31) || (int64_t)M * lds * 2 >= (int64_t(1) << 31))
        return 0;
    for (int i = 0; i < count; ++i)
        if (reinterpret_cast<uintptr_t>(Q[i]) % 16 != 0 ||
            reinterpret_cast<uintptr_t>(S[i]) % 16 != 0 ||
            reinterpret_cast<uintptr_t>(x[i]) % 16 != 0)
            return 0;
    return n;
}

// count <= PACKED_MAX_BATCH products, part holding count * slices * M floats.
hipError_t launch_sliced(int slices, int count, int M, const uint8_t *const *Q, int64_t ldq,
                         const uint16_t *const *S, int64_t lds, const float *const *x,
                         float *const *y, float *part, hipStream_t s) {
    // 8 steps (64 rows) per workgroup: 1.085 us per product at 40 x 1,536 x
    // 12,288, against 1.099 with 16 steps, 1.085-1.090 with 24 and 1.211
    // with 32 (fewer waves per SIMD fit)
    constexpr int NB = PACKED_MAX_BATCH, T = 8, W = SLICE_K / 512;
    PackedPtrs<NB> p;
    OutPtrs<NB> o;
    for (int b = 0; b < NB; ++b) {
        const int i = b < count ? b : 0;
        p.Q[b] = Q[i];
        p.S[b] = S[i];
        p.x[b] = x[i];
        p.y[b] = part + (size_t)i * slices * M;
        o.y[b] = y[i];
    }
    const dim3 grid((M + 8 * T - 1) / (8 * T), slices, count);
    hipError_t e = launch(gemv_q2_idot<W, T, NB, true>, grid, dim3(64 * W), s, M, ldq, lds, p);
    if (e != hipSuccess) return e;
    return launch(gemv_slices_sum<NB>, dim3((M + 255) / 256, count), dim3(256), s, M, slices,
                  (const float *)part, o);
}

// Rows split 32 ways unless the rows are long and few: at K >= 6,144 (each
// of 256 lanes then holds at least one live unit per pass in two of its
// three slots) with fewer rows than 32-way groups of one product would need
// to fill the chip, the row is split over the whole workgroup.
inline bool deep_split(int M, int K) { return K >= 6144 && M < 12288; }

template <int BITS, int NB>
hipError_t launch_split(int count, int M, int K, const uint8_t *const *Q, int64_t ldq,
                        const uint16_t *const *S, int64_t lds, const float *const *x,
                        float *const *y, hipStream_t s) {
    if constexpr (BITS == 2 && NB > 1) {
        const int waves = idot_waves(count, M, K, Q, ldq, S, lds, x);
        if (waves) return launch_idot<NB>(waves, count, M, Q, ldq, S, lds, x, y, s);
    }
    const int cpr = flat_cpr<BITS>(count, M, K, Q, ldq, lds, x);
    if (cpr) return launch_flat<BITS, NB>(count, M, cpr, Q, ldq, S, lds, x, y, s);
    return deep_split(M, K)
               ? launch_chunk<BITS, THREADS, NB>(count, M, K, Q, ldq, S, lds, x, y, s)
               : launch_chunk<BITS, 32, NB>(count, M, K, Q, ldq, S, lds, x, y, s);
}

template <int BITS>
hipError_t launch_batch(int count, int M, int K, const uint8_t *const *Q, int64_t ldq,
                        const uint16_t *const *S, int64_t lds, const float *const *x,
                        float *const *y, float *ws, hipStream_t s) {
    if (BITS == 2 && ws != nullptr) {
        const int slices = sliced_slices(count, M, K, Q, ldq, S, lds, x);
        if (slices) {
            // the workspace holds one launch's partial sums and is reused by
            // the next launch, which the stream orders after the sums
            for (int b0 = 0; b0 < count; b0 += PACKED_MAX_BATCH) {
                const int n = count - b0 < PACKED_MAX_BATCH ? count - b0 : PACKED_MAX_BATCH;
                const hipError_t e = launch_sliced(slices, n, M, Q + b0, ldq, S + b0, lds, x + b0,
                                                   y + b0, ws, s);
                if (e != hipSuccess) return e;
            }
            return hipSuccess;
        }
    }
    if (count == 1) return launch_split<BITS, 1>(1, M, K, Q, ldq, S, lds, x, y, s);
    // Up to PACKED_MAX_BATCH products per launch (their pointers travel in
    // the kernel arguments); larger batches take several launches in order.
    for (int b0 = 0; b0 < count; b0 += PACKED_MAX_BATCH) {
        const int n = count - b0 < PACKED_MAX_BATCH ? count - b0 : PACKED_MAX_BATCH;
        const hipError_t e = launch_split<BITS, PACKED_MAX_BATCH>(n, M, K, Q + b0, ldq, S + b0,
                                                                  lds, x + b0, y + b0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_gemv_q2(int count, int M, int K, const uint8_t *const *Q, int64_t ldq,
                          const uint16_t *const *S, int64_t lds, const float *const *x,
                          float *const *y, float *ws, hipStream_t s) {
    return launch_batch<2>(count, M, K, Q, ldq, S, lds, x, y, ws, s);
}

hipError_t launch_gemv_q4(int count, int M, int K, const uint8_t *const *Q, int64_t ldq,
                          const uint16_t *const *S, int64_t lds, const float *const *x,
                          float *const *y, hipStream_t s) {
    return launch_batch<4>(count, M, K, Q, ldq, S, lds, x, y, nullptr, s);
}

}  // namespace gg
