// wave.hpp -- cross-lane sums inside a wave64, for the matrix-vector kernels.
//
// The row sums of a split dot product are taken in registers with DPP lane
// shuffles (within each 16-lane DPP row) and ds_swizzle (across the two rows
// of a 32-lane half), so no LDS storage, barrier or atomic is involved and
// the reduction tree is fixed: results do not depend on timing.
#pragma once
#include <hip/hip_runtime.h>

namespace gg {

// gfx9 DPP controls.
constexpr int DPP_QUAD_XOR1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;   // lane i <- lane 15-i within a row
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane i <- lane 7-i within 8

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(
        0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over each 16-lane DPP row; every lane of the row receives the sum.
// Order: pairs, then quads, then halves of 8, then the two 8-lane halves.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<DPP_QUAD_XOR1>(v);
    v += dpp<DPP_QUAD_XOR2>(v);
    v += dpp<DPP_ROW_HALF_MIRROR>(v);
    v += dpp<DPP_ROW_MIRROR>(v);
    return v;
}

// Sum over each 32-lane half of the wave; every lane of the half receives it.
__device__ __forceinline__ float half32_sum(float v) {
    v = row16_sum(v);
    // ds_swizzle bit mode: and_mask 0x1f, or_mask 0, xor_mask 0x10 (lane ^ 16)
    v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
    return v;
}

// Sum over the whole wave; every lane receives it.
__device__ __forceinline__ float wave64_sum(float v) {
    v = half32_sum(v);
    const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    return lo + hi;
}

}  // namespace gg
