// Device-side helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace q4 {

// Sum over the 16 lanes of a DPP row; every lane of the row gets the sum.
// quad_perm [1,0,3,2] and [2,3,0,1] sum each quad, row_half_mirror pairs
// the two quads of each half-row, row_mirror pairs the two half-rows.
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
             0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
             0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
             0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
             0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    return v;
}

// Sum over aligned groups of LPR lanes (16, 32 or 64); every lane of a group
// gets its group's sum.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    v = row16_sum(v);
    if constexpr (LPR >= 32) v += __shfl_xor(v, 16);
    if constexpr (LPR >= 64) v += __shfl_xor(v, 32);
    return v;
}

}  // namespace q4
