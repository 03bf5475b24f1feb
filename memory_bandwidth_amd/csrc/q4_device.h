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

// Sum over the 8 lanes of each half of a DPP row: the quad sums, then
// row_half_mirror pairs the two quads.
__device__ __forceinline__ float row8_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
             0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
             0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
             0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    return v;
}

// Sum over aligned groups of LPR lanes (8, 16, 32 or 64); every lane of a
// group gets its group's sum.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (LPR == 8) return row8_sum(v);
    v = row16_sum(v);
    if constexpr (LPR >= 32) v += __shfl_xor(v, 16);
    if constexpr (LPR >= 64) v += __shfl_xor(v, 32);
    return v;
}

// v_permlane32_swap_b32 a, b (gfx950): lanes 32..63 of a trade places with
// lanes 0..31 of b.  Written as inline asm because the compiler builtin for
// it returns the first result in both slots.  The s_nop covers the hazard
// between a VALU write of either operand and the permute reading it.
__device__ __forceinline__ void permlane32_swap(float &a, float &b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// v_permlane16_swap_b32 a, b (gfx950): the odd 16-lane rows of a trade
// places with the even 16-lane rows of b.
__device__ __forceinline__ void permlane16_swap(float &a, float &b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// Transposing reduction of R per-lane partial sums (R in 1, 2, 4, 8) over all
// 64 lanes.  Each swap-and-add halves the lanes a row spans while packing two
// rows into one register: 4 rows cost 3 swaps, 3 adds and 4 DPP steps in
// total, where reducing them one by one costs 6 steps each.
// out[q] (q < (R + 3) / 4) holds, in every lane of 16-lane row h = lane >> 4,
// the full sum of row reduced_row<R>(q, h).
template <int R>
__device__ __forceinline__ void wave_reduce_rows(float (&v)[R], float (&out)[(R + 3) / 4]) {
    static_assert(R == 1 || R == 2 || R == 4 || R == 8, "R must be 1, 2, 4 or 8");
    if constexpr (R == 1) {
        float a = v[0], b = v[0];
        permlane32_swap(a, b);
        float s = a + b, t = s;
        permlane16_swap(s, t);
        out[0] = row16_sum(s + t);
    } else if constexpr (R == 2) {
        float a = v[0], b = v[1];
        permlane32_swap(a, b);
        float s = a + b, t = s;
        permlane16_swap(s, t);
        out[0] = row16_sum(s + t);
    } else {
#pragma unroll
        for (int q = 0; q < R / 4; ++q) {
            float a0 = v[4 * q], b0 = v[4 * q + 1], a1 = v[4 * q + 2], b1 = v[4 * q + 3];
            permlane32_swap(a0, b0);
            permlane32_swap(a1, b1);
            float s0 = a0 + b0, s1 = a1 + b1;
            permlane16_swap(s0, s1);
            out[q] = row16_sum(s0 + s1);
        }
    }
}

// Row (0 .. R-1) whose sum wave_reduce_rows left in out[q] on 16-lane row h.
template <int R>
__device__ __forceinline__ int reduced_row(int q, int h) {
    if constexpr (R == 1) return 0;
    else if constexpr (R == 2) return h >> 1;
    else return 4 * q + ((h & 1) << 1) + (h >> 1);
}

}  // namespace q4
