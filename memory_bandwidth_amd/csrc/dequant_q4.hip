// dequant_q4.hip -- debug dequantiser for gfx950.
//
// For every (n, k): codes_out = q and w_out = (float)(q - z) * s, following
// gerbil "WGSL Kernel Reference", section 3 MatMulInt4 ("INT4 Packing",
// "Dequantization").  (q - z) needs 4 bits plus sign and a binary16 scale 11
// significant bits, so the fp32 product is exact and the output is unique.
// One thread handles one 32-bit word of codes (8 weights of one row, inside
// one group): two 16-byte stores of weights and one 8-byte store of codes.
#include "q4_common.h"

namespace {

constexpr int kBlock = 256;
constexpr int kMaxGrid = 16384;

__global__ __launch_bounds__(kBlock) void dequant_q4_kernel(
    const uint32_t *__restrict__ wq, const uint16_t *__restrict__ scales,
    const uint8_t *__restrict__ zeros, float *__restrict__ w_out, uint8_t *__restrict__ codes_out,
    int K, int gshift, size_t nwords) {
    const int wpr = K >> 3;                     // code words per row
    const int G = K >> (gshift + 5);
    const int ZB = (G + 1) >> 1;
    for (size_t idx = (size_t)blockIdx.x * kBlock + threadIdx.x; idx < nwords;
         idx += (size_t)gridDim.x * kBlock) {
        const size_t n = idx / wpr;
        const int k0 = (int)(idx - n * wpr) << 3;
        const int j = k0 >> (gshift + 5);
        const uint32_t word = wq[idx];
        const int z = (zeros[n * ZB + (j >> 1)] >> ((j & 1) << 2)) & 0xF;
        const float s = (float)__builtin_bit_cast(_Float16, scales[n * G + j]);
        const size_t o = n * K + k0;
        if (w_out) {
            float v[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) v[p] = (float)((int)((word >> (4 * p)) & 0xF) - z) * s;
            float4 *dst = reinterpret_cast<float4 *>(w_out + o);
            dst[0] = make_float4(v[0], v[1], v[2], v[3]);
            dst[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
        if (codes_out) {
            // byte p of the pair = code of element k0 + p
            const uint32_t lo = (word & 0xFu) | ((word >> 4) & 0xFu) << 8 |
                                ((word >> 8) & 0xFu) << 16 | ((word >> 12) & 0xFu) << 24;
            const uint32_t hi = ((word >> 16) & 0xFu) | ((word >> 20) & 0xFu) << 8 |
                                ((word >> 24) & 0xFu) << 16 | ((word >> 28) & 0xFu) << 24;
            *reinterpret_cast<uint2 *>(codes_out + o) = make_uint2(lo, hi);
        }
    }
}

}  // namespace

extern "C" int dequant_q4(const uint8_t *wq, const uint16_t *scales, const uint8_t *zeros,
                          float *w_out, uint8_t *codes_out, int N, int K, int group_size,
                          void *stream) {
    if (N < 0 || K <= 0 || (group_size != 32 && group_size != 128) || K < group_size ||
        K % group_size != 0)
        return Q4_EINVAL;
    if (N == 0) return Q4_OK;
    if (!wq || !scales || !zeros || (!w_out && !codes_out)) return Q4_ENULL;
    if (!q4::aligned(wq, 16) || !q4::aligned(scales, 2) || (w_out && !q4::aligned(w_out, 16)) ||
        (codes_out && !q4::aligned(codes_out, 8)))
        return Q4_EALIGN;
    const int dev = q4::check_device();
    if (dev != Q4_OK) return dev;
    const size_t nwords = (size_t)N * (K / 8);
    size_t blocks = (nwords + kBlock - 1) / kBlock;
    if (blocks > (size_t)kMaxGrid) blocks = kMaxGrid;
    hipLaunchKernelGGL(dequant_q4_kernel, dim3((unsigned)blocks), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), reinterpret_cast<const uint32_t *>(wq),
                       scales, zeros, w_out, codes_out, K, group_size == 32 ? 0 : 2, nwords);
    return q4::launch_status();
}
