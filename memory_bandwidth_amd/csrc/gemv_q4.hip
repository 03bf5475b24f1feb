// gemv_q4.hip -- int4 decode GEMV, y[M,N] = x[M,K] . dequant(W_q[N,K])^T, for gfx950.
//
// What is computed follows gerbil "WGSL Kernel Reference", section 3 MatMulInt4
// ("Computes", "INT4 Packing", "Dequantization"), with the weights stored
// N-major: every output row n reads its own contiguous K/2 bytes of codes.
//
// Mapping onto CDNA4 (no MFMA: at M <= 8 this is a streaming dot product):
//   * A 16-byte chunk holds 32 consecutive codes of one row and lies inside
//     one quantisation group (g = 32: exactly one group; g = 128: a quarter).
//     Lanes take consecutive chunks, so one global_load_dwordx4 per wavefront
//     reads 1 KiB contiguous.
//   * A wavefront owns R row slots.  LPR lanes share one row (LPR = 64 for
//     long rows; 32 or 16 when a row has fewer chunks than a wavefront has
//     lanes, so two or four rows share one load instruction).
//   * S wavefronts of a workgroup may split one row block's K range; their
//     partial sums meet in LDS (the only cross-wavefront combine).
//   * x is staged through LDS once per workgroup, in segments when M*K*4
//     exceeds the LDS budget.  Its 16-byte slots are XOR-swizzled by chunk
//     index so that eight consecutive lanes reading the same slot of their
//     own chunks hit eight different bank groups.
//   * Dequantisation stays exact and cheap: a code q in bits 0-3 of a half
//     word OR 0x6400 is the binary16 value 1024 + q, and q in bits 4-7 gives
//     1024 + 16q, so one v_and_or_b32 yields two weights and one
//     v_pk_add_f16 subtracting (1024 + z) or (1024 + 16z) gives the exact
//     integers (q - z) or 16(q - z).  v_fma_mix_f32 multiplies the binary16
//     value by the fp32 x and accumulates in fp32.  The high-nibble weights
//     go into their own accumulator, scaled back by 1/16 (exact) with the
//     group scale once per chunk.  The zero point is never factored out of
//     the sum, so q == z gives exactly zero.
//   * Per-lane partial sums are reduced across the LPR lanes of a row with
//     DPP row operations and two cross-row shuffles.
#include "q4_common.h"
#include "q4_device.h"

#include <algorithm>
#include <mutex>
#include <shared_mutex>

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;                     // wavefronts per workgroup
constexpr int kBlock = kWaves * q4::kWave;
constexpr int kLdsBytes = 64 * 1024;          // dynamic LDS budget per workgroup

// Row slots per wavefront as a function of M: keeps the per-lane register
// footprint (codes in flight + x slice + accumulators) near 128 VGPRs.
constexpr int row_slots(int M) { return M == 1 ? 4 : (M <= 4 ? 2 : 1); }

// (a & m) | o in one VALU op; gfx9 VOP3 takes no literal, so the compiler
// would otherwise split it into v_and_b32 + v_or_b32.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(o));
    return r;
}

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// Eight weights of one 32-bit word of codes against x values xv[m][0..7].
// Word bits 4p..4p+3 hold element p (p = 0..7).
template <int M>
__device__ __forceinline__ void dot_word(uint32_t wd, half2_t z1, half2_t z16, uint32_t magic,
                                         const float (&xv)[M][8], float (&ae)[M],
                                         float (&ao)[M]) {
    const uint32_t w8 = wd >> 8;
    const half2_t d0 = as_h2(and_or(wd, 0x000F000Fu, magic)) - z1;   // elements 0, 4
    const half2_t d1 = as_h2(and_or(wd, 0x00F000F0u, magic)) - z16;  // 16 x elements 1, 5
    const half2_t d2 = as_h2(and_or(w8, 0x000F000Fu, magic)) - z1;   // elements 2, 6
    const half2_t d3 = as_h2(and_or(w8, 0x00F000F0u, magic)) - z16;  // 16 x elements 3, 7
#pragma unroll
    for (int m = 0; m < M; ++m) {
        ae[m] = __builtin_fmaf((float)d0.x, xv[m][0], ae[m]);
        ao[m] = __builtin_fmaf((float)d1.x, xv[m][1], ao[m]);
        ae[m] = __builtin_fmaf((float)d2.x, xv[m][2], ae[m]);
        ao[m] = __builtin_fmaf((float)d3.x, xv[m][3], ao[m]);
        ae[m] = __builtin_fmaf((float)d0.y, xv[m][4], ae[m]);
        ao[m] = __builtin_fmaf((float)d1.y, xv[m][5], ao[m]);
        ae[m] = __builtin_fmaf((float)d2.y, xv[m][6], ae[m]);
        ao[m] = __builtin_fmaf((float)d3.y, xv[m][7], ao[m]);
    }
}

// x staging batch: float4 per thread per activation row fetched ahead of the
// weight loads (all of x for M = 1 and K <= 4096).
constexpr int x_batch(int M) { return M == 1 ? 4 : (M == 2 ? 2 : 1); }

// LDS layout of the x segment: chunk c of activation row m (32 floats) at
// float offset (m * segC + c) * kXStride.  The 4-float pad makes the stride
// 144 bytes, so the 16 lanes of one LDS pass reading the same 16-byte slot of
// 16 consecutive chunks land in 16 distinct 4-bank groups.
constexpr int kXStride = 36;

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));   // a plain vector, never an aggregate copy

// Buffer resource for a raw (untyped) byte range on gfx9: base, no stride,
// num_records bytes (reads past it return zero), default dword-3 format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// The bytes from a wavefront's first row to the end of an array, for a
// resource's 32-bit range field: formed in 64 bits and clamped.  The
// wavefront itself only reads its own rows (at most a few rows past the
// base, well inside 4 GiB for any K that validate() accepts), so the clamp
// never cuts off a byte it reads.
__device__ __forceinline__ uint32_t span32(uint64_t rows, uint64_t row_bytes) {
    const uint64_t b = rows * row_bytes;
    return b > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)b;
}

// Cache-policy bits of a buffer load: non-temporal, for the weight stream
// that is read once.
constexpr int kNonTemporal = 2;

// Stores one output.  With epi set the GEMV is the gate projection of a
// SwiGLU block: y already holds the up projection u, and silu(v) * u, with
// silu(v) = v / (1 + e^-v), replaces it.
__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

__device__ __forceinline__ void store_y(float *y, size_t i, float v, int epi) {
    if (epi) v = silu(v) * y[i];
    y[i] = v;
}

// M: activation rows.  LPR: lanes per output row.  JP: chunk positions per
// lane per segment (a lane's chunks are LPR apart).  R: row slots per wave.
//
// Addressing: pointers are wave-uniform bases (SGPRs) plus one 32-bit
// per-lane offset shared by all rows of the wave when LPR = 64.
template <int M, int LPR, int JP, int R>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 4))) void gemv_q4_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ wq,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    float *__restrict__ y, int N, int K, int gshift, int S, int seg_chunks, int epi) {
    constexpr int RG = q4::kWave / LPR;   // rows sharing one load instruction
    constexpr int RPW = R * RG;           // output rows per wavefront
    constexpr int XB = x_batch(M);
    extern __shared__ float lds[];
    float *xs = lds;                                        // [M][segC][kXStride]
    float *comb = lds + M * seg_chunks * kXStride;          // [waves][RPW][M]

    const int C = K >> 5;              // chunks per row
    const int G = K >> (gshift + 5);   // groups per row
    const int ZB = (G + 1) >> 1;       // zero-point bytes per row
    const int RB = K >> 1;             // code bytes per row
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int rb = wave / S;           // row block of this wavefront within the workgroup
    const int ks = wave - rb * S;      // K-split index
    const int row_first = (blockIdx.x * (kWaves / S) + rb) * RPW;   // may be >= N
    const int row_base = min(row_first, N - 1);
    const int rgl = RG == 1 ? 0 : lane / LPR;
    const int li = RG == 1 ? lane : lane % LPR;
    const uint32_t magic = 0x64006400u;

    // Wave-uniform buffer resources starting at the wave's first row; per-row
    // byte offsets are uniform (SGPR soffset) when RG == 1 and per-lane
    // otherwise.  Rows past N re-read row N-1 and are not stored.
    const uint32_t rows_left = (uint32_t)(N - row_base);
    const __amdgpu_buffer_rsrc_t wq_r = raw_rsrc(wq + (size_t)row_base * RB, span32(rows_left, RB));
    const __amdgpu_buffer_rsrc_t sc_r = raw_rsrc(scales + (size_t)row_base * G, span32(rows_left, 2u * G));
    const __amdgpu_buffer_rsrc_t zp_r = raw_rsrc(zeros + (size_t)row_base * ZB, span32(rows_left, ZB));
    uint32_t roff[R], soff[R], zoff[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t rr = (uint32_t)(min(row_first + r * RG + rgl, N - 1) - row_base);
        roff[r] = rr * (uint32_t)RB;
        soff[r] = rr * (uint32_t)G * 2u;
        zoff[r] = rr * (uint32_t)ZB;
    }

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

    for (int seg0 = 0; seg0 < C; seg0 += seg_chunks) {
        const int segC = min(seg_chunks, C - seg0);
        const int part = (segC + S - 1) / S;
        const int lo = seg0 + ks * part;
        const int hi = min(seg0 + segC, lo + part);
        const int nx4 = segC * 8;                       // float4 per x row in this segment
        const float *xseg = x + seg0 * 32;

        // x segment, first batch: global -> registers ahead of the weight
        // loads, so that waiting for x does not wait for the weights (vmcnt
        // retires loads in issue order).  Guards are uniform except in a
        // batch that straddles the end of the segment.
        f32x4_t xr[M][XB];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int t = 0; t < XB; ++t)   // indexes past the segment re-read its last float4
                xr[m][t] = reinterpret_cast<const f32x4_t *>(xseg + (size_t)m * K)[min(t * kBlock + tid, nx4 - 1)];
        // Keep the x loads ahead of the weight loads in issue order.
        __builtin_amdgcn_sched_barrier(0);

        // Weight stream: every load of the lane is issued before any
        // arithmetic, the small scale and zero-point loads first, then the
        // codes in the order they are consumed.  Loads retire in issue order
        // (vmcnt), so with the metadata ahead the arithmetic on the first
        // chunk waits for that chunk only, not for the whole wave's data.
        // Positions past this wave's range re-read its last chunk (always in
        // bounds) and are skipped below.
        uint4 w[JP][R];
        uint32_t sr[JP][R];
        uint32_t zr[JP][R];
        const int clast = max(lo, hi - 1) < seg0 + segC ? max(lo, hi - 1) : seg0 + segC - 1;
#pragma unroll
        for (int j = 0; j < JP; ++j) {
            const uint32_t gi = (uint32_t)min(lo + li + j * LPR, clast) >> gshift;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                sr[j][r] = __builtin_amdgcn_raw_buffer_load_b16(
                    sc_r, RG == 1 ? gi * 2u : gi * 2u + soff[r], RG == 1 ? soff[r] : 0u, 0);
                zr[j][r] = __builtin_amdgcn_raw_buffer_load_b8(
                    zp_r, RG == 1 ? (gi >> 1) : (gi >> 1) + zoff[r], RG == 1 ? zoff[r] : 0u, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < JP; ++j) {
            const uint32_t coff = (uint32_t)min(lo + li + j * LPR, clast) * 16u;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                // RG == 1: row offset in soffset (SGPR), chunk offset in voffset.
                const uint32_t vw = RG == 1 ? coff : coff + roff[r];
                const uint32_t sw = RG == 1 ? roff[r] : 0u;
                const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(wq_r, vw, sw, kNonTemporal);
                w[j][r] = make_uint4(t.x, t.y, t.z, t.w);
            }
        }

        // Unconditional stores (lanes past the segment rewrite its last float4
        // with the value it already holds): a guarded store would let the
        // compiler sink the x loads behind the weight loads.
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int t = 0; t < XB; ++t) {
                const int i = min(t * kBlock + tid, nx4 - 1);
                *reinterpret_cast<f32x4_t *>(xs + (m * segC + (i >> 3)) * kXStride + (i & 7) * 4) = xr[m][t];
            }
        for (int m = 0; m < M; ++m)
            for (int i = XB * kBlock + tid; i < nx4; i += kBlock)
                *reinterpret_cast<f32x4_t *>(xs + (m * segC + (i >> 3)) * kXStride + (i & 7) * 4) =
                    reinterpret_cast<const f32x4_t *>(xseg + (size_t)m * K)[i];
        __syncthreads();                                // x segment visible

#pragma unroll
        for (int j = 0; j < JP; ++j) {
            const int c = lo + li + j * LPR;
            if (c < hi) {
                const float *xc = xs + (c - seg0) * kXStride;
                const uint32_t gi = (uint32_t)c >> gshift;
                const uint32_t zsh = (gi & 1u) << 2;
                half2_t z1[R], z16[R];
                float ae[R][M], ao[R][M];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t z = (zr[j][r] >> zsh) & 0xFu;
                    z1[r] = as_h2(z * 0x00010001u + magic);
                    z16[r] = as_h2(z * 0x00100010u + magic);
#pragma unroll
                    for (int m = 0; m < M; ++m) ae[r][m] = ao[r][m] = 0.f;
                }
#pragma unroll
                for (int wd = 0; wd < 4; ++wd) {
                    float xv[M][8];
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const float *base = xc + m * segC * kXStride + wd * 8;
                        const float4 a = *reinterpret_cast<const float4 *>(base);
                        const float4 b = *reinterpret_cast<const float4 *>(base + 4);
                        xv[m][0] = a.x; xv[m][1] = a.y; xv[m][2] = a.z; xv[m][3] = a.w;
                        xv[m][4] = b.x; xv[m][5] = b.y; xv[m][6] = b.z; xv[m][7] = b.w;
                    }
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const uint32_t word = wd == 0 ? w[j][r].x : wd == 1 ? w[j][r].y
                                            : wd == 2 ? w[j][r].z : w[j][r].w;
                        dot_word<M>(word, z1[r], z16[r], magic, xv, ae[r], ao[r]);
                    }
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sr[j][r]);
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        acc[r][m] = __builtin_fmaf(s, __builtin_fmaf(ao[r][m], 0.0625f, ae[r][m]),
                                                   acc[r][m]);
                }
            }
        }
        if (seg0 + seg_chunks < C) __syncthreads();    // x segment fully read before the next overwrites it
    }

    if constexpr (LPR == 64) {
        // One transposing reduction for all R rows; on 16-lane row h, out[m][q]
        // holds the sum of row slot reduced_row<R>(q, h).  Lane 16h stores it.
        constexpr int NQ = (R + 3) / 4;
        float out[M][NQ];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float v[R];
#pragma unroll
            for (int r = 0; r < R; ++r) v[r] = acc[r][m];
            q4::wave_reduce_rows<R>(v, out[m]);
        }
        const int h = lane >> 4;
        const bool writer = (lane & 15) == 0 && (R >= 4 || (h & (R == 2 ? 1 : 3)) == 0);
        if (S == 1) {
            if (writer) {
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const int row = row_first + q4::reduced_row<R>(q, h);
                    if (row < N)
#pragma unroll
                        for (int m = 0; m < M; ++m) store_y(y, (size_t)m * N + row, out[m][q], epi);
                }
            }
            return;
        }
        if (writer) {
#pragma unroll
            for (int q = 0; q < NQ; ++q)
#pragma unroll
                for (int m = 0; m < M; ++m)
                    comb[(wave * RPW + q4::reduced_row<R>(q, h)) * M + m] = out[m][q];
        }
        __syncthreads();
        if (ks == 0 && writer) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int rs = q4::reduced_row<R>(q, h);
                const int row = row_first + rs;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    float v = out[m][q];
                    for (int t = 1; t < S; ++t) v += comb[((wave + t) * RPW + rs) * M + m];
                    if (row < N) store_y(y, (size_t)m * N + row, v, epi);
                }
            }
        }
    } else {
        // Rows narrower than a wavefront: reduce each over its LPR lanes.
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = q4::group_sum<LPR>(acc[r][m]);
        if (S == 1) {
            if (li == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int row = row_first + r * RG + rgl;
                    if (row < N)
#pragma unroll
                        for (int m = 0; m < M; ++m) store_y(y, (size_t)m * N + row, acc[r][m], epi);
                }
            }
            return;
        }
        if (li == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m) comb[(wave * RPW + r * RG + rgl) * M + m] = acc[r][m];
        }
        __syncthreads();
        if (ks == 0 && li == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int row = row_first + r * RG + rgl;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    float v = acc[r][m];
                    for (int t = 1; t < S; ++t) v += comb[((wave + t) * RPW + r * RG + rgl) * M + m];
                    if (row < N) store_y(y, (size_t)m * N + row, v, epi);
                }
            }
        }
    }
}

// ---------------------------------------------------------------- the integer path
//
// The (q - z) * x products are formed in integer arithmetic, eight per
// instruction, on x written in block fixed point.  With e the binary exponent
// of a 32-value chunk's largest |x| (|x| < 2^e) and sh = 26 - e, each element
// becomes X = rint(x * 2^sh), |X| <= 2^26, and an exact residual
// r = x * 2^sh - X, |r| <= 1/2, so that x = (X + r) * 2^-sh exactly.
// X is held as seven signed 4-bit digits, X = sum_l d_l 16^l with d_l in
// [-8, 7] (the nibbles of (X + 0x8888888) ^ 0x8888888), and the digits of 8
// consecutive x values are transposed into one 32-bit word per digit, so that
// v_dot8_i32_i4 of such a word against a word of 8 codes, each read as q - 8
// in [-8, 7] by one XOR with 0x88888888, sums the 8 products of one digit.
// Then
//     sum_k (q_k - z) X_k = sum_l 16^l sum_k (q_k - 8) d_l[k] + (8 - z) sum_k X_k
// exactly: digits 0-3 (with (8 - z) times the low 16 bits of SX = sum X) and
// digits 4-6 (with (8 - z) times SX >> 16) are each combined in int32, below
// 2^24 and 2^20 in magnitude, so both convert to fp32 exactly and one fused
// multiply-add joins them.  q == z still gives exactly 0.
//
// X alone carries x to within |r| <= 1/2 unit, a small fraction of
// |x * 2^sh| except for values far below the chunk's largest.  An element
// whose residual exceeds 2^-14 of |x * 2^sh| (one more than about 2^12 below
// the chunk's largest) is flagged, and (q - z) * r is added for it in fp32
// from its exact residual, so every product (q - z) * x is carried to within
// 2^-14 of itself whatever the spread of x inside a chunk.  Then a multiply
// by 2^-sh and the group scale accumulate into the row's fp32 sum.

// Record of one chunk of x in LDS, kIW dwords:
//   [4d + w]  digit plane d (0..6) of code word w (0..3)
//   [28]      SX = sum of X (|SX| <= 2^31 - 32)
//   [29]      2^-sh as fp32 (NaN when the chunk holds Inf or NaN)
//   [30]      flags: bit k set when element k takes the fp32 residual correction
//   [31]      residual slots: bits 0-10 for elements 0-15, bits 11-21 for
//             16-31 (kNoSlot: not stored, recomputed from x), bits 23-31 sh + 128
//   [32..35]  unused: 144 bytes, an odd number of 16-byte slots, so that the
//             16-byte reads of consecutive lanes (consecutive chunks) fall in
//             distinct LDS banks (a 128-byte stride measured 16% slower)
// A slot holds the 16 fp32 residuals of one half chunk.
constexpr int kPlanes = 7;
constexpr int kIW = 36;
constexpr int kTail = 4 * kPlanes;
constexpr uint32_t kNoSlot = 0x7FF;
constexpr int kIntVPT = 16;                         // x values a lane pair's lanes convert each
constexpr int kIntTPC = 32 / kIntVPT;               // lanes per chunk of x
constexpr float kRhoInv = 16384.0f;                 // residuals above 2^-14 of |x * 2^sh| are flagged

// 8x8 transpose of 4-bit fields: on return nibble p of a[l] is nibble l of
// the input a[p].  Three butterfly stages: nibbles between neighbouring
// words, bytes between words two apart, half-words between words four apart.
__device__ __forceinline__ void transpose_nibbles(uint32_t (&a)[8]) {
#pragma unroll
    for (int p = 0; p < 8; p += 2) {
        const uint32_t lo = a[p], hi = a[p + 1];
        a[p] = (lo & 0x0F0F0F0Fu) | ((hi << 4) & 0xF0F0F0F0u);
        a[p + 1] = ((lo >> 4) & 0x0F0F0F0Fu) | (hi & 0xF0F0F0F0u);
    }
#pragma unroll
    for (int p = 0; p < 8; p += (p & 1) ? 3 : 1) {      // pairs (0,2) (1,3) (4,6) (5,7)
        const uint32_t u = a[p], v = a[p + 2];
        a[p] = __builtin_amdgcn_perm(v, u, 0x06020400u);
        a[p + 2] = __builtin_amdgcn_perm(v, u, 0x07030501u);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t u = a[p], v = a[p + 4];
        a[p] = __builtin_amdgcn_perm(v, u, 0x05040100u);
        a[p + 4] = __builtin_amdgcn_perm(v, u, 0x07060302u);
    }
}

// DPP reads within a quad of lanes: the value of lane ^ 1, lane ^ 2, lane ^ 3.
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
}
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
}
__device__ __forceinline__ uint32_t dpp_xor3(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x1B, 0xF, 0xF, false);   // quad_perm [3,2,1,0]
}

// Converts one chunk of x to the digit planes, SX and 2^-sh of its LDS
// record and returns sh.  The chunk's 32 values are held by 32 / V
// consecutive lanes (a pair or a quad), V each in order; `part` is the lane's
// index among them.  Every lane of the wavefront must call it (the lanes of a
// chunk exchange partial results by DPP); only lanes with `store` set write.
template <int V>
__device__ __forceinline__ int store_int_chunk(const f32x4_t (&xr)[V / 4], int part, bool store, uint32_t *rec) {
    static_assert(V == 8 || V == 16, "a chunk is converted by a lane pair or a lane quad");
    float v[V];
#pragma unroll
    for (int i = 0; i < V / 4; ++i) {
        v[4 * i] = xr[i].x; v[4 * i + 1] = xr[i].y; v[4 * i + 2] = xr[i].z; v[4 * i + 3] = xr[i].w;
    }
    // NaN-propagating maximum (v_maximum3_f32), so a NaN anywhere reaches m
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) m = __builtin_elementwise_maximum(m, __builtin_fabsf(v[i]));
    m = __builtin_elementwise_maximum(m, __builtin_bit_cast(float, dpp_xor1(__builtin_bit_cast(uint32_t, m))));
    if (V == 8)
        m = __builtin_elementwise_maximum(m, __builtin_bit_cast(float, dpp_xor2(__builtin_bit_cast(uint32_t, m))));
    const int sh = 26 - __builtin_amdgcn_frexp_expf(m);   // |x| * 2^sh < 2^26 (m == 0: sh = 26)
    uint32_t dg[V];
    uint32_t sx = 0;                                       // sum of X, two's complement
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const uint32_t X = (uint32_t)(int)__builtin_rintf(__builtin_amdgcn_ldexpf(v[i], sh));
        sx += X;
        dg[i] = (X + 0x8888888u) ^ 0x8888888u;
    }
    sx += dpp_xor1(sx);
    if (V == 8) sx += dpp_xor2(sx);
    if (!store) return sh;
#pragma unroll
    for (int w = 0; w < V / 8; ++w) {
        uint32_t a[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) a[p] = dg[8 * w + p];
        transpose_nibbles(a);
#pragma unroll
        for (int d = 0; d < kPlanes; ++d) rec[4 * d + (V / 8) * part + w] = a[d];
    }
    if (part == 0) {
        // a chunk holding Inf or NaN gets a NaN scale, so its rows come out NaN
        const float scale = m <= 3.4028235e38f ? __builtin_amdgcn_ldexpf(1.0f, -sh) : m - m;
        rec[kTail] = sx;
        rec[kTail + 1] = __builtin_bit_cast(uint32_t, scale);
    }
    return sh;
}

// Flags the chunk's elements whose residual exceeds 2^-14 of |x * 2^sh| and
// stores the residuals of each half chunk holding a flag in a slot of
// `pool`: slot `dense_slot` (the half's own, for a lane quad: its lanes
// write 8 residuals each) when it is >= 0, else, for a lane pair, the next
// free one of `cap`, taken from the LDS counter `*next` (a half that finds
// the pool full keeps kNoSlot, and its residuals are recomputed from x where
// they are used).  Writes the record's flags and slots.  Every lane of the
// wavefront must call it, with the arguments of store_int_chunk and the sh
// it returned.
template <int V>
__device__ __forceinline__ void store_int_flags(const f32x4_t (&xr)[V / 4], int sh, int part, bool store,
                                                uint32_t *rec, float *pool, int dense_slot, uint32_t *next,
                                                uint32_t cap) {
    float r[V];
    uint32_t fl = 0;
#pragma unroll
    for (int i = V - 1; i >= 0; --i) {
        const float vs = __builtin_amdgcn_ldexpf(xr[i / 4][i % 4], sh);
        r[i] = vs - __builtin_rintf(vs);                   // exact
        fl = (fl << 1) | (__builtin_fabsf(r[i]) * kRhoInv > __builtin_fabsf(vs) ? 1u : 0u);
    }
    if constexpr (V == 16) {
        uint32_t slot = kNoSlot;
        if (store && fl) {
            const uint32_t s = dense_slot >= 0 ? (uint32_t)dense_slot : __hip_atomic_fetch_add(
                next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (s < cap) {
                slot = s;
                f32x4_t *dst = reinterpret_cast<f32x4_t *>(pool + (size_t)s * 16);
#pragma unroll
                for (int i = 0; i < V / 4; ++i) dst[i] = f32x4_t{r[4 * i], r[4 * i + 1], r[4 * i + 2], r[4 * i + 3]};
            }
        }
        const uint32_t pfl = dpp_xor1(fl), pslot = dpp_xor1(slot);
        if (store && part == 0) {
            rec[kTail + 2] = fl | (pfl << 16);
            rec[kTail + 3] = slot | (pslot << 11) | ((uint32_t)(sh + 128) << 23);
        }
    } else {
        // lane quad, dense slots only: lanes 2h and 2h + 1 hold half h
        const uint32_t f1 = dpp_xor1(fl), f2 = dpp_xor2(fl), f3 = dpp_xor3(fl);
        if (store && fl) {
            f32x4_t *dst = reinterpret_cast<f32x4_t *>(pool + (size_t)dense_slot * 16 + (part & 1) * 8);
            dst[0] = f32x4_t{r[0], r[1], r[2], r[3]};
            dst[1] = f32x4_t{r[4], r[5], r[6], r[7]};
        }
        if (store && part == 0) {
            rec[kTail + 2] = fl | (f1 << 8) | (f2 << 16) | (f3 << 24);
            rec[kTail + 3] = (uint32_t)dense_slot | ((uint32_t)(dense_slot + 1) << 11) | ((uint32_t)(sh + 128) << 23);
        }
    }
}

// Exact residual r = v * 2^sh - rint(v * 2^sh) of one x value (the same
// operations as the conversion, so the same value wherever it is formed).
__device__ __forceinline__ float int_residual(float v, int sh) {
    const float vs = __builtin_amdgcn_ldexpf(v, sh);
    return vs - __builtin_rintf(vs);
}

// Fields of a record's tail as the dot-product loops use them.
struct IntChunk {
    int sxl, sxh;      // SX = 65536 * sxh + sxl, 0 <= sxl < 65536
    float cscale;      // 2^-sh
    uint32_t flags, slots;
};

__device__ __forceinline__ IntChunk int_chunk_tail(const uint32_t *rec) {
    const u32x4_t t = *reinterpret_cast<const u32x4_t *>(rec + kTail);
    IntChunk c;
    c.sxl = (int)(t.x & 0xFFFFu);
    c.sxh = (int)t.x >> 16;
    const uint32_t scale_bits = t.y;   // copied out before the bit cast
    c.cscale = __builtin_bit_cast(float, scale_bits);
    c.flags = t.z;
    c.slots = t.w;
    return c;
}

// Sum of (q - z) * X over one chunk for one weight row, as fp32: 28 dot
// products of the row's four code words (XORed here with `xor_mask` to hold
// q - 8) against the seven digit planes, the zero-point term (8 - z) * SX
// entering as (8 - z) * sxl in digit 0 and (8 - z) * sxh in digit 4
// (weight 16^4 = 2^16); digits 0-3 and 4-6 each combined exactly in int32,
// then one fused multiply-add.
__device__ __forceinline__ float int_chunk_dot(const u32x4_t &w, const u32x4_t (&D)[kPlanes], int nz, int sxl,
                                               int sxh, uint32_t xor_mask) {
    int a[kPlanes];
    const uint32_t c0 = w.x ^ xor_mask;
#pragma unroll
    for (int d = 0; d < kPlanes; ++d) {
        if (d == 0) a[d] = __builtin_amdgcn_sdot8((int)c0, (int)D[d].x, __mul24(nz, sxl), false);
        else if (d == 4) a[d] = __builtin_amdgcn_sdot8((int)c0, (int)D[d].x, __mul24(nz, sxh), false);
        else asm("v_dot8_i32_i4 %0, %1, %2, 0" : "=v"(a[d]) : "v"(c0), "v"(D[d].x));
    }
#pragma unroll
    for (int wd = 1; wd < 4; ++wd) {
        const uint32_t cw = (wd == 1 ? w.y : wd == 2 ? w.z : w.w) ^ xor_mask;
#pragma unroll
        for (int d = 0; d < kPlanes; ++d) {
            const uint32_t dw = wd == 1 ? D[d].y : wd == 2 ? D[d].z : D[d].w;
            a[d] = __builtin_amdgcn_sdot8((int)cw, (int)dw, a[d], false);
        }
    }
    const int lo = a[0] + 16 * (a[1] + 16 * (a[2] + 16 * a[3]));   // |lo| < 2^24
    const int hi = a[4] + 16 * (a[5] + 16 * a[6]);                 // |hi| < 2^20
    return __builtin_fmaf(65536.0f, (float)hi, (float)lo);
}

// Code q (0..15) of element k (0..31) of a chunk's four code words; `xm` is
// the XOR the words already carry (0, or 0x88888888 when they hold q - 8).
__device__ __forceinline__ int chunk_code(const u32x4_t &w, uint32_t k, uint32_t xm) {
    const uint32_t lo = (k & 8u) ? w.y : w.x;
    const uint32_t hi = (k & 8u) ? w.w : w.z;
    const uint32_t word = ((k & 16u) ? hi : lo) ^ xm;
    return (int)__builtin_amdgcn_ubfe(word, (k & 7u) << 2, 4);
}

// W: wavefronts per workgroup.  JP: chunk positions per lane (a lane's chunks
// are 64 apart).  R: row slots per wavefront.  A workgroup owns rpg
// consecutive rows, split as evenly as possible over W / S row groups; the S
// wavefronts of a row group split its K range and meet in LDS.  MULTI: x has
// more chunks than one pass of the workgroup converts.  S and MULTI are
// template parameters so that the common case (S = 1, one pass) carries no
// division and no unused path.
// x values each converting lane takes in the one-row kernel: 16 (lane pairs
// per chunk) or 8 (lane quads, one code word's values per lane, every
// wavefront converting after issuing its weight loads: 8.25 against 7.82 us
// per 4096 -> 14336 launch, 10.98 against 10.05 at 14336 -> 4096).
constexpr int kM1XV = 16;

template <int W, int LPR, int JP, int R, int S, bool MULTI, bool SWI = false, int XV = kM1XV>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(1, 4))) void gemv_q4_int_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ wq,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    float *__restrict__ y, int N, int K, int gshift, int rpg, int epi,
    const uint8_t *__restrict__ wq2, const uint16_t *__restrict__ scales2,
    const uint8_t *__restrict__ zeros2) {
    static_assert(!SWI || S == 1, "the SwiGLU form has no K-split");
    extern __shared__ uint32_t ilds[];
    const int tid = threadIdx.x;
    // x first, before any address arithmetic: a CU returns loads in the
    // order they were issued, so x issued later would wait behind weight
    // loads.  The 32 / XV lanes from 32i / XV on load chunk i, XV values
    // each; reads past K return 0.  Wavefronts whose chunks all lie past the
    // end of x (the non-stagers) skip the conversion.
    constexpr int XT = 32 / XV;                        // lanes per chunk of x
    constexpr int XWC = 64 / XT;                       // chunks one wavefront converts per pass
    constexpr int kPass = W * XWC;                     // chunks converted per workgroup pass
    const int C = K >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool stager = wave * XWC < C;
    const int hc = tid / XT, xpart = tid % XT;
    const int xslot = XV == 16 ? xpart : xpart >> 1;   // half chunk of the lane's values
    const __amdgpu_buffer_rsrc_t x_r = raw_rsrc(x, (uint32_t)K * 4u);
    f32x4_t xr[XV / 4];
    if (stager) {
#pragma unroll
        for (int i = 0; i < XV / 4; ++i)
            xr[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                x_r, (uint32_t)(hc * 32 + xpart * XV + 4 * i) * 4u, 0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);

    const int G = K >> (gshift + 5);
    const int ZB = (G + 1) >> 1;
    const int RB = K >> 1;
    uint32_t *xrec = ilds;                                           // [C][kIW]
    float *xres = reinterpret_cast<float *>(ilds + C * kIW);         // [C][32]: slot 2c + h, half h of chunk c
    float *comb = xres + C * 32;                                     // [W][R]
    const int lane = tid & 63;
    constexpr int RG = 64 / LPR;               // rows one load instruction covers
    static_assert(LPR == 64 || (S == 1 && JP == 1), "short rows: no K-split, one chunk per lane");
    const int li = LPR == 64 ? lane : lane % LPR;    // chunk position within the row
    const int rgl = LPR == 64 ? 0 : lane / LPR;      // row of the slot this lane works on
    const int NG = W / S;                      // row groups per workgroup
    const int rg = wave / S;
    const int ks = wave - rg * S;
    const int gq = rpg / NG, grem = rpg - gq * NG;
    const int gstart = blockIdx.x * rpg + rg * gq + min(rg, grem);
    const int nrows = max(0, min(gq + (rg < grem ? 1 : 0), N - gstart));   // rows of this group, <= R * RG
    const int rbase = min(gstart, N - 1);
    const int part = (C + S - 1) / S;
    const int lo = ks * part;
    const int hi = min(C, lo + part);
    const int clast = min(max(lo, hi - 1), C - 1);   // loads past the slice re-read a valid chunk
    const uint32_t magic8 = 0x88888888u;

    const uint32_t rows_left = (uint32_t)(N - rbase);
    // Row of each slot (of this lane's half, with short rows): slots past the
    // group's rows re-read its last row.  Uniform (an SGPR offset) for whole
    // 64-lane rows, per lane (added to the VGPR offset) for short rows.
    uint32_t lr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) lr[r] = (uint32_t)min(r * RG + rgl, max(nrows, 1) - 1);

    // With 8 or 16 wavefronts the stagers convert the first pass of x before
    // issuing their own weight loads, so that the x loads of every workgroup
    // on a CU sit ahead of most weight traffic while the non-stagers' loads
    // keep the stream busy.  With 4 (small shapes, where every wavefront
    // stages and the kernel is latency-bound) the weights go first.  Then
    // group metadata, then the codes in the order they are consumed.
    constexpr bool kStageFirst = W >= 8 && XV == 16;
    int xsh = 0;
    if (kStageFirst && stager) xsh = store_int_chunk<XV>(xr, xpart, hc < C, xrec + hc * kIW);
    __builtin_amdgcn_sched_barrier(0);

    // The SwiGLU form (SWI) runs the loads and arithmetic twice on the same
    // converted x: phase 0 the gate matrix (wq, scales, zeros), phase 1 the
    // up matrix (wq2, scales2, zeros2), whose loads are issued after phase
    // 0's arithmetic.
    constexpr int NPH = SWI ? 2 : 1;
    float acc[NPH][R];
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
    const uint8_t *wqp = ph ? wq2 : wq;
    const uint16_t *scp = ph ? scales2 : scales;
    const uint8_t *zpp = ph ? zeros2 : zeros;
    const __amdgpu_buffer_rsrc_t wq_r = raw_rsrc(wqp + (size_t)rbase * RB, span32(rows_left, RB));
    const __amdgpu_buffer_rsrc_t sc_r = raw_rsrc(scp + (size_t)rbase * G, span32(rows_left, 2u * G));
    const __amdgpu_buffer_rsrc_t zp_r = raw_rsrc(zpp + (size_t)rbase * ZB, span32(rows_left, ZB));
    uint32_t sr[JP][R], zr[JP][R];
#pragma unroll
    for (int j = 0; j < JP; ++j) {
        const uint32_t gi = (uint32_t)min(lo + li + LPR * j, clast) >> gshift;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t rs = LPR == 64 ? lr[r] : 0u, rv = LPR == 64 ? 0u : lr[r];
            sr[j][r] = __builtin_amdgcn_raw_buffer_load_b16(sc_r, gi * 2u + rv * (uint32_t)G * 2u,
                                                            rs * (uint32_t)G * 2u, 0);
            zr[j][r] = __builtin_amdgcn_raw_buffer_load_b8(zp_r, (gi >> 1) + rv * (uint32_t)ZB,
                                                           rs * (uint32_t)ZB, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4_t w[JP][R];
#pragma unroll
    for (int j = 0; j < JP; ++j) {
        const uint32_t coff = (uint32_t)min(lo + li + LPR * j, clast) * 16u;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t rs = LPR == 64 ? lr[r] : 0u, rv = LPR == 64 ? 0u : lr[r];
            w[j][r] = __builtin_amdgcn_raw_buffer_load_b128(wq_r, coff + rv * (uint32_t)RB, rs * (uint32_t)RB,
                                                            kNonTemporal);
        }
    }

    if (ph == 0) {
        // The flags and residuals of the first pass (after this wavefront's
        // weight loads), then the chunks of x past the first pass, loaded and
        // converted here.  Every half chunk has its own residual slot.
        if (stager) {
            if (!kStageFirst) xsh = store_int_chunk<XV>(xr, xpart, hc < C, xrec + hc * kIW);
            store_int_flags<XV>(xr, xsh, xpart, hc < C, xrec + hc * kIW, xres, 2 * hc + xslot, nullptr, 2u * C);
        }
        if (MULTI)
        for (int cb = kPass; cb < C; cb += kPass) {
            if (cb + wave * XWC >= C) break;
            const int c = cb + hc;
#pragma unroll
            for (int i = 0; i < XV / 4; ++i)
                xr[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                    x_r, (uint32_t)(c * 32 + xpart * XV + 4 * i) * 4u, 0, 0));
            const int sh = store_int_chunk<XV>(xr, xpart, c < C, xrec + c * kIW);
            store_int_flags<XV>(xr, sh, xpart, c < C, xrec + c * kIW, xres, 2 * c + xslot, nullptr, 2u * C);
        }
        __syncthreads();
    }

#pragma unroll
    for (int r = 0; r < R; ++r) acc[ph][r] = 0.f;
#pragma unroll
    for (int j = 0; j < JP; ++j) {
        const int c = lo + li + LPR * j;
        if (c < hi) {
            const uint32_t *rec = xrec + c * kIW;
            u32x4_t D[kPlanes];
#pragma unroll
            for (int d = 0; d < kPlanes; ++d) D[d] = *reinterpret_cast<const u32x4_t *>(rec + 4 * d);
            const IntChunk ic = int_chunk_tail(rec);
            const uint32_t zsh = (((uint32_t)c >> gshift) & 1u) << 2;
            int nz[R];
            float t[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                nz[r] = 8 - (int)__builtin_amdgcn_ubfe(zr[j][r], zsh, 4);
                t[r] = 0.f;
                if (r * RG + rgl < nrows)
                    t[r] = int_chunk_dot(w[j][r], D, nz[r], ic.sxl, ic.sxh, magic8);
            }
            // Flagged elements: (q - z) * r from their exact residuals.
            for (uint32_t fm = ic.flags; fm; fm &= fm - 1) {
                const uint32_t k = (uint32_t)__builtin_ctz(fm);
                const uint32_t slot = (ic.slots >> (k < 16 ? 0 : 11)) & kNoSlot;
                const float res = xres[slot * 16 + (k & 15u)];
#pragma unroll
                for (int r = 0; r < R; ++r)
                    if (r * RG + rgl < nrows)
                        t[r] = __builtin_fmaf((float)(chunk_code(w[j][r], k, 0u) - 8 + nz[r]), res, t[r]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (r * RG + rgl < nrows) {
                    const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sr[j][r]);
                    acc[ph][r] = __builtin_fmaf(s, t[r] * ic.cscale, acc[ph][r]);
                }
            }
        }
    }
    }   // phases

    if constexpr (LPR < 64) {
        // Short rows: each slot's sum over its LPR lanes; lane 0 of the group stores.
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float v = q4::group_sum<LPR>(acc[0][r]);
            const float u = SWI ? q4::group_sum<LPR>(acc[NPH - 1][r]) : 0.f;
            if (li == 0 && r * RG + rgl < nrows) {
                if (SWI) y[gstart + r * RG + rgl] = silu(v) * u;
                else store_y(y, gstart + r * RG + rgl, v, epi);
            }
        }
        return;
    }
    constexpr int NQ = (R + 3) / 4;
    float out[NQ], outu[NQ];
    q4::wave_reduce_rows<R>(acc[0], out);
    if (SWI) q4::wave_reduce_rows<R>(acc[NPH - 1], outu);
    const int h = lane >> 4;
    const bool writer = (lane & 15) == 0 && (R >= 4 || (h & (R == 2 ? 1 : 3)) == 0);
    if (S == 1) {
        if (writer) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int rr = q4::reduced_row<R>(q, h);
                if (rr < nrows) {
                    if (SWI) y[gstart + rr] = silu(out[q]) * outu[q];
                    else store_y(y, gstart + rr, out[q], epi);
                }
            }
        }
        return;
    }
    if (writer) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) comb[wave * R + q4::reduced_row<R>(q, h)] = out[q];
    }
    __syncthreads();
    if (ks == 0 && writer) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int rr = q4::reduced_row<R>(q, h);
            if (rr < nrows) {
                float v = out[q];
                for (int t = 1; t < S; ++t) v += comb[(wave + t) * R + rr];
                store_y(y, gstart + rr, v, epi);
            }
        }
    }
}

// The integer path for 2 to 8 activation rows.  Every row of x is converted
// as for one row (chunk records of kIW dwords, row m's records after row
// m-1's); a lane's code word then meets the digit planes of each x row in
// turn, so the codes are loaded once for all rows.  MP is M rounded up to 2,
// 4 or 8 (rows past M are skipped by a uniform branch).  x is converted in
// K segments of seg_chunks chunks when M rows of records would overflow the
// LDS budget; the weights of a segment are loaded before its x is converted.
// The S wavefronts of a row group split each segment's chunks and meet in
// LDS at the end.  Residuals of flagged half chunks go to a pool of `cap`
// slots per segment, dealt out by an LDS counter; half chunks past the pool
// recompute theirs from x where they are used.
template <int W, int MP, int JP, int R, int S>
__global__ __launch_bounds__(W * 64) void gemv_q4_intm_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ wq,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    float *__restrict__ y, int M, int N, int K, int gshift, int rpg, int seg_chunks, int cap, int epi) {
    static_assert(kIntTPC == 2, "two threads convert one chunk");
    extern __shared__ uint32_t ilds[];
    const int tid = threadIdx.x;
    const int C = K >> 5;
    const int G = K >> (gshift + 5);
    const int ZB = (G + 1) >> 1;
    const int RB = K >> 1;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int hc = tid >> 1, half = tid & 1;
    const int NG = W / S;
    const int rg = wave / S;
    const int ks = wave - rg * S;
    const int gq = rpg / NG, grem = rpg - gq * NG;
    const int gstart = blockIdx.x * rpg + rg * gq + min(rg, grem);
    const int nrows = max(0, min(gq + (rg < grem ? 1 : 0), N - gstart));
    const int rbase = min(gstart, N - 1);
    const uint32_t magic8 = 0x88888888u;
    uint32_t *xrec = ilds;                                                 // [M][seg][kIW]
    float *pool = reinterpret_cast<float *>(ilds + M * seg_chunks * kIW);  // [cap][16]
    float *comb = pool + cap * 16;                                         // [W][R][MP]
    uint32_t *next = reinterpret_cast<uint32_t *>(comb + W * R * MP);      // next free pool slot

    const __amdgpu_buffer_rsrc_t x_r = raw_rsrc(x, (uint32_t)(M * K) * 4u);   // M K <= 2^27 (validate)
    const uint32_t rows_left = (uint32_t)(N - rbase);
    const __amdgpu_buffer_rsrc_t wq_r = raw_rsrc(wq + (size_t)rbase * RB, span32(rows_left, RB));
    const __amdgpu_buffer_rsrc_t sc_r = raw_rsrc(scales + (size_t)rbase * G, span32(rows_left, 2u * G));
    const __amdgpu_buffer_rsrc_t zp_r = raw_rsrc(zeros + (size_t)rbase * ZB, span32(rows_left, ZB));
    uint32_t lr[R];   // row offset of each slot: slots past the group's rows re-read its last row
#pragma unroll
    for (int r = 0; r < R; ++r) lr[r] = (uint32_t)min(r, max(nrows, 1) - 1);

    float acc[R][MP];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MP; ++m) acc[r][m] = 0.f;

    for (int seg0 = 0; seg0 < C; seg0 += seg_chunks) {
        const int segC = min(seg_chunks, C - seg0);
        const int part = (segC + S - 1) / S;
        const int lo = seg0 + ks * part;
        const int hi = min(seg0 + segC, lo + part);
        const int clast = min(max(lo, hi - 1), seg0 + segC - 1);
        const int nx = M * segC;                  // chunk records of this segment

        // x first: every pass's loads, then the conversion, then the barrier,
        // all before any weight load is issued.  The pool counter is reset
        // before the conversion (the previous segment's pool is no longer read).
        {
            f32x4_t xr[2][4];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int p = min(q * W * 32 + hc, nx - 1);
                const int m = p / segC, c = p - m * segC;
                const uint32_t off = (uint32_t)(m * K + (seg0 + c) * 32 + half * 16) * 4u;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xr[q][i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(x_r, off + 16u * i, 0, 0));
            }
            if (tid == 0) *next = 0u;
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int pb = q * W * 32;
                if (pb < nx) {
                    const int p = min(pb + hc, nx - 1);
                    const int m = p / segC, c = p - m * segC;
                    uint32_t *rec = xrec + (m * segC + c) * kIW;
                    const int sh = store_int_chunk<kIntVPT>(xr[q], half, pb + hc < nx, rec);
                    store_int_flags<kIntVPT>(xr[q], sh, half, pb + hc < nx, rec, pool, -1, next, (uint32_t)cap);
                }
            }
            for (int pb = 2 * W * 32; pb < nx; pb += W * 32) {
                const int p = min(pb + hc, nx - 1);
                const int m = p / segC, c = p - m * segC;
                const uint32_t off = (uint32_t)(m * K + (seg0 + c) * 32 + half * 16) * 4u;
                f32x4_t xq[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xq[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(x_r, off + 16u * i, 0, 0));
                uint32_t *rec = xrec + (m * segC + c) * kIW;
                const int sh = store_int_chunk<kIntVPT>(xq, half, pb + hc < nx, rec);
                store_int_flags<kIntVPT>(xq, sh, half, pb + hc < nx, rec, pool, -1, next, (uint32_t)cap);
            }
        }
        __syncthreads();
        uint32_t sr[JP][R], zr[JP][R];
#pragma unroll
        for (int j = 0; j < JP; ++j) {
            const uint32_t gi = (uint32_t)min(lo + lane + 64 * j, clast) >> gshift;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                sr[j][r] = __builtin_amdgcn_raw_buffer_load_b16(sc_r, gi * 2u, lr[r] * (uint32_t)G * 2u, 0);
                zr[j][r] = __builtin_amdgcn_raw_buffer_load_b8(zp_r, gi >> 1, lr[r] * (uint32_t)ZB, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        u32x4_t w[JP][R];
#pragma unroll
        for (int j = 0; j < JP; ++j) {
            const uint32_t coff = (uint32_t)min(lo + lane + 64 * j, clast) * 16u;
#pragma unroll
            for (int r = 0; r < R; ++r)
                w[j][r] = __builtin_amdgcn_raw_buffer_load_b128(wq_r, coff, lr[r] * (uint32_t)RB, kNonTemporal);
        }

#pragma unroll
        for (int j = 0; j < JP; ++j) {
            const int c = lo + lane + 64 * j;
            if (c < hi) {
                const uint32_t zsh = (((uint32_t)c >> gshift) & 1u) << 2;
                int nz[R];
                float s[R];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    nz[r] = 8 - (int)__builtin_amdgcn_ubfe(zr[j][r], zsh, 4);
                    s[r] = (float)__builtin_bit_cast(_Float16, (uint16_t)sr[j][r]);
                    w[j][r] ^= magic8;   // codes as signed nibbles q - 8, once for every x row
                }
#pragma unroll
                for (int m = 0; m < MP; ++m) {
                    if (m < M) {
                        const uint32_t *rec = xrec + (m * segC + c - seg0) * kIW;
                        u32x4_t D[kPlanes];
#pragma unroll
                        for (int d = 0; d < kPlanes; ++d) D[d] = *reinterpret_cast<const u32x4_t *>(rec + 4 * d);
                        const IntChunk ic = int_chunk_tail(rec);
                        float t[R];
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            t[r] = 0.f;
                            if (r < nrows) t[r] = int_chunk_dot(w[j][r], D, nz[r], ic.sxl, ic.sxh, 0u);
                        }
                        // Flagged elements: (q - z) * r from their exact residuals.
                        for (uint32_t fm = ic.flags; fm; fm &= fm - 1) {
                            const uint32_t k = (uint32_t)__builtin_ctz(fm);
                            const uint32_t slot = (ic.slots >> (k < 16 ? 0 : 11)) & kNoSlot;
                            float res;
                            if (slot != kNoSlot) {
                                res = pool[slot * 16 + (k & 15u)];
                            } else {
                                const float xv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                    x_r, (uint32_t)(m * K + c * 32 + (int)k) * 4u, 0, 0));
                                res = int_residual(xv, (int)(ic.slots >> 23) - 128);
                            }
#pragma unroll
                            for (int r = 0; r < R; ++r)
                                if (r < nrows)
                                    t[r] = __builtin_fmaf((float)(chunk_code(w[j][r], k, magic8) - 8 + nz[r]), res, t[r]);
                        }
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            if (r < nrows) acc[r][m] = __builtin_fmaf(s[r], t[r] * ic.cscale, acc[r][m]);
                    }
                }
            }
        }
        if (seg0 + seg_chunks < C) __syncthreads();   // records fully read before the next segment's
    }

    constexpr int NQ = (R + 3) / 4;
    float out[MP][NQ];
#pragma unroll
    for (int m = 0; m < MP; ++m) {
        float v[R];
#pragma unroll
        for (int r = 0; r < R; ++r) v[r] = acc[r][m];
        q4::wave_reduce_rows<R>(v, out[m]);
    }
    const int h = lane >> 4;
    const bool writer = (lane & 15) == 0 && (R >= 4 || (h & (R == 2 ? 1 : 3)) == 0);
    if (S == 1) {
        if (writer) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int rr = q4::reduced_row<R>(q, h);
                if (rr < nrows) {
#pragma unroll
                    for (int m = 0; m < MP; ++m)
                        if (m < M) store_y(y, (size_t)m * N + gstart + rr, out[m][q], epi);
                }
            }
        }
        return;
    }
    if (writer) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int rr = q4::reduced_row<R>(q, h);
#pragma unroll
            for (int m = 0; m < MP; ++m) comb[(wave * R + rr) * MP + m] = out[m][q];
        }
    }
    __syncthreads();
    if (ks == 0 && writer) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int rr = q4::reduced_row<R>(q, h);
            if (rr < nrows) {
#pragma unroll
                for (int m = 0; m < MP; ++m) {
                    if (m < M) {
                        float v = out[m][q];
                        for (int t = 1; t < S; ++t) v += comb[((wave + t) * R + rr) * MP + m];
                        store_y(y, (size_t)m * N + gstart + rr, v, epi);
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------- 2 to 8 activation rows: fp32 multiply-add
//
// With several activation rows every weight serves M products, so it pays to
// form each weight once as an exact fp32 value and to run plain fp32 fused
// multiply-adds, which on gfx950 issue at about twice the rate of the 4-bit
// dot products and the mixed-precision multiply-adds, and which need no
// conversion of x.  A code q at bits 4p..4p+3 of a 32-bit word (p <= 4) is
// masked into the mantissa of a float whose exponent is that of 2^23: the
// float is 2^23 + q 16^p, and subtracting 2^23 + z 16^p (both in [2^23,
// 2^24), so the difference is exact) leaves (q - z) 16^p.  The word's upper
// three codes take the same steps after a shift by 20.  x is staged in LDS
// divided by the same power of two 16^p (exact), so every product is
// (q - z) x, and the group scale multiplies each 32-code chunk's partial sum.
// Per weight: one AND and one subtract, both of the fast-issuing kind.
//
// Lanes: 16 per row.  One 16-byte load instruction covers four rows (256
// contiguous bytes each), and the four rows' lanes read the same x from LDS
// (a broadcast), so four rows share each read of x.  A wavefront owns R
// slots of four rows; S wavefronts split a row group's K range and meet in
// LDS; a workgroup's rpg rows are dealt to its W / S row groups.
constexpr int kFmStride = 36;   // floats per staged chunk of x: 144 bytes, an odd number of 16-byte slots

// 16^-p for the code at nibble k (0..7) of its word: nibbles 0-4 in place,
// 5-7 after the shift by 20 (positions 0-2).
__host__ __device__ constexpr float fm_x_scale(int k) {
    return k == 0 || k == 5 ? 1.0f : k == 1 || k == 6 ? 0.0625f : k == 2 || k == 7 ? 0.00390625f
                                                             : k == 3 ? 0.000244140625f : 1.52587890625e-05f;
}

// The value of v, hidden from the compiler's algebra (so that a mask on a
// pre-ORed base stays one AND rather than being re-associated into two).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

template <int W, int MX, int R, int LPR, int S, int JP, int PD = 2, bool XPD = (W <= 8 || MX * R <= 4)>
__global__ __launch_bounds__(W * 64) void gemv_q4_fm_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ wq,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    float *__restrict__ y, int N, int K, int gshift, int rpg, int seg_chunks, int epi,
    float *__restrict__ part, int ks_log2, int kpart) {
    constexpr int SUBR = 64 / LPR;             // rows one load instruction covers (a slot)
    constexpr int NG = W / S;                  // row groups per workgroup
    // float4 of one x row one thread loads ahead of the weights: the first
    // 512 / 256 / 128 chunks of the segment for 2 / 3-4 / 5-8 rows
    constexpr int XQ = (MX <= 2 ? 256 : 128) * 8 / (W * 64) > 0 ? (MX <= 2 ? 256 : 128) * 8 / (W * 64) : 1;
    extern __shared__ float fms[];
    float *xs = fms;                                                   // [MX][seg][kFmStride]
    float *comb = fms + MX * seg_chunks * kFmStride;                   // [W][SUBR R][MX]
    // every argument in registers at once: one round trip for the kernel
    // arguments instead of one per use site
    asm volatile("" ::"s"(x), "s"(wq), "s"(scales), "s"(zeros), "s"(y), "s"(N), "s"(K), "s"(gshift),
                 "s"(rpg), "s"(seg_chunks), "s"(epi), "s"(part), "s"(ks_log2), "s"(kpart));
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int sub = lane / LPR, li = lane % LPR;
    const int rg = wave / S, ks = wave - rg * S;
    const int C = K >> 5;
    const int G = K >> (gshift + 5);
    const int ZB = (G + 1) >> 1;
    const int RB = K >> 1;
    // KS workgroups may split the K range of one block of rpg rows: this one
    // takes chunks [kc0, kc1) of the rows from rb * rpg, and with KS > 1
    // writes partial sums that fm_sum_parts adds.
    const int KS = 1 << ks_log2;   // a power of two: no division on the way to the first load
    const int rb = (int)blockIdx.x >> ks_log2, kb = (int)blockIdx.x & (KS - 1);
    const int kc0 = kb * kpart, kc1 = min(C, kc0 + kpart);
    const int gq = rpg / NG, grem = rpg - gq * NG;
    const int gstart = rb * rpg + rg * gq + min(rg, grem);
    const int nrows = max(0, min(gq + (rg < grem ? 1 : 0), N - gstart));   // rows of this group, <= SUBR R
    const int rbase = min(gstart, N - 1);
    const uint32_t rows_left = (uint32_t)(N - rbase);
    const __amdgpu_buffer_rsrc_t x_r = raw_rsrc(x, (uint32_t)(MX * K) * 4u);   // M K <= 2^27 (validate)
    const __amdgpu_buffer_rsrc_t wq_r = raw_rsrc(wq + (size_t)rbase * RB, span32(rows_left, RB));
    const __amdgpu_buffer_rsrc_t sc_r = raw_rsrc(scales + (size_t)rbase * G, span32(rows_left, 2u * G));
    const __amdgpu_buffer_rsrc_t zp_r = raw_rsrc(zeros + (size_t)rbase * ZB, span32(rows_left, ZB));
    // the row each slot of this lane works on (past the group's rows: its last row, not stored)
    uint32_t lr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) lr[r] = (uint32_t)min(SUBR * r + sub, max(nrows, 1) - 1);

    float acc[R][MX];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MX; ++m) acc[r][m] = 0.f;

    for (int seg0 = kc0; seg0 < kc1; seg0 += seg_chunks) {
        const int segC = min(seg_chunks, kc1 - seg0);
        const int part = (segC + S - 1) / S;
        const int lo = seg0 + ks * part;
        const int hi = min(seg0 + segC, lo + part);
        const int clast = max(lo, hi - 1);        // loads past the range re-read a chunk inside it
        const int n4 = segC * 8;                   // float4 of one x row in the segment
        // x of the segment first (a CU returns loads in issue order), its
        // first XQ * W * 64 float4 per row; then every code and metadata load of this
        // wavefront's chunks; then x into LDS, divided by its codes' 16^p.
        f32x4_t xv4[MX][XQ];
#pragma unroll
        for (int m = 0; m < MX; ++m)
#pragma unroll
            for (int q = 0; q < XQ; ++q) {
                const int i = min(q * W * 64 + tid, n4 - 1);
                xv4[m][q] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                    x_r, (uint32_t)(m * K + seg0 * 32 + 4 * i) * 4u, 0, 0));
            }
        __builtin_amdgcn_sched_barrier(0);
        // Code and metadata loads, PD chunk positions ahead of the arithmetic:
        // each wavefront's loads are paced by its own work, so that the
        // wavefronts of a CU (whose loads return in issue order) receive
        // their data at the same rate rather than one after another.
        u32x4_t w[JP][R];
        uint32_t sr[JP][R], zr[JP][R];
        auto issue = [&](int j) {
            const uint32_t c = (uint32_t)min(lo + li + LPR * j, clast);
            const uint32_t gi = c >> gshift;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                sr[j][r] = __builtin_amdgcn_raw_buffer_load_b16(sc_r, gi * 2u + lr[r] * (uint32_t)G * 2u, 0, 0);
                zr[j][r] = __builtin_amdgcn_raw_buffer_load_b8(zp_r, (gi >> 1) + lr[r] * (uint32_t)ZB, 0, 0);
                w[j][r] = __builtin_amdgcn_raw_buffer_load_b128(wq_r, c * 16u + lr[r] * (uint32_t)RB, 0, kNonTemporal);
            }
        };
        const f32x4_t sc_even = {fm_x_scale(0), fm_x_scale(1), fm_x_scale(2), fm_x_scale(3)};
        const f32x4_t sc_odd = {fm_x_scale(4), fm_x_scale(5), fm_x_scale(6), fm_x_scale(7)};
        for (int m = 0; m < MX; ++m)                  // the rest of longer segments, before any weight load
            for (int i = XQ * W * 64 + tid; i < n4; i += W * 64) {
                const f32x4_t v = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                    x_r, (uint32_t)(m * K + seg0 * 32 + 4 * i) * 4u, 0, 0));
                *reinterpret_cast<f32x4_t *>(xs + (m * segC + (i >> 3)) * kFmStride + 4 * (i & 7)) =
                    v * ((i & 1) ? sc_odd : sc_even);
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < PD && j < JP; ++j) issue(j);
        __builtin_amdgcn_sched_barrier(0);
        // Threads past the segment store their clamped (last) element again:
        // the same value to the same place, and no store under a condition,
        // which would let the compiler sink the x load below the weight loads.
#pragma unroll
        for (int m = 0; m < MX; ++m)
#pragma unroll
            for (int q = 0; q < XQ; ++q) {
                const int i = min(q * W * 64 + tid, n4 - 1);
                *reinterpret_cast<f32x4_t *>(xs + (m * segC + (i >> 3)) * kFmStride + 4 * (i & 7)) =
                    xv4[m][q] * ((i & 1) ? sc_odd : sc_even);
            }
        __syncthreads();

        // x of each (chunk, half word) is read from LDS one step ahead of its use
        // (XPD), or just before it where the second buffer would not fit in registers.
        float xw[XPD ? 2 : 1][MX][4];
        auto xload = [&](int stp, float (&xr)[MX][4]) {
            const int c = min(lo + li + LPR * (stp >> 3), clast);
            const float *xc = xs + (c - seg0) * kFmStride + 4 * (stp & 7);
#pragma unroll
            for (int m = 0; m < MX; ++m) {
                const f32x4_t a = *reinterpret_cast<const f32x4_t *>(xc + m * segC * kFmStride);
                xr[m][0] = a.x; xr[m][1] = a.y; xr[m][2] = a.z; xr[m][3] = a.w;
            }
        };
        if constexpr (XPD) xload(0, xw[0]);
#pragma unroll
        for (int j = 0; j < JP; ++j) {
            if (j + PD < JP) issue(j + PD);
            __builtin_amdgcn_sched_barrier(0);
            const int c = lo + li + LPR * j;
            const uint32_t gi = (uint32_t)min(c, clast) >> gshift;
            float t[R][MX];
            float cz[R][5];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float zf = (float)__builtin_amdgcn_ubfe(zr[j][r], (gi & 1u) << 2, 4);
#pragma unroll
                for (int p = 0; p < 5; ++p) cz[r][p] = __builtin_fmaf(zf, (float)(1 << (4 * p)), 8388608.0f);
#pragma unroll
                for (int m = 0; m < MX; ++m) t[r][m] = 0.f;
            }
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) {
                float f[R][8];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t cw = wd == 0 ? w[j][r].x : wd == 1 ? w[j][r].y : wd == 2 ? w[j][r].z : w[j][r].w;
                    const uint32_t blo = opaque((cw & 0x000FFFFFu) | 0x4B000000u);
                    const uint32_t bhi = opaque((cw >> 20) | 0x4B000000u);
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const uint32_t bb = k < 5 ? blo : bhi;
                        const int p = k < 5 ? k : k - 5;
                        f[r][k] = __builtin_bit_cast(float, bb & (0xFF800000u | (0xFu << (4 * p)))) - cz[r][p];
                    }
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int stp = 8 * j + 2 * wd + h;
                    // the fence keeps each LDS read one step ahead, not hoisted further
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (XPD) {
                        if (stp + 1 < 8 * JP) xload(stp + 1, xw[(stp + 1) & 1]);
                    } else {
                        xload(stp, xw[0]);
                    }
                    const int xb = XPD ? (stp & 1) : 0;
                    // R x MX independent accumulators, element by element
#pragma unroll
                    for (int k = 0; k < 4; ++k)
#pragma unroll
                        for (int m = 0; m < MX; ++m)
#pragma unroll
                            for (int r = 0; r < R; ++r)
                                t[r][m] = __builtin_fmaf(f[r][4 * h + k], xw[xb][m][k], t[r][m]);
                    // pin this step's products before the next fence (pure arithmetic
                    // is otherwise free to sink past it, and the reads pile up)
#pragma unroll
                    for (int m = 0; m < MX; ++m)
#pragma unroll
                        for (int r = 0; r < R; ++r) asm volatile("" : "+v"(t[r][m]));
                }
            }
            if (c < hi) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float scf = (float)__builtin_bit_cast(_Float16, (uint16_t)sr[j][r]);
#pragma unroll
                    for (int m = 0; m < MX; ++m) acc[r][m] = __builtin_fmaf(scf, t[r][m], acc[r][m]);
                }
            }
        }
        if (seg0 + seg_chunks < kc1) __syncthreads();   // x segment fully read before the next overwrites it
    }

    // Each slot's sum over its LPR lanes; lane 0 of the group holds it.
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MX; ++m) acc[r][m] = q4::group_sum<LPR>(acc[r][m]);
    // A row's sum over this workgroup's K range: the output itself, or (K
    // split over KS workgroups) this workgroup's partial sum, [kb][m][row].
    auto emit = [&](int m, int row, float v) {
        if (KS == 1)
            store_y(y, (size_t)m * N + row, v, epi);
        else
            part[((size_t)kb * MX + m) * N + row] = v;
    };
    if (S == 1) {
        if (li == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int rr = SUBR * r + sub;
                if (rr < nrows)
#pragma unroll
                    for (int m = 0; m < MX; ++m) emit(m, gstart + rr, acc[r][m]);
            }
        }
        return;
    }
    if (li == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MX; ++m) comb[(wave * SUBR * R + SUBR * r + sub) * MX + m] = acc[r][m];
    }
    __syncthreads();
    if (ks == 0 && li == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int rr = SUBR * r + sub;
            if (rr < nrows) {
#pragma unroll
                for (int m = 0; m < MX; ++m) {
                    float v = acc[r][m];
                    for (int u = 1; u < S; ++u) v += comb[((wave + u) * SUBR * R + SUBR * r + sub) * MX + m];
                    emit(m, gstart + rr, v);
                }
            }
        }
    }
}

// The second launch of a K split over workgroups: every output is the sum of
// its KS partial sums, added in workgroup order (the result does not depend
// on which workgroup finished first), then stored as gemv_q4_fm_kernel would.
__global__ __launch_bounds__(256) void fm_sum_parts(float *__restrict__ y, const float *__restrict__ part,
                                                   int MN, int KS, int epi) {
    const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (i >= MN) return;
    float v = 0.f;
    for (int k = 0; k < KS; ++k) v += part[(size_t)k * MN + i];
    store_y(y, (size_t)i, v, epi);
}

// One int4 matrix of a call.
struct Q4Matrix {
    const uint8_t *wq;
    const uint16_t *scales;
    const uint8_t *zeros;
};

struct Geometry {
    int M, LPR, JP, S, seg_chunks, segments, grid, rows_per_wave;
    bool integer;   // the exact integer path (gemv_q4_int_kernel, gemv_q4_intm_kernel)
    int rpg;        // integer path: rows per workgroup
    int waves;      // wavefronts per workgroup
    int mp;         // integer path, M > 1: M rounded up to 2, 4 or 8
    int pool;       // integer path, M > 1: residual slots (half chunks) per x segment
    bool fm;        // M > 1: fp32 multiply-add on exactly dequantised weights (gemv_q4_fm_kernel)
    int epi;        // launch-time: finish a SwiGLU block in the store (see store_y)
    int fma_r;      // multiply-add path: row slots per wavefront
    int ks_wg;      // fm: workgroups splitting one row block's K range (partial sums in a workspace)
    int kpart;      // fm: chunks of K per workgroup
    const Q4Matrix *swi;   // launch-time: the up matrix of a one-launch SwiGLU block
    float *work;           // launch-time: the workspace of a K split over workgroups
};

constexpr int kCUs = 256;   // compute units of an MI355X
constexpr int kLdsMax = 160 * 1024;   // LDS of one CU, and the most one workgroup may use

// The integer path serves one activation row when every lane owns whole
// chunks (LPR = 64) and x fits the LDS budget in one piece.  Its K-split is
// raised until a lane holds at most 3 chunk positions.  Workgroups have 8
// wavefronts when that still gives every CU a workgroup (each converts x
// once, so fewer and larger workgroups convert it less often), 16 with a
// four-way K-split (a long x, read once per workgroup, would otherwise cost
// as many bytes as the weights of the workgroup's 8 rows), else 4.  Rows
// are dealt to workgroups so that, beyond one round of workgroups, every CU
// gets the same number of them (2 x 8 wavefronts of 3.5 rows rather than
// 1.75 x 8 of 4).
// Knobs a caller may fix for one shape (gemv_q4_set_geometry); 0 or -1 = the plan's choice.
struct Knobs {
    int path = -1;     // Q4_PATH_FMA or Q4_PATH_INTEGER
    int waves = 0;     // wavefronts per workgroup
    int ksplit = 0;    // wavefronts splitting one row's K range
};

bool plan_integer(Geometry &p, int N, int K, const Knobs &k) {
    const int C = K / 32;
    if (p.M != 1 || (p.LPR != 64 && p.LPR != 32)) return false;
    if (p.LPR == 32) {
        // Short rows (512 < K <= 1024): two rows per load instruction, no
        // K-split, one chunk per lane; 8 wavefronts once that still gives
        // every CU a workgroup, else 4.  2 row slots below 16384 rows (more,
        // smaller wavefronts for these latency-bound shapes: 896 x 896 g32
        // 3.32 -> 2.78 us, 4864 x 896 3.41 -> 3.12 us), else 4 (the 151936-row
        // LM head: 17.4 against 18.9 us with 2, 24.1 with 8).
        if (k.ksplit && k.ksplit != 1) return false;
        const int R = N < 16384 ? 2 : row_slots(1);
        const long groups = ((long)N + 2 * R - 1) / (2 * R);
        const int W = k.waves ? k.waves : (groups >= 8L * kCUs ? 8 : 4);
        const long grid = (groups + W - 1) / W;
        p.integer = true;
        p.waves = W;
        p.S = 1;
        p.JP = 1;
        p.grid = (int)grid;
        p.rpg = (int)((N + grid - 1) / grid);
        p.rows_per_wave = 2 * R;
        p.seg_chunks = C;
        p.segments = 1;
        return true;
    }
    int S = k.ksplit ? k.ksplit : p.S;
    if (!k.ksplit)
        while (S < 4 && (C + S - 1) / S > 3 * 64) S *= 2;
    const int part = (C + S - 1) / S;
    const int JP = (part + 63) / 64;
    const int R = row_slots(1);
    const long groups = ((long)N + R - 1) / R;
    const long waves = groups * S;
    // Records and residual slots of the whole x; two workgroups share a CU's
    // LDS only while they take at most half of it each.
    const size_t xbytes = (size_t)C * (kIW * 4 + 32 * 4);
    const bool half_cu = xbytes + (size_t)8 * R * 4 <= (size_t)kLdsMax / 2;
    const int W = k.waves ? k.waves
                          : ((S == 4 || (S > 1 && !half_cu)) && waves >= 16L * kCUs ? 16
                                                                              : (waves >= 8L * kCUs ? 8 : 4));
    if (JP > 3 || W < S || xbytes + (size_t)W * R * 4 > (size_t)kLdsMax)
        return false;
    const int groups_per_wg = W / S;
    long grid = (groups + groups_per_wg - 1) / groups_per_wg;
    if (grid * W > (long)kCUs * 4) grid = (grid + kCUs - 1) / kCUs * kCUs;
    p.integer = true;
    p.waves = W;
    p.S = S;
    p.JP = JP;
    p.grid = (int)grid;
    p.rpg = (int)((N + grid - 1) / grid);
    p.rows_per_wave = R;
    p.seg_chunks = C;
    p.segments = 1;
    return true;
}

// The integer path for 2 to 8 activation rows: workgroups of 8 wavefronts, 2
// per CU (16 and 1 per CU at MP = 8, whose records need more LDS), each
// owning about N / (workgroups) rows and converting x once.  x is cut into
// segments of whole lane sweeps when M rows of records exceed the LDS share
// (only at MP = 8; smaller M takes the multiply-add path then).
// The K-split S grows while the row groups that remain still hold the
// workgroup's rows and each split keeps a full lane sweep, and until a lane
// holds at most 2 chunk positions.
bool plan_integer_m(Geometry &p, int M, int N, int K, const Knobs &k) {
    const int C = K / 32;
    if (M < 2 || p.LPR != 64 || K <= 1024) return false;
    const int MP = M <= 2 ? 2 : (M <= 4 ? 4 : 8);
    const int W = MP == 8 ? 16 : 8;
    if (k.waves && k.waves != W) return false;
    const int wpc = MP == 8 ? 1 : 2;
    const int R = 4;
    // Per segment chunk and x row: its record and a sixteenth of a chunk's
    // residuals in the pool (a pool slot holds half a chunk's; under
    // x ~ N(0, 1) about 0.3% of half chunks hold a flag); the counter.
    const int budget = kLdsMax / wpc - W * R * MP * 4 - 16;
    int seg = std::min(C, budget / (M * (kIW * 4 + 8)));
    if (seg < C) seg = seg / 64 * 64;
    // Segmented x costs a barrier and a pipeline drain per segment: below 5
    // rows the multiply-add path measures faster there (unless asked for).
    if (seg < 64 || (seg < C && MP <= 4 && k.path != Q4_PATH_INTEGER)) return false;
    const long target = (long)kCUs * wpc;
    const long rpw = std::max<long>((N + target - 1) / target, W);
    int S = 1;
    if (k.ksplit) {
        S = k.ksplit;
    } else {
        while (S < 4 && (long)(W / (2 * S)) * R >= rpw && seg / (2 * S) >= 64) S *= 2;
        while (S < 4 && (seg + S - 1) / S > 128) S *= 2;
    }
    if ((seg + S - 1) / S > 128) seg = 128 * S;
    const int part = (seg + S - 1) / S;
    const int JP = (part + 63) / 64;
    const long cap = (long)(W / S) * R;
    const long grid = ((long)N + std::min(cap, rpw) - 1) / std::min(cap, rpw);
    p.integer = true;
    p.mp = MP;
    p.waves = W;
    p.S = S;
    p.JP = JP;
    p.grid = (int)grid;
    p.rpg = (int)((N + grid - 1) / grid);
    p.rows_per_wave = R;
    p.seg_chunks = seg;
    p.segments = (C + seg - 1) / seg;
    p.pool = std::max(2, M * seg / 8);
    if (p.pool >= (int)kNoSlot) return false;   // slot numbers are 11-bit fields
    return true;
}

// The fp32 multiply-add kernel for 2 to 8 activation rows: 8 wavefronts of
// two 4-row slots (16 lanes per row), one workgroup per CU (more only past
// 64 rows per CU), the rows of a workgroup dealt to its row groups, and the
// K-split the largest that still leaves every row group room for its rows
// (or the one a caller fixed; then a workgroup takes no more rows than its
// row groups hold).  x is staged in segments when M rows of it exceed the
// LDS.
constexpr int kFmW = 8, kFmR = 2, kFmLPR = 16;   // wavefronts, slots per wavefront, lanes per row
// Chunk positions per lane and segment: past 8 for 7-8 rows of x the unrolled
// body no longer fits the compiler's unrolling budget.
constexpr int fm_jp_max(int M) { return M >= 7 ? 8 : 16; }

// Segments of x for a K range of C chunks: JP chunk positions per lane (a
// power of two from 2 to jmax) cover LPR * S * JP chunks; of the JP whose
// segments fit the LDS, the one with the fewest positions in all (a lane's
// steps, each a full pass of arithmetic whether its chunk exists or not),
// then the fewest segments.
void fm_segments(int M, int C, int S, int &seg, int &JP) {
    constexpr int W = kFmW, R = kFmR, LPR = kFmLPR, SUBR = 64 / LPR;
    const int comb = W * SUBR * R * M * 4;
    const int fit = (kLdsMax - comb) / (M * kFmStride * 4);
    const int jmax = fm_jp_max(M);
    seg = 0;
    JP = 0;
    long best = -1;
    for (int jp = 2; jp <= jmax; jp *= 2) {
        const int sweep = LPR * S * jp;
        if (sweep > fit && jp > 2) break;
        const int sg = std::min(C, sweep);
        const long steps = (long)(C + sg - 1) / sg * jp;   // every segment runs all jp positions
        if (best < 0 || steps < best || (steps == best && sg > seg)) {
            best = steps;
            seg = sg;
            JP = jp;
        }
    }
    if (seg > fit) seg = fit / (LPR * S) * (LPR * S);   // jp = 2 did not fit: a partial sweep
    if (seg < LPR * S) seg = std::min(C, LPR * S);
}

// split: a workspace is available for a K split over workgroups.  It is
// taken when x would otherwise be staged in several segments (long K at
// several rows: every CU would read all of x for a few rows' weights):
// KS workgroups per block of rows, each over a KS-th of K, KS doubling while
// the blocks still fill half their CUs' row slots and every part keeps at
// least one lane sweep (measured: 8 rows of 14336 -> 4096, 27.2 -> 23.6 us
// with the partial sums' own launch; 2 rows, one segment, 11.6 -> 13.3).
bool plan_fm(Geometry &p, int M, int N, int K, const Knobs &k, bool split = false) {
    const int C = K / 32;
    constexpr int W = kFmW, R = kFmR, LPR = kFmLPR, SUBR = 64 / LPR;
    constexpr int slots = W * SUBR * R;           // rows one workgroup holds
    if ((k.waves && k.waves != W) || (k.ksplit && W % k.ksplit != 0)) return false;
    int KS = 1;
    for (int pass = 0; pass < 2; ++pass) {
        long blocks = std::max<long>(1, std::min<long>(kCUs / KS, N));
        long rpg = (N + blocks - 1) / blocks;
        // a K split over workgroups takes the wavefront split from its rows,
        // not from the knob (which sets the unsplit plan)
        const int ks_knob = KS > 1 ? 0 : k.ksplit;
        int S = ks_knob ? ks_knob : 4;
        if (!ks_knob)
            while (S > 1 && (W / S) * SUBR * R < rpg) S /= 2;
        const long cap = (long)(W / S) * SUBR * R;    // rows the row groups hold
        if (rpg > cap) rpg = cap;
        blocks = (N + rpg - 1) / rpg;
        const int kpart = (C + KS - 1) / KS;
        int seg, JP;
        fm_segments(M, kpart, S, seg, JP);
        if (pass == 0 && split && seg < C) {
            // several segments unsplit: split K over workgroups and plan again
            while (KS < 8 && (long)N * 2 * KS <= (long)kCUs * slots && C >= 2 * KS * LPR * S) KS *= 2;
            if (KS > 1) continue;
        }
        p.fm = true;
        p.integer = false;
        p.mp = M;
        p.waves = W;
        p.S = S;
        p.LPR = LPR;
        p.JP = JP;
        p.ks_wg = KS;
        p.kpart = kpart;
        p.grid = (int)(blocks * KS);
        p.rpg = (int)rpg;
        p.rows_per_wave = SUBR * R;
        p.seg_chunks = seg;
        p.segments = (kpart + seg - 1) / seg;
        return true;
    }
    return false;
}

// Workspace bytes a launch needs: KS partial sums per output of a K split
// over workgroups, none otherwise.
size_t fm_work_bytes(const Geometry &p, int N) {
    return p.fm && p.ks_wg > 1 ? (size_t)p.ks_wg * p.M * N * sizeof(float) : 0;
}

// Chooses the launch geometry for a validated shape, with any knobs fixed;
// *ok is cleared when the knobs cannot be met.
Geometry plan_with(int M, int N, int K, const Knobs &k, bool *ok, bool split = false) {
    Geometry p{};
    p.M = M;
    const int C = K / 32;
    p.LPR = C <= 16 ? 16 : (C <= 32 ? 32 : 64);
    // Short rows (K <= 1024) of one activation row: 2 row slots below 16384
    // rows (more, smaller wavefronts for these latency-bound shapes), else 4.
    const int R = M == 1 && p.LPR < 64 && N < 16384 ? 2 : row_slots(M);
    p.fma_r = R;
    p.rows_per_wave = R * (q4::kWave / p.LPR);
    const long row_waves = ((long)N + p.rows_per_wave - 1) / p.rows_per_wave;
    // K-split, decided on the length of one x segment: enough wavefronts to
    // fill the chip (>= 2 per SIMD) and at most two chunk positions per lane,
    // while every split keeps a full lane sweep.
    const int seg_len = std::min(C, kLdsBytes / (M * kXStride * (int)sizeof(float)));
    p.S = 1;
    if (k.path == Q4_PATH_FMA && k.ksplit) {
        p.S = k.ksplit;
    } else {
        while (p.S < kWaves && 2 * p.S * p.LPR <= seg_len &&
               (row_waves * p.S < 2048 || (seg_len + p.S * p.LPR - 1) / (p.S * p.LPR) > 2))
            p.S *= 2;
    }
    // x segment: the LDS left after the K-split partial sums, in whole chunks;
    // when x needs several segments, each is a whole number of lane sweeps.
    const int comb = p.S > 1 ? kWaves * p.rows_per_wave * M * (int)sizeof(float) : 0;
    const int max_seg = (kLdsBytes - comb) / (M * kXStride * (int)sizeof(float));
    if (C <= max_seg) {
        p.seg_chunks = C;
    } else {
        const int sweep = p.S * p.LPR;
        p.seg_chunks = max_seg >= sweep ? max_seg / sweep * sweep : max_seg;
    }
    int part = (p.seg_chunks + p.S - 1) / p.S;
    p.JP = (part + p.LPR - 1) / p.LPR;
    if (p.JP > 4) {                    // JP is instantiated for 1, 2 and 4 only
        p.seg_chunks = p.S * 4 * p.LPR;
        p.JP = 4;
    } else if (p.JP == 3) {
        p.JP = 4;
    }
    p.segments = (C + p.seg_chunks - 1) / p.seg_chunks;
    const long rows_per_wg = (long)p.rows_per_wave * (kWaves / p.S);
    p.grid = (int)((N + rows_per_wg - 1) / rows_per_wg);
    p.rpg = (int)std::min<long>(rows_per_wg, N);
    if (M > 1 && k.path != Q4_PATH_INTEGER) {
        if (!plan_fm(p, M, N, K, k, split)) *ok = false;
        return p;
    }
    if (k.path == Q4_PATH_FMA) {
        if (k.waves && k.waves != kWaves) *ok = false;
        return p;
    }
    const bool integer = M == 1 ? plan_integer(p, N, K, k) : plan_integer_m(p, M, N, K, k);
    if (k.path == Q4_PATH_INTEGER && !integer) *ok = false;
    return p;
}

// Geometries fixed by gemv_q4_set_geometry, looked up by exact shape.
struct Override {
    int M, N, K, g;
    Knobs k;
};
constexpr int kMaxOverrides = 256;
Override g_over[kMaxOverrides];
int g_n_over = 0;
// Callers on several threads: launches read the table under a shared lock,
// gemv_q4_set_geometry / gemv_q4_clear_geometry write it under an exclusive
// one, so a launch sees a shape's setting either before or after a change,
// never half of one.
std::shared_mutex g_over_mutex;

Geometry plan(int M, int N, int K, int g, bool split = false) {
    Knobs k;
    bool found = false;
    {
        std::shared_lock<std::shared_mutex> lock(g_over_mutex);
        for (int i = 0; i < g_n_over; ++i) {
            const Override &o = g_over[i];
            if (o.M == M && o.N == N && o.K == K && o.g == g) {
                k = o.k;
                found = true;
                break;
            }
        }
    }
    if (found) {
        bool ok = true;
        const Geometry p = plan_with(M, N, K, k, &ok, split);
        if (ok) return p;
    }
    bool ok = true;
    return plan_with(M, N, K, Knobs{}, &ok, split);
}

// Longest row a call accepts: every per-lane and per-wavefront byte offset
// (x up to 8 rows, a wavefront's rows of codes, scales and zero points)
// then fits the 32-bit offsets and ranges of the buffer loads.
constexpr int kMaxK = 1 << 24;

int validate(int M, int N, int K, int g) {
    if (M < 1 || M > 8 || N < 0 || K <= 0 || K > kMaxK) return Q4_EINVAL;
    if (g != 32 && g != 128) return Q4_EINVAL;
    if (K < g || K % g != 0) return Q4_EINVAL;
    return Q4_OK;
}

// LDS bytes a launch needs: the x segment plus, with a K-split, one partial
// sum per (wavefront, row, m).
size_t lds_bytes(const Geometry &p) {
    if (p.fm)                   // x segment, partial sums
        return (size_t)p.M * p.seg_chunks * kFmStride * 4 + (size_t)p.waves * p.rows_per_wave * p.M * 4;
    if (p.integer && p.M > 1)   // records, residual pool, partial sums, pool counter
        return (size_t)p.M * p.seg_chunks * kIW * 4 + (size_t)p.pool * 64 +
               (size_t)p.waves * p.rows_per_wave * p.mp * 4 + 16;
    if (p.integer)              // records, a residual slot per half chunk, partial sums
        return (size_t)p.seg_chunks * (kIW * 4 + 128) +
               (p.S > 1 ? (size_t)p.waves * p.rows_per_wave * 4 : 0);
    size_t b = (size_t)p.M * p.seg_chunks * kXStride * sizeof(float);
    if (p.S > 1) b += (size_t)kWaves * p.rows_per_wave * p.M * sizeof(float);
    return b;
}

template <int M, int LPR, int JP>
void launch(const Geometry &p, const float *x, const uint8_t *wq, const uint16_t *scales,
            const uint8_t *zeros, float *y, int N, int K, int gshift, hipStream_t st) {
    if constexpr (M == 1 && LPR < 64) {
        if (p.fma_r == 2) {
            hipLaunchKernelGGL((gemv_q4_kernel<1, LPR, JP, 2>), dim3(p.grid), dim3(kBlock), lds_bytes(p), st,
                               x, wq, scales, zeros, y, N, K, gshift, p.S, p.seg_chunks, p.epi);
            return;
        }
    }
    hipLaunchKernelGGL((gemv_q4_kernel<M, LPR, JP, row_slots(M)>), dim3(p.grid), dim3(kBlock),
                       lds_bytes(p), st, x, wq, scales, zeros, y, N, K, gshift, p.S, p.seg_chunks, p.epi);
}

template <int M, int LPR>
void dispatch_jp(const Geometry &p, const float *x, const uint8_t *wq, const uint16_t *scales,
                 const uint8_t *zeros, float *y, int N, int K, int gshift, hipStream_t st) {
    switch (p.JP) {
    case 1: launch<M, LPR, 1>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    case 2: launch<M, LPR, 2>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    default: launch<M, LPR, 4>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    }
}

template <int W, int JP, int S, bool MULTI, int LPR = 64, int RS = row_slots(1)>
void launch_integer(const Geometry &p, const float *x, const uint8_t *wq, const uint16_t *scales,
                    const uint8_t *zeros, float *y, int N, int K, int gshift, hipStream_t st) {
    if constexpr (S == 1) {
        if (p.swi) {
            hipLaunchKernelGGL((gemv_q4_int_kernel<W, LPR, JP, RS, S, MULTI, true>), dim3(p.grid),
                               dim3(W * 64), lds_bytes(p), st, x, wq, scales, zeros, y, N, K, gshift, p.rpg, 0,
                               p.swi->wq, p.swi->scales, p.swi->zeros);
            return;
        }
    }
    hipLaunchKernelGGL((gemv_q4_int_kernel<W, LPR, JP, RS, S, MULTI>), dim3(p.grid), dim3(W * 64),
                       lds_bytes(p), st, x, wq, scales, zeros, y, N, K, gshift, p.rpg, p.epi,
                       nullptr, nullptr, nullptr);
}

template <int W, int S>
void dispatch_integer_jp(const Geometry &p, const float *x, const uint8_t *wq, const uint16_t *scales,
                         const uint8_t *zeros, float *y, int N, int K, int gshift, hipStream_t st) {
    if constexpr (S == 1) {
        if (p.LPR == 32) {   // two rows per load instruction: 2 row slots (4 rows) or 4
            if (p.rows_per_wave == 4) launch_integer<W, 1, 1, false, 32, 2>(p, x, wq, scales, zeros, y, N, K, gshift, st);
            else launch_integer<W, 1, 1, false, 32>(p, x, wq, scales, zeros, y, N, K, gshift, st);
            return;
        }
    }
    const bool multi = K / 32 > W * (2 * kM1XV);
    switch (p.JP) {
    case 1:
        if (multi) launch_integer<W, 1, S, true>(p, x, wq, scales, zeros, y, N, K, gshift, st);
        else launch_integer<W, 1, S, false>(p, x, wq, scales, zeros, y, N, K, gshift, st);
        break;
    case 2:
        if (multi) launch_integer<W, 2, S, true>(p, x, wq, scales, zeros, y, N, K, gshift, st);
        else launch_integer<W, 2, S, false>(p, x, wq, scales, zeros, y, N, K, gshift, st);
        break;
    default:   // a multi-pass kernel also serves a single pass
        launch_integer<W, 3, S, true>(p, x, wq, scales, zeros, y, N, K, gshift, st);
        break;
    }
}

template <int S>
void dispatch_integer(const Geometry &p, const float *x, const uint8_t *wq, const uint16_t *scales,
                      const uint8_t *zeros, float *y, int N, int K, int gshift, hipStream_t st) {
    if (p.waves == 16) dispatch_integer_jp<16, S>(p, x, wq, scales, zeros, y, N, K, gshift, st);
    else if (p.waves == 8) dispatch_integer_jp<8, S>(p, x, wq, scales, zeros, y, N, K, gshift, st);
    else dispatch_integer_jp<4, S>(p, x, wq, scales, zeros, y, N, K, gshift, st);
}

template <int W, int MP, int JP, int S>
void launch_intm(const Geometry &p, const float *x, const uint8_t *wq, const uint16_t *scales,
                 const uint8_t *zeros, float *y, int M, int N, int K, int gshift, hipStream_t st) {
    hipLaunchKernelGGL((gemv_q4_intm_kernel<W, MP, JP, 4, S>), dim3(p.grid), dim3(W * 64), lds_bytes(p), st,
                       x, wq, scales, zeros, y, M, N, K, gshift, p.rpg, p.seg_chunks, p.pool, p.epi);
}

template <int W, int MP>
void dispatch_intm_mp(const Geometry &p, const float *x, const uint8_t *wq, const uint16_t *scales,
                      const uint8_t *zeros, float *y, int M, int N, int K, int gshift, hipStream_t st) {
    if (p.JP == 1) {
        switch (p.S) {
        case 1: launch_intm<W, MP, 1, 1>(p, x, wq, scales, zeros, y, M, N, K, gshift, st); break;
        case 2: launch_intm<W, MP, 1, 2>(p, x, wq, scales, zeros, y, M, N, K, gshift, st); break;
        default: launch_intm<W, MP, 1, 4>(p, x, wq, scales, zeros, y, M, N, K, gshift, st); break;
        }
    } else {
        switch (p.S) {
        case 1: launch_intm<W, MP, 2, 1>(p, x, wq, scales, zeros, y, M, N, K, gshift, st); break;
        case 2: launch_intm<W, MP, 2, 2>(p, x, wq, scales, zeros, y, M, N, K, gshift, st); break;
        default: launch_intm<W, MP, 2, 4>(p, x, wq, scales, zeros, y, M, N, K, gshift, st); break;
        }
    }
}

template <int MX, int S, int JP>
void launch_fm(const Geometry &p, const float *x, const uint8_t *wq, const uint16_t *scales,
               const uint8_t *zeros, float *y, int N, int K, int gshift, hipStream_t st) {
    hipLaunchKernelGGL((gemv_q4_fm_kernel<kFmW, MX, kFmR, kFmLPR, S, JP>), dim3(p.grid), dim3(kFmW * 64),
                       lds_bytes(p), st, x, wq, scales, zeros, y, N, K, gshift, p.rpg, p.seg_chunks, p.epi,
                       p.work, p.ks_wg == 8 ? 3 : (p.ks_wg == 4 ? 2 : (p.ks_wg == 2 ? 1 : 0)), p.kpart);
    if (p.ks_wg > 1) {
        const int MN = MX * N;   // the split is planned only for KS * N <= 16384
        hipLaunchKernelGGL(fm_sum_parts, dim3((MN + 255) / 256), dim3(256), 0, st, y, p.work, MN, p.ks_wg, p.epi);
    }
}

template <int MX, int S>
void dispatch_fm_jp(const Geometry &p, const float *x, const uint8_t *wq, const uint16_t *scales,
                    const uint8_t *zeros, float *y, int N, int K, int gshift, hipStream_t st) {
    switch (p.JP) {
    case 2: launch_fm<MX, S, 2>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    case 4: launch_fm<MX, S, 4>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    case 8: launch_fm<MX, S, 8>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    default:
        if constexpr (fm_jp_max(MX) >= 16) launch_fm<MX, S, 16>(p, x, wq, scales, zeros, y, N, K, gshift, st);
        break;
    }
}

template <int MX>
void dispatch_fm_s(const Geometry &p, const float *x, const uint8_t *wq, const uint16_t *scales,
                   const uint8_t *zeros, float *y, int N, int K, int gshift, hipStream_t st) {
    switch (p.S) {
    case 1: dispatch_fm_jp<MX, 1>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    case 2: dispatch_fm_jp<MX, 2>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    default: dispatch_fm_jp<MX, 4>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    }
}

void dispatch_fm(const Geometry &p, const float *x, const uint8_t *wq, const uint16_t *scales,
                 const uint8_t *zeros, float *y, int M, int N, int K, int gshift, hipStream_t st) {
    switch (M) {
    case 2: dispatch_fm_s<2>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    case 3: dispatch_fm_s<3>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    case 4: dispatch_fm_s<4>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    case 5: dispatch_fm_s<5>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    case 6: dispatch_fm_s<6>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    case 7: dispatch_fm_s<7>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    default: dispatch_fm_s<8>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    }
}

void dispatch_intm(const Geometry &p, const float *x, const uint8_t *wq, const uint16_t *scales,
                   const uint8_t *zeros, float *y, int M, int N, int K, int gshift, hipStream_t st) {
    switch (p.mp) {
    case 2: dispatch_intm_mp<8, 2>(p, x, wq, scales, zeros, y, M, N, K, gshift, st); break;
    case 4: dispatch_intm_mp<8, 4>(p, x, wq, scales, zeros, y, M, N, K, gshift, st); break;
    default: dispatch_intm_mp<16, 8>(p, x, wq, scales, zeros, y, M, N, K, gshift, st); break;
    }
}

template <int M>
void dispatch_lpr(const Geometry &p, const float *x, const uint8_t *wq, const uint16_t *scales,
                  const uint8_t *zeros, float *y, int N, int K, int gshift, hipStream_t st) {
    switch (p.LPR) {
    case 16: dispatch_jp<M, 16>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    case 32: dispatch_jp<M, 32>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    default: dispatch_jp<M, 64>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    }
}

}  // namespace

extern "C" int gemv_q4_geometry(int M, int N, int K, int group_size, int *grid, int *block,
                                int *rows_per_wave, int *lanes_per_row, int *ksplit,
                                int *segments) {
    const int v = validate(M, N, K, group_size);
    if (v != Q4_OK) return v;
    const Geometry p = plan(M, N, K, group_size);
    if (grid) *grid = p.grid;
    if (block) *block = (p.integer || p.fm) ? p.waves * q4::kWave : kBlock;
    if (rows_per_wave) *rows_per_wave = p.rows_per_wave;
    if (lanes_per_row) *lanes_per_row = p.LPR;
    if (ksplit) *ksplit = p.S;
    if (segments) *segments = p.segments;
    return Q4_OK;
}

extern "C" int gemv_q4_path(int M, int N, int K, int group_size) {
    const int v = validate(M, N, K, group_size);
    if (v != Q4_OK) return v;
    return plan(M, N, K, group_size).integer ? Q4_PATH_INTEGER : Q4_PATH_FMA;
}

extern "C" int gemv_q4_set_geometry(int M, int N, int K, int group_size, int path, int waves,
                                    int ksplit) {
    const int v = validate(M, N, K, group_size);
    if (v != Q4_OK) return v;
    if ((path != Q4_PATH_FMA && path != Q4_PATH_INTEGER) ||
        (waves != 0 && waves != 4 && waves != 8 && waves != 16) ||
        (ksplit != 0 && ksplit != 1 && ksplit != 2 && ksplit != 4))
        return Q4_EINVAL;
    Knobs k;
    k.path = path;
    k.waves = waves;
    k.ksplit = ksplit;
    bool ok = true;
    plan_with(M, N, K, k, &ok);
    if (!ok) return Q4_EINVAL;
    std::unique_lock<std::shared_mutex> lock(g_over_mutex);
    int i = 0;
    while (i < g_n_over && !(g_over[i].M == M && g_over[i].N == N && g_over[i].K == K &&
                             g_over[i].g == group_size))
        ++i;
    if (i == kMaxOverrides) return Q4_EINVAL;
    g_over[i] = Override{M, N, K, group_size, k};
    if (i == g_n_over) ++g_n_over;
    return Q4_OK;
}

extern "C" int gemv_q4_clear_geometry(void) {
    std::unique_lock<std::shared_mutex> lock(g_over_mutex);
    g_n_over = 0;
    return Q4_OK;
}

namespace {

// Launches one GEMV of a validated, checked call (see gemv_q4, gemv_q4_swiglu).
int launch_gemv_q4(const float *x, const uint8_t *wq, const uint16_t *scales, const uint8_t *zeros,
                   float *y, int M, int N, int K, int group_size, int epi, void *stream,
                   const Q4Matrix *swi = nullptr, float *work = nullptr, size_t work_bytes = 0) {
    Geometry p = plan(M, N, K, group_size, work != nullptr);
    if (fm_work_bytes(p, N) > work_bytes) p = plan(M, N, K, group_size, false);
    p.epi = epi;
    p.swi = swi;
    p.work = work;
    const int gshift = group_size == 32 ? 0 : 2;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.fm) {
        dispatch_fm(p, x, wq, scales, zeros, y, M, N, K, gshift, st);
        return q4::launch_status();
    }
    if (p.integer && M > 1) {
        dispatch_intm(p, x, wq, scales, zeros, y, M, N, K, gshift, st);
        return q4::launch_status();
    }
    if (p.integer) {
        switch (p.S) {
        case 1: dispatch_integer<1>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
        case 2: dispatch_integer<2>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
        default: dispatch_integer<4>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
        }
        return q4::launch_status();
    }
    // The half-precision multiply-add kernel: one activation row only (the
    // planner sends 2 to 8 rows to the fp32 multiply-add or integer kernels).
    if (M != 1) return Q4_EINVAL;
    dispatch_lpr<1>(p, x, wq, scales, zeros, y, N, K, gshift, st);
    return q4::launch_status();
}

// Argument checks shared by the GEMV entry points.
int check_q4_args(const float *x, const uint8_t *wq, const uint16_t *scales, const uint8_t *zeros,
                  const float *y) {
    if (!x || !wq || !scales || !zeros || !y) return Q4_ENULL;
    if (!q4::aligned(x, 16) || !q4::aligned(wq, 16) || !q4::aligned(scales, 2) || !q4::aligned(y, 4))
        return Q4_EALIGN;
    return Q4_OK;
}

}  // namespace

extern "C" int gemv_q4(const float *x, const uint8_t *wq, const uint16_t *scales,
                       const uint8_t *zeros, float *y, int M, int N, int K, int group_size,
                       void *stream) {
    const int v = validate(M, N, K, group_size);
    if (v != Q4_OK) return v;
    if (N == 0) return Q4_OK;
    const int a = check_q4_args(x, wq, scales, zeros, y);
    if (a != Q4_OK) return a;
    const int dev = q4::check_device();
    if (dev != Q4_OK) return dev;
    return launch_gemv_q4(x, wq, scales, zeros, y, M, N, K, group_size, 0, stream);
}

extern "C" int gemv_q4_workspace_size(int M, int N, int K, int group_size, size_t *bytes) {
    const int v = validate(M, N, K, group_size);
    if (v != Q4_OK) return v;
    if (!bytes) return Q4_ENULL;
    *bytes = N == 0 ? 0 : fm_work_bytes(plan(M, N, K, group_size, true), N);
    return Q4_OK;
}

extern "C" int gemv_q4_ws(const float *x, const uint8_t *wq, const uint16_t *scales,
                          const uint8_t *zeros, float *y, int M, int N, int K, int group_size,
                          void *workspace, size_t workspace_bytes, void *stream) {
    const int v = validate(M, N, K, group_size);
    if (v != Q4_OK) return v;
    if (N == 0) return Q4_OK;
    const int a = check_q4_args(x, wq, scales, zeros, y);
    if (a != Q4_OK) return a;
    if (workspace && !q4::aligned(workspace, 16)) return Q4_EALIGN;
    const int dev = q4::check_device();
    if (dev != Q4_OK) return dev;
    return launch_gemv_q4(x, wq, scales, zeros, y, M, N, K, group_size, 0, stream, nullptr,
                          workspace ? static_cast<float *>(workspace) : nullptr,
                          workspace ? workspace_bytes : 0);
}

// ---------------------------------------------------------------- without allocation
// gemv_q4_static's workspace: a file-scope device array, one copy on each GPU
// the library runs on, held until the process ends.  512 KiB covers every
// K split the planner makes (KS * N <= 16384 at M <= 8, 4 bytes each).  Its
// contents carry nothing from one call to the next (partial sums are written
// before they are read), so nothing in it needs clearing.
namespace {
constexpr size_t kScratchBytes = 512 * 1024;
__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

// In host code `scratch` names a host-side stand-in, not the device array:
// each device's address is looked up once, with that device current, and
// kept here.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float *g_scratch_ptr[kMaxDevices];

float *scratch_on_current_device(int *status) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        *status = Q4_EDEVICE;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            *status = Q4_EDEVICE;
            return nullptr;
        }
        g_scratch_ptr[dev] = static_cast<float *>(ptr);
    }
    return g_scratch_ptr[dev];
}
}  // namespace

extern "C" int gemv_q4_static(const float *x, const uint8_t *wq, const uint16_t *scales,
                              const uint8_t *zeros, float *y, int M, int N, int K, int group_size,
                              void *stream) {
    const int v = validate(M, N, K, group_size);
    if (v != Q4_OK) return v;
    if (N == 0) return Q4_OK;
    const int a = check_q4_args(x, wq, scales, zeros, y);
    if (a != Q4_OK) return a;
    const int dev = q4::check_device();
    if (dev != Q4_OK) return dev;
    const size_t need = fm_work_bytes(plan(M, N, K, group_size, true), N);
    if (need > kScratchBytes) return Q4_EINVAL;
    float *work = nullptr;
    if (need) {
        int status = Q4_OK;
        work = scratch_on_current_device(&status);
        if (!work) return status;
    }
    return launch_gemv_q4(x, wq, scales, zeros, y, M, N, K, group_size, 0, stream, nullptr, work,
                          work ? kScratchBytes : 0);
}

extern "C" int gemv_q4_swiglu(const float *x, const uint8_t *wq_gate, const uint16_t *scales_gate,
                              const uint8_t *zeros_gate, const uint8_t *wq_up,
                              const uint16_t *scales_up, const uint8_t *zeros_up, float *y,
                              int M, int N, int K, int group_size, void *stream) {
    const int v = validate(M, N, K, group_size);
    if (v != Q4_OK) return v;
    if (N == 0) return Q4_OK;
    int a = check_q4_args(x, wq_gate, scales_gate, zeros_gate, y);
    if (a == Q4_OK) a = check_q4_args(x, wq_up, scales_up, zeros_up, y);
    if (a != Q4_OK) return a;
    const int dev = q4::check_device();
    if (dev != Q4_OK) return dev;
    // One activation row on the integer path without a K-split: one launch
    // that converts x once and runs the gate and then the up matrix.
    const Geometry p = plan(M, N, K, group_size);
    if (M == 1 && p.integer && p.S == 1) {
        const Q4Matrix up{wq_up, scales_up, zeros_up};
        return launch_gemv_q4(x, wq_gate, scales_gate, zeros_gate, y, M, N, K, group_size, 0, stream, &up);
    }
    const int r = launch_gemv_q4(x, wq_up, scales_up, zeros_up, y, M, N, K, group_size, 0, stream);
    if (r != Q4_OK) return r;
    return launch_gemv_q4(x, wq_gate, scales_gate, zeros_gate, y, M, N, K, group_size, 1, stream);
}
