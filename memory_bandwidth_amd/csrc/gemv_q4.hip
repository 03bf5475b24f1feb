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

// Cache-policy bits of a buffer load: non-temporal, for the weight stream
// that is read once.
constexpr int kNonTemporal = 2;

// M: activation rows.  LPR: lanes per output row.  JP: chunk positions per
// lane per segment (a lane's chunks are LPR apart).  R: row slots per wave.
//
// Addressing: pointers are wave-uniform bases (SGPRs) plus one 32-bit
// per-lane offset shared by all rows of the wave when LPR = 64.
template <int M, int LPR, int JP, int R>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 4))) void gemv_q4_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ wq,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    float *__restrict__ y, int N, int K, int gshift, int S, int seg_chunks) {
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
    const __amdgpu_buffer_rsrc_t wq_r = raw_rsrc(wq + (size_t)row_base * RB,
        (uint32_t)std::min<uint64_t>((uint64_t)rows_left * RB, 0xFFFFFFFFull));
    const __amdgpu_buffer_rsrc_t sc_r = raw_rsrc(scales + (size_t)row_base * G, rows_left * (uint32_t)G * 2u);
    const __amdgpu_buffer_rsrc_t zp_r = raw_rsrc(zeros + (size_t)row_base * ZB, rows_left * (uint32_t)ZB);
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
                        for (int m = 0; m < M; ++m) y[(size_t)m * N + row] = out[m][q];
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
                    if (row < N) y[(size_t)m * N + row] = v;
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
                        for (int m = 0; m < M; ++m) y[(size_t)m * N + row] = acc[r][m];
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
                    if (row < N) y[(size_t)m * N + row] = v;
                }
            }
        }
    }
}

struct Geometry {
    int M, LPR, JP, S, seg_chunks, segments, grid, rows_per_wave;
};

// Chooses the launch geometry for a validated shape.
Geometry plan(int M, int N, int K, int g) {
    (void)g;
    Geometry p{};
    p.M = M;
    const int C = K / 32;
    p.LPR = C <= 16 ? 16 : (C <= 32 ? 32 : 64);
    const int R = row_slots(M);
    p.rows_per_wave = R * (q4::kWave / p.LPR);
    const long row_waves = ((long)N + p.rows_per_wave - 1) / p.rows_per_wave;
    // K-split, decided on the length of one x segment: enough wavefronts to
    // fill the chip (>= 2 per SIMD) and at most two chunk positions per lane,
    // while every split keeps a full lane sweep.
    const int seg_len = std::min(C, kLdsBytes / (M * kXStride * (int)sizeof(float)));
    p.S = 1;
    while (p.S < kWaves && 2 * p.S * p.LPR <= seg_len &&
           (row_waves * p.S < 2048 || (seg_len + p.S * p.LPR - 1) / (p.S * p.LPR) > 2))
        p.S *= 2;
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
    return p;
}

int validate(int M, int N, int K, int g) {
    if (M < 1 || M > 8 || N < 0 || K <= 0) return Q4_EINVAL;
    if (g != 32 && g != 128) return Q4_EINVAL;
    if (K < g || K % g != 0) return Q4_EINVAL;
    return Q4_OK;
}

// LDS bytes a launch needs: the x segment plus, with a K-split, one partial
// sum per (wavefront, row, m).
size_t lds_bytes(const Geometry &p) {
    size_t b = (size_t)p.M * p.seg_chunks * kXStride * sizeof(float);
    if (p.S > 1) b += (size_t)kWaves * p.rows_per_wave * p.M * sizeof(float);
    return b;
}

template <int M, int LPR, int JP>
void launch(const Geometry &p, const float *x, const uint8_t *wq, const uint16_t *scales,
            const uint8_t *zeros, float *y, int N, int K, int gshift, hipStream_t st) {
    hipLaunchKernelGGL((gemv_q4_kernel<M, LPR, JP, row_slots(M)>), dim3(p.grid), dim3(kBlock),
                       lds_bytes(p), st, x, wq, scales, zeros, y, N, K, gshift, p.S, p.seg_chunks);
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
    if (block) *block = kBlock;
    if (rows_per_wave) *rows_per_wave = p.rows_per_wave;
    if (lanes_per_row) *lanes_per_row = p.LPR;
    if (ksplit) *ksplit = p.S;
    if (segments) *segments = p.segments;
    return Q4_OK;
}

extern "C" int gemv_q4(const float *x, const uint8_t *wq, const uint16_t *scales,
                       const uint8_t *zeros, float *y, int M, int N, int K, int group_size,
                       void *stream) {
    const int v = validate(M, N, K, group_size);
    if (v != Q4_OK) return v;
    if (N == 0) return Q4_OK;
    if (!x || !wq || !scales || !zeros || !y) return Q4_ENULL;
    if (!q4::aligned(x, 16) || !q4::aligned(wq, 16) || !q4::aligned(scales, 2) ||
        !q4::aligned(y, 4))
        return Q4_EALIGN;
    const int dev = q4::check_device();
    if (dev != Q4_OK) return dev;
    const Geometry p = plan(M, N, K, group_size);
    const int gshift = group_size == 32 ? 0 : 2;
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (M) {
    case 1: dispatch_lpr<1>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    case 2: dispatch_lpr<2>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    case 3: dispatch_lpr<3>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    case 4: dispatch_lpr<4>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    case 5: dispatch_lpr<5>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    case 6: dispatch_lpr<6>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    case 7: dispatch_lpr<7>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    default: dispatch_lpr<8>(p, x, wq, scales, zeros, y, N, K, gshift, st); break;
    }
    return q4::launch_status();
}
