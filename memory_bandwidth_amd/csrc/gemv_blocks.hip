// gemv_blocks.hip -- decode GEMV and dequantiser over the block quantisation
// formats of the cera page's decode benchmark (Q4_0, Q8_0, Q4_K, Q5_K, Q6_K),
// for gfx950.  The formats are the published GGML block formats of those
// names; their layouts are spelled out in q4blocks.h.
//
// Mapping onto CDNA4 (one activation row; a streaming dot product, no MFMA):
//   * A lane owns a 64-element unit of a row: two blocks of Q4_0 or Q8_0, or
//     a quarter of a 256-element K-format block.  64, 32 or 16 lanes share a
//     row, so one load instruction covers one, two or four rows, and
//     consecutive lanes read consecutive unit bytes of their row.  Rows with
//     more units than their lanes take several passes.
//   * Workgroups loop over blocks of rows; each stages x once in LDS, with
//     one float4 of padding per 16 so that 16 consecutive lanes reading their
//     units' slices hit 16 different bank groups, and a lane keeps its
//     unit's 64 x values in registers while they stay the same.  The loads
//     of the next block are issued before the arithmetic of the current one.
//   * The default launch gives each workgroup one row block in one pass.
//     That kernel keeps no second set of loads, and Q4_0 / Q4_K lanes hold
//     only the 32 x values of the run they are on, with the sums of x of the
//     Q4_K min term formed once per workgroup in LDS: 55-70 VGPRs, so that
//     all seven wavefronts per SIMD of a 4096 -> 14336 launch are resident
//     at once (162 VGPRs, three at a time, before).
//   * Unit bytes come in with dword-aligned buffer loads.  Fields that start
//     2 bytes past a dword boundary (the first block of a Q4_0 or Q8_0 pair,
//     every odd Q6_K block) are shifted into place with v_alignbyte_b32;
//     every Q6_K load stays inside its own block.
//   * Each weight is an exact small integer -- the code minus its offset
//     (8 for Q4_0, 32 for Q6_K, none otherwise) -- times x, so a code equal
//     to its offset contributes exactly zero.  Q4_0, Q4_K and Q6_K form two
//     such integers at once in binary16 (a code OR 0x6400 is 1024 + code,
//     one v_pk_add_f16 removes 1024 + offset) and v_fma_mix_f32 multiplies
//     them by fp32 x; Q8_0 and Q5_K convert with v_bfe / v_cvt.  Sums run
//     in fp32 per 16 or 32 elements and take their block or sub-block scale
//     once; the Q4_K/Q5_K min term is dmin * m_j times the sub-block's sum
//     of x.
//   * The dequantiser decodes through the same per-format code and forms
//     each weight as fma(scale, integer, -min), one rounding of its exact
//     value.
#include "q4_common.h"
#include "q4_device.h"
#include "q4blocks.h"

#include <algorithm>
#include <atomic>

namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Buffer resource for a raw byte range: reads past `bytes` return zero.
__device__ __forceinline__ rsrc_t raw_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// Default cache policy: a lane's unit is not a whole cache line, so one load
// instruction touches each line of its stretch only in part and the unit's
// other loads find the line in cache.  (Loads marked non-temporal, the
// weights being read once, were 7-40% slower: the lines left the cache
// before the other loads of the stretch reached them.)
__device__ __forceinline__ u32x4_t ld128(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t ld32(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t ld16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

__device__ __forceinline__ float f16lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float f16hi(uint32_t v) { return f16lo(v >> 16); }

// Bytes sh .. sh+3 of the 8-byte little-endian pair (lo, hi).
__device__ __forceinline__ uint32_t realign(uint32_t lo, uint32_t hi, uint32_t sh) {
    return __builtin_amdgcn_alignbyte(hi, lo, sh);
}

// Signed field of `bits` bits at bit `at`, as a float (exact).  The builtin
// returns the sign-extended field in an unsigned type: convert it as int.
__device__ __forceinline__ float sfield(uint32_t v, int at, int bits) {
    return (float)(int)__builtin_amdgcn_sbfe(v, at, bits);
}
// Byte j of v as a float (v_cvt_f32_ubyte<j>).
__device__ __forceinline__ float ubyte(uint32_t v, int j) { return (float)((v >> (8 * j)) & 0xFFu); }

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// (a & m) | o in one VALU op (gfx9 VOP3 takes no literal, so the compiler
// would split it into v_and_b32 + v_or_b32).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(o));
    return r;
}
__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// Binary16 decoding of small codes: a code c in bits 0..9 of a half word OR
// 0x6400 is the binary16 value 1024 + c (1024 <= v < 2048 has unit spacing),
// so one v_and_or_b32 unpacks two codes and one v_pk_add_f16 subtracting
// 1024 + offset leaves the exact integers c - offset; v_fma_mix_f32 then
// multiplies them by the fp32 x.  A code in bits 4..7 gives 1024 + 16 c, and
// 16 (c - offset) after the subtraction, also exact.
constexpr uint32_t kMagic = 0x64006400u;

// ---------------------------------------------------------------------------
// Per-format unit decoding.  For unit u of a row starting at byte `ro` of a
// buffer resource:
//   load(raw, rs, ro, u)    issues the unit's loads
//   xstart(u, run)          first element of run 0 / run 1 (32 elements each)
//                           of the lane's 64 x values
//   affine(raw, u, a, b)    weight of lane element e = a[e/16] * v + b[e/16]
//                           (b = -dmin * m_j, or -0 where there is no min)
//   visit(raw, u, fn)       fn(e, v) for e = 0..63 with v the exact integer
//   dot(raw, u, xv, dk)     (formats with kDot) dk[k] = sum over lane
//                           elements 16k .. 16k + 15 of v * xv[e], the same
//                           products as visit, decoded two at a time
//   dot_half<R>(raws, u, x32, d, h)
//                           (formats with kHalf) the same sums for k = 2h,
//                           2h + 1 of every row slot into d[r][k], from the
//                           32 x values of run h alone
// kMin: the format has a min term (b != -0).  kMaxR: the most row slots per
// lane that compile without spilling.
// ---------------------------------------------------------------------------

struct FmtQ4_0 {
    static constexpr int kMaxR = 4;   // row slots per lane without spilling
    static constexpr bool kMin = false;
    static constexpr bool kDot = true;
    static constexpr bool kHalf = true;
    struct Raw { uint32_t v[9]; };
    __device__ static void load(Raw &r, rsrc_t rs, uint32_t ro, int u) {
        const uint32_t o = ro + 36u * (uint32_t)u;      // two 18-byte blocks
        const u32x4_t a = ld128(rs, o), b = ld128(rs, o + 16);
        r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
        r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
        r.v[8] = ld32(rs, o + 32);
    }
    __device__ static int xstart(int u, int run) { return 64 * u + 32 * run; }
    __device__ static void affine(const Raw &r, int, float (&a)[4], float (&b)[4]) {
        const float dA = f16lo(r.v[0]), dB = f16hi(r.v[4]);
        a[0] = a[1] = dA;
        a[2] = a[3] = dB;
        b[0] = b[1] = b[2] = b[3] = -0.f;   // fma(a, v, -0) keeps the sign of a zero product
    }
    // dk[k]: sums over lane elements 16k .. 16k + 15 of (c - 8) x.
    __device__ static void dot(const Raw &r, int, const float (&xv)[64], float (&dk)[4]) {
        const half2_t z1 = as_h2(0x64086408u), z16 = as_h2(0x64806480u);   // 1024 + 8, 1024 + 128
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            float lo = 0.f, hi = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w = blk == 0 ? realign(r.v[i], r.v[i + 1], 2) : r.v[5 + i];
                const uint32_t w8 = w >> 8;
                const half2_t d0 = as_h2(and_or(w, 0x000F000Fu, kMagic)) - z1;    // elements 4i, 4i + 2
                const half2_t d1 = as_h2(and_or(w8, 0x000F000Fu, kMagic)) - z1;   // 4i + 1, 4i + 3
                const half2_t d2 = as_h2(and_or(w, 0x00F000F0u, kMagic)) - z16;   // 16 x (16 + 4i, 16 + 4i + 2)
                const half2_t d3 = as_h2(and_or(w8, 0x00F000F0u, kMagic)) - z16;  // 16 x (16 + 4i + 1, + 3)
                const float *x = xv + 32 * blk + 4 * i;
                lo = __builtin_fmaf((float)d0.x, x[0], lo);
                lo = __builtin_fmaf((float)d1.x, x[1], lo);
                lo = __builtin_fmaf((float)d0.y, x[2], lo);
                lo = __builtin_fmaf((float)d1.y, x[3], lo);
                hi = __builtin_fmaf((float)d2.x, x[16], hi);
                hi = __builtin_fmaf((float)d3.x, x[17], hi);
                hi = __builtin_fmaf((float)d2.y, x[18], hi);
                hi = __builtin_fmaf((float)d3.y, x[19], hi);
            }
            dk[2 * blk] = lo;
            dk[2 * blk + 1] = hi * 0.0625f;
        }
    }
    // Block blk of the pair for every row slot, one slot after another (the
    // low and high nibbles' chains interleave; one slot's codes are live at
    // a time).
    template <int R>
    __device__ static void dot_half(const Raw (&raw)[R], int, const float (&x32)[32], float (&d)[R][4], int blk) {
        const half2_t z1 = as_h2(0x64086408u), z16 = as_h2(0x64806480u);   // 1024 + 8, 1024 + 128
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float lo = 0.f, hi = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float *x = x32 + 4 * i;
                const uint32_t w = blk == 0 ? realign(raw[r].v[i], raw[r].v[i + 1], 2) : raw[r].v[5 + i];
                const uint32_t w8 = w >> 8;
                const half2_t d0 = as_h2(and_or(w, 0x000F000Fu, kMagic)) - z1;
                const half2_t d1 = as_h2(and_or(w8, 0x000F000Fu, kMagic)) - z1;
                const half2_t d2 = as_h2(and_or(w, 0x00F000F0u, kMagic)) - z16;
                const half2_t d3 = as_h2(and_or(w8, 0x00F000F0u, kMagic)) - z16;
                lo = __builtin_fmaf((float)d0.x, x[0], lo);
                lo = __builtin_fmaf((float)d1.x, x[1], lo);
                lo = __builtin_fmaf((float)d0.y, x[2], lo);
                lo = __builtin_fmaf((float)d1.y, x[3], lo);
                hi = __builtin_fmaf((float)d2.x, x[16], hi);
                hi = __builtin_fmaf((float)d3.x, x[17], hi);
                hi = __builtin_fmaf((float)d2.y, x[18], hi);
                hi = __builtin_fmaf((float)d3.y, x[19], hi);
            }
            d[r][2 * blk] = lo;
            d[r][2 * blk + 1] = hi * 0.0625f;
        }
    }
    template <class Fn> __device__ static void visit(const Raw &r, int, Fn &&fn) {
        // Nibble c ^ 8, sign-extended, is c - 8.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t ta = realign(r.v[i], r.v[i + 1], 2) ^ 0x88888888u;   // block A bytes 2..17
            const uint32_t tb = r.v[5 + i] ^ 0x88888888u;                        // block B bytes 20..35
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                fn(4 * i + j, sfield(ta, 8 * j, 4));
                fn(16 + 4 * i + j, sfield(ta, 8 * j + 4, 4));
                fn(32 + 4 * i + j, sfield(tb, 8 * j, 4));
                fn(48 + 4 * i + j, sfield(tb, 8 * j + 4, 4));
            }
        }
    }
};

struct FmtQ8_0 {
    static constexpr int kMaxR = 4;   // row slots per lane without spilling
    static constexpr bool kMin = false;
    static constexpr bool kDot = false;
    static constexpr bool kHalf = false;
    struct Raw { uint32_t v[17]; };
    __device__ static void load(Raw &r, rsrc_t rs, uint32_t ro, int u) {
        const uint32_t o = ro + 68u * (uint32_t)u;      // two 34-byte blocks
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4_t t = ld128(rs, o + 16 * i);
            r.v[4 * i] = t.x; r.v[4 * i + 1] = t.y; r.v[4 * i + 2] = t.z; r.v[4 * i + 3] = t.w;
        }
        r.v[16] = ld32(rs, o + 64);
    }
    __device__ static int xstart(int u, int run) { return 64 * u + 32 * run; }
    __device__ static void affine(const Raw &r, int, float (&a)[4], float (&b)[4]) {
        const float dA = f16lo(r.v[0]), dB = f16hi(r.v[8]);
        a[0] = a[1] = dA;
        a[2] = a[3] = dB;
        b[0] = b[1] = b[2] = b[3] = -0.f;   // fma(a, v, -0) keeps the sign of a zero product
    }
    template <class Fn> __device__ static void visit(const Raw &r, int, Fn &&fn) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t qa = realign(r.v[i], r.v[i + 1], 2);   // block A bytes 2..33
            const uint32_t qb = r.v[9 + i];                       // block B bytes 36..67
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                fn(4 * i + j, sfield(qa, 8 * j, 8));
                fn(32 + 4 * i + j, sfield(qb, 8 * j, 8));
            }
        }
    }
};

// Scales and mins of the lane's pair of sub-blocks 2p, 2p + 1 (p = u % 4),
// from header dwords 1..3 (bytes 4..15 of a Q4_K / Q5_K block: the 12 packed
// bytes).  Sub-blocks 2p and 2p + 1 use bytes 2(p % 2) and 2(p % 2) + 1 of
// each of those dwords, so one shift brings both into the low 16 bits:
//   p < 2:  s = b1 & 63,                       m = b2 & 63
//   p >= 2: s = (b3 & 15) | (b1 >> 6) << 4,    m = (b3 >> 4) | (b2 >> 6) << 4
// and the two 6-bit fields of each pair come out in bytes 0 and 1.
__device__ __forceinline__ void k_affine(const uint32_t *hd, int u, float (&a)[4], float (&b)[4]) {
    const uint32_t sh = (uint32_t)(u & 1) * 16u;
    const uint32_t b1 = hd[1] >> sh, b2 = hd[2] >> sh, b3 = hd[3] >> sh;
    const bool low = (u & 2) == 0;
    const uint32_t sw = low ? (b1 & 0x3F3Fu) : ((b3 & 0x0F0Fu) | ((b1 >> 2) & 0x3030u));
    const uint32_t mw = low ? (b2 & 0x3F3Fu) : (((b3 >> 4) & 0x0F0Fu) | ((b2 >> 2) & 0x3030u));
    const float d = f16lo(hd[0]), dmin = f16hi(hd[0]);
    a[0] = a[1] = d * ubyte(sw, 0);          // exact: 11 + 6 significant bits
    a[2] = a[3] = d * ubyte(sw, 1);
    b[0] = b[1] = -(dmin * ubyte(mw, 0));
    b[2] = b[3] = -(dmin * ubyte(mw, 1));
}

struct FmtQ4_K {
    static constexpr int kMaxR = 4;   // row slots per lane without spilling
    static constexpr bool kMin = true;
    static constexpr bool kDot = true;
    static constexpr bool kHalf = true;
    struct Raw { uint32_t v[12]; };
    __device__ static void load(Raw &r, rsrc_t rs, uint32_t ro, int u) {
        const uint32_t ob = ro + 144u * (uint32_t)(u >> 2);
        const uint32_t oq = ob + 16u + 32u * (uint32_t)(u & 3);
        const u32x4_t h = ld128(rs, ob), c0 = ld128(rs, oq), c1 = ld128(rs, oq + 16);
        r.v[0] = h.x; r.v[1] = h.y; r.v[2] = h.z; r.v[3] = h.w;
        r.v[4] = c0.x; r.v[5] = c0.y; r.v[6] = c0.z; r.v[7] = c0.w;
        r.v[8] = c1.x; r.v[9] = c1.y; r.v[10] = c1.z; r.v[11] = c1.w;
    }
    __device__ static int xstart(int u, int run) { return 64 * u + 32 * run; }
    __device__ static void affine(const Raw &r, int u, float (&a)[4], float (&b)[4]) {
        k_affine(r.v, u, a, b);
    }
    // dk[0], dk[1]: sub-block 2p (low nibbles), dk[2], dk[3]: sub-block 2p + 1.
    __device__ static void dot(const Raw &r, int, const float (&xv)[64], float (&dk)[4]) {
        const half2_t z = as_h2(kMagic);                 // 1024
        float hi[2] = {0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 2; ++k) dk[k] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t w = r.v[4 + i], w8 = w >> 8;
            const half2_t d0 = as_h2(and_or(w, 0x000F000Fu, kMagic)) - z;    // elements 4i, 4i + 2
            const half2_t d1 = as_h2(and_or(w8, 0x000F000Fu, kMagic)) - z;   // 4i + 1, 4i + 3
            const half2_t d2 = as_h2(and_or(w, 0x00F000F0u, kMagic)) - z;    // 16 x (32 + 4i, 32 + 4i + 2)
            const half2_t d3 = as_h2(and_or(w8, 0x00F000F0u, kMagic)) - z;   // 16 x (32 + 4i + 1, + 3)
            const int k = i >> 2;
            const float *xa = xv + 4 * i, *xb = xv + 32 + 4 * i;
            dk[k] = __builtin_fmaf((float)d0.x, xa[0], dk[k]);
            dk[k] = __builtin_fmaf((float)d1.x, xa[1], dk[k]);
            dk[k] = __builtin_fmaf((float)d0.y, xa[2], dk[k]);
            dk[k] = __builtin_fmaf((float)d1.y, xa[3], dk[k]);
            hi[k] = __builtin_fmaf((float)d2.x, xb[0], hi[k]);
            hi[k] = __builtin_fmaf((float)d3.x, xb[1], hi[k]);
            hi[k] = __builtin_fmaf((float)d2.y, xb[2], hi[k]);
            hi[k] = __builtin_fmaf((float)d3.y, xb[3], hi[k]);
        }
        dk[2] = hi[0] * 0.0625f;
        dk[3] = hi[1] * 0.0625f;
    }
    // h = 0: sub-block 2p (low nibbles) into d[r][0], d[r][1]; h = 1:
    // sub-block 2p + 1 (high nibbles) into d[r][2], d[r][3].  x32 holds the
    // sub-block's 32 x values; the row slots' chains interleave.
    template <int R>
    __device__ static void dot_half(const Raw (&raw)[R], int, const float (&x32)[32], float (&d)[R][4], int h) {
        const half2_t z = as_h2(kMagic);                 // 1024
        const uint32_t m = h ? 0x00F000F0u : 0x000F000Fu;
#pragma unroll
        for (int r = 0; r < R; ++r) d[r][2 * h] = d[r][2 * h + 1] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int k = 2 * h + (i >> 2);
            const float *xa = x32 + 4 * i;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t w = raw[r].v[4 + i], w8 = w >> 8;
                const half2_t d0 = as_h2(and_or(w, m, kMagic)) - z;    // elements 4i, 4i + 2 (16 x for h = 1)
                const half2_t d1 = as_h2(and_or(w8, m, kMagic)) - z;   // 4i + 1, 4i + 3
                d[r][k] = __builtin_fmaf((float)d0.x, xa[0], d[r][k]);
                d[r][k] = __builtin_fmaf((float)d1.x, xa[1], d[r][k]);
                d[r][k] = __builtin_fmaf((float)d0.y, xa[2], d[r][k]);
                d[r][k] = __builtin_fmaf((float)d1.y, xa[3], d[r][k]);
            }
        }
        if (h) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                d[r][2] *= 0.0625f;
                d[r][3] *= 0.0625f;
            }
        }
    }
    template <class Fn> __device__ static void visit(const Raw &r, int, Fn &&fn) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t lo = r.v[4 + i] & 0x0F0F0F0Fu;
            const uint32_t hi = (r.v[4 + i] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                fn(4 * i + j, ubyte(lo, j));
                fn(32 + 4 * i + j, ubyte(hi, j));
            }
        }
    }
};

struct FmtQ5_K {
    static constexpr int kMaxR = 2;   // row slots per lane without spilling
    static constexpr bool kMin = true;
    static constexpr bool kDot = false;
    static constexpr bool kHalf = false;
    struct Raw { uint32_t v[20]; };
    __device__ static void load(Raw &r, rsrc_t rs, uint32_t ro, int u) {
        const uint32_t ob = ro + 176u * (uint32_t)(u >> 2);
        const uint32_t oq = ob + 48u + 32u * (uint32_t)(u & 3);
        const u32x4_t h = ld128(rs, ob), e0 = ld128(rs, ob + 16), e1 = ld128(rs, ob + 32);
        const u32x4_t c0 = ld128(rs, oq), c1 = ld128(rs, oq + 16);
        r.v[0] = h.x; r.v[1] = h.y; r.v[2] = h.z; r.v[3] = h.w;
        r.v[4] = e0.x; r.v[5] = e0.y; r.v[6] = e0.z; r.v[7] = e0.w;
        r.v[8] = e1.x; r.v[9] = e1.y; r.v[10] = e1.z; r.v[11] = e1.w;
        r.v[12] = c0.x; r.v[13] = c0.y; r.v[14] = c0.z; r.v[15] = c0.w;
        r.v[16] = c1.x; r.v[17] = c1.y; r.v[18] = c1.z; r.v[19] = c1.w;
    }
    __device__ static int xstart(int u, int run) { return 64 * u + 32 * run; }
    __device__ static void affine(const Raw &r, int u, float (&a)[4], float (&b)[4]) {
        k_affine(r.v, u, a, b);
    }
    template <class Fn> __device__ static void visit(const Raw &r, int u, Fn &&fn) {
        const uint32_t p2 = 2u * (uint32_t)(u & 3);     // fifth bit of sub-block 2p, 2p + 1
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t q = r.v[12 + i], qh = r.v[4 + i];
            const uint32_t lo = (q & 0x0F0F0F0Fu) | (((qh >> p2) & 0x01010101u) << 4);
            const uint32_t hi = ((q >> 4) & 0x0F0F0F0Fu) | (((qh >> (p2 + 1)) & 0x01010101u) << 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                fn(4 * i + j, ubyte(lo, j));
                fn(32 + 4 * i + j, ubyte(hi, j));
            }
        }
    }
};

// Q6_K: unit u is block b = u / 4, half hf = (u / 2) % 2, side s = u % 2.
// The lane takes the 32 ql bytes 64 hf + 32 s .. +31 with both nibbles:
// low nibbles are elements 128 hf + 32 s + l (quarter s), high nibbles
// elements 128 hf + 64 + 32 s + l (quarter s + 2), and the 32 qh bytes of
// its half.  Blocks are 210 bytes, so a block may start 2 bytes past a
// dword boundary; its ql and qh runs are read as 9 aligned dwords each and
// shifted into place, its scales and d with 16-bit loads.
// The 6-bit codes of one Q6_K dword: bits 0..3 of byte j of the first result
// are the low nibble of ql byte j and bits 4, 5 the two top bits at bit s2 of
// qh byte j (quarter s), and the same from the high nibbles and bits s2 + 4
// for the second (quarter s + 2).  Bits 6, 7 of each byte are left over from
// the shifted qh and must be masked by the caller; one v_bfi_b32 merges the
// nibble with the shifted top bits, whose spill into the neighbouring byte's
// low nibble the merge discards.
__device__ __forceinline__ void q6_codes(uint32_t ql, uint32_t qh, uint32_t s2, uint32_t &ca,
                                         uint32_t &cb) {
    constexpr uint32_t m = 0x0F0F0F0Fu;
    ca = (ql & m) | ((qh << (4u - s2)) & ~m);
    cb = ((ql >> 4) & m) | ((qh >> s2) & ~m);
}

struct FmtQ6_K {
    static constexpr int kMaxR = 2;   // row slots per lane without spilling
    static constexpr bool kMin = false;
    static constexpr bool kDot = true;
    static constexpr bool kHalf = false;
    struct Raw { uint32_t l[9], h[9], sa, sb, d, sh; };
    __device__ static void load(Raw &r, rsrc_t rs, uint32_t ro, int u) {
        const uint32_t hf = (uint32_t)(u >> 1) & 1u, s = (uint32_t)u & 1u;
        const uint32_t ob = ro + 210u * (uint32_t)(u >> 2);
        const uint32_t o1 = ob + 64u * hf + 32u * s, o2 = ob + 128u + 32u * hf;
        const uint32_t a1 = o1 & ~3u, a2 = o2 & ~3u;   // o1, o2 differ by a multiple of 4
        r.sh = o1 & 3u;
        const u32x4_t l0 = ld128(rs, a1), l1 = ld128(rs, a1 + 16);
        const u32x4_t h0 = ld128(rs, a2), h1 = ld128(rs, a2 + 16);
        r.l[0] = l0.x; r.l[1] = l0.y; r.l[2] = l0.z; r.l[3] = l0.w;
        r.l[4] = l1.x; r.l[5] = l1.y; r.l[6] = l1.z; r.l[7] = l1.w;
        r.l[8] = ld32(rs, a1 + 32);
        r.h[0] = h0.x; r.h[1] = h0.y; r.h[2] = h0.z; r.h[3] = h0.w;
        r.h[4] = h1.x; r.h[5] = h1.y; r.h[6] = h1.z; r.h[7] = h1.w;
        r.h[8] = ld32(rs, a2 + 32);
        r.sa = ld16(rs, ob + 192u + 8u * hf + 2u * s);   // scales of quarter s, both 16-element halves
        r.sb = ld16(rs, ob + 196u + 8u * hf + 2u * s);   // scales of quarter s + 2
        r.d = ld16(rs, ob + 208u);
    }
    __device__ static int xstart(int u, int run) {
        return 256 * (u >> 2) + 128 * ((u >> 1) & 1) + 32 * (u & 1) + 64 * run;
    }
    __device__ static void affine(const Raw &r, int, float (&a)[4], float (&b)[4]) {
        const float d = f16lo(r.d);
        a[0] = d * sfield(r.sa, 0, 8);     // exact: 11 + 8 significant bits
        a[1] = d * sfield(r.sa, 8, 8);
        a[2] = d * sfield(r.sb, 0, 8);
        a[3] = d * sfield(r.sb, 8, 8);
        b[0] = b[1] = b[2] = b[3] = -0.f;   // fma(a, v, -0) keeps the sign of a zero product
    }
    __device__ static void dot(const Raw &r, int u, const float (&xv)[64], float (&dk)[4]) {
        const uint32_t s2 = 2u * ((uint32_t)u & 1u);
        const half2_t z = as_h2(0x64206420u);   // 1024 + 32
#pragma unroll
        for (int k = 0; k < 4; ++k) dk[k] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t ql = realign(r.l[i], r.l[i + 1], r.sh);
            const uint32_t qh = realign(r.h[i], r.h[i + 1], r.sh);
            uint32_t ca, cb;
            q6_codes(ql, qh, s2, ca, cb);
            const half2_t a0 = as_h2(and_or(ca, 0x003F003Fu, kMagic)) - z;        // elements 4i, 4i + 2
            const half2_t a1 = as_h2(and_or(ca >> 8, 0x003F003Fu, kMagic)) - z;   // 4i + 1, 4i + 3
            const half2_t b0 = as_h2(and_or(cb, 0x003F003Fu, kMagic)) - z;        // 32 + 4i, ...
            const half2_t b1 = as_h2(and_or(cb >> 8, 0x003F003Fu, kMagic)) - z;
            const int ka = i >> 2, kb = 2 + (i >> 2);
            const float *xa = xv + 4 * i, *xb = xv + 32 + 4 * i;
            dk[ka] = __builtin_fmaf((float)a0.x, xa[0], dk[ka]);
            dk[ka] = __builtin_fmaf((float)a1.x, xa[1], dk[ka]);
            dk[ka] = __builtin_fmaf((float)a0.y, xa[2], dk[ka]);
            dk[ka] = __builtin_fmaf((float)a1.y, xa[3], dk[ka]);
            dk[kb] = __builtin_fmaf((float)b0.x, xb[0], dk[kb]);
            dk[kb] = __builtin_fmaf((float)b1.x, xb[1], dk[kb]);
            dk[kb] = __builtin_fmaf((float)b0.y, xb[2], dk[kb]);
            dk[kb] = __builtin_fmaf((float)b1.y, xb[3], dk[kb]);
        }
    }
    template <class Fn> __device__ static void visit(const Raw &r, int u, Fn &&fn) {
        const uint32_t s2 = 2u * ((uint32_t)u & 1u);
        // A 6-bit code c ^ 32, sign-extended, is c - 32.
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t ql = realign(r.l[i], r.l[i + 1], r.sh);
            const uint32_t qh = realign(r.h[i], r.h[i + 1], r.sh);
            uint32_t ca, cb;
            q6_codes(ql, qh, s2, ca, cb);
            ca ^= 0x20202020u;
            cb ^= 0x20202020u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                fn(4 * i + j, sfield(ca, 8 * j, 6));
                fn(32 + 4 * i + j, sfield(cb, 8 * j, 6));
            }
        }
    }
};

// ---------------------------------------------------------------------------
// GEMV kernel.
//
// LPR lanes share a row: a row's units are spread over LPR lanes (64, or 32
// and 16 for rows of at most 32 or 16 units, so that one load instruction
// covers RG = 64 / LPR rows).  A lane has R row slots, a wavefront RPW =
// R * RG rows and a workgroup of W wavefronts a block of W * RPW rows.
// Workgroups stride over the row blocks, staging x in LDS once; a block with
// more units than LPR takes several passes, each an item of the workgroup's
// loop.  The loads of the next item are issued before the arithmetic of the
// current one.
// ---------------------------------------------------------------------------

// LDS slot of x's float4 number f: one float4 of padding after every 16.
__device__ __forceinline__ int xslot(int f) { return f + (f >> 4); }

template <class T, int R, int W, int LPR, bool ONE>
__global__ __launch_bounds__(W * 64) void gemv_blk_kernel(const float *__restrict__ x,
                                                          const uint8_t *__restrict__ w,
                                                          float *__restrict__ y, int N, int K,
                                                          uint32_t RB) {
    constexpr int RG = 64 / LPR;
    constexpr int RPW = R * RG;
    constexpr int RPB = RPW * W;
    extern __shared__ float blds[];
    f32x4_t *xs = reinterpret_cast<f32x4_t *>(blds);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = LPR == 64 ? 0 : lane / LPR;      // row of the lane within a load instruction
    const int ul = LPR == 64 ? lane : lane % LPR;  // unit of the lane within a pass
    const int U = K >> 6;                          // units per row
    const int P = (U + LPR - 1) / LPR;             // passes per row block
    const int nblk = (N + RPB - 1) / RPB;
    const int nitems = (nblk - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x * P;

    // Issues the loads of item `it` (row block, pass) into raw.  Rows past N
    // re-read row N - 1 and units past U re-read unit U - 1; neither is used.
    auto load_item = [&](typename T::Raw (&raw)[R], int it) {
        const int blk = (int)blockIdx.x + it / P * (int)gridDim.x;
        const int pass = it % P;
        const int rb0 = blk * RPB + wave * RPW;
        const int rbase = min(rb0, N - 1);
        const uint64_t byte0 = (uint64_t)rbase * RB;
        const uint32_t delta = (uint32_t)(byte0 & 15u);
        const uint64_t span = (uint64_t)(N - rbase) * RB + delta;
        const rsrc_t rs = raw_rsrc(w + (byte0 - delta), (uint32_t)std::min<uint64_t>(span, 0xFFFFFFFFull));
        const int uc = min(pass * LPR + ul, U - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t ro = delta + (uint32_t)(min(rb0 + r * RG + g, N - 1) - rbase) * RB;
            T::load(raw[r], rs, ro, uc);
        }
    };

    // x: the first 4096 elements go to registers ahead of the first item's
    // loads (loads retire in issue order), the rest after them.
    const f32x4_t *x4 = reinterpret_cast<const f32x4_t *>(x);
    const int nx4 = K >> 2;
    constexpr int XB = 1024 / (W * 64);
    f32x4_t xr[XB];
#pragma unroll
    for (int t = 0; t < XB; ++t) {
        const int i = t * W * 64 + tid;
        xr[t] = i < nx4 ? x4[i] : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    __builtin_amdgcn_sched_barrier(0);
    typename T::Raw ra[R], rb[R];
    load_item(ra, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < XB; ++t) {
        const int i = t * W * 64 + tid;
        if (i < nx4) xs[xslot(i)] = xr[t];
    }
    for (int i = XB * W * 64 + tid; i < nx4; i += W * 64) xs[xslot(i)] = x4[i];
    __syncthreads();
    // One item per workgroup (ONE): formats with kHalf decode a run of the
    // unit at a time with only its 32 x values in registers, and keep no
    // second set of loads, so that every wavefront of a CU fits at once.
    // A min term's sums of x over each 16 consecutive elements are formed
    // once per workgroup here (one per thread at K = 4096 and 256 threads),
    // and read after a barrier that follows the dot products.
    constexpr bool HALF = ONE && T::kHalf;
    float *sxs = reinterpret_cast<float *>(xs + xslot(nx4 - 1) + 1);
    if constexpr (HALF && T::kMin) {
        for (int i = tid; i < (K >> 4); i += W * 64) {
            float t = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4_t v = xs[xslot(4 * i + q)];
                t += v.x; t += v.y; t += v.z; t += v.w;
            }
            sxs[i] = t;
        }
    }

    float xv[64], sx[4];
    int xpass = -1;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;

    // Arithmetic of item `it` on raw; after a block's last pass, the row sums
    // are reduced across the LPR lanes of each row and stored.
    auto process = [&](const typename T::Raw (&raw)[R], int it) {
        const int blk = (int)blockIdx.x + it / P * (int)gridDim.x;
        const int pass = it % P;
        const int u = pass * LPR + ul;
        const int uc = min(u, U - 1);
        if constexpr (HALF) {
            float a[R][4], b[R][4], d[R][4];
            if (u < U) {
#pragma unroll
                for (int r = 0; r < R; ++r) T::affine(raw[r], uc, a[r], b[r]);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    __builtin_amdgcn_sched_barrier(0);   // run h's x reads stay after run h - 1's arithmetic
                    float x32[32];
                    const int f = T::xstart(uc, h) >> 2;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const f32x4_t v = xs[xslot(f + i)];
                        x32[4 * i] = v.x; x32[4 * i + 1] = v.y; x32[4 * i + 2] = v.z; x32[4 * i + 3] = v.w;
                    }
                    T::template dot_half<R>(raw, uc, x32, d, h);
                    if constexpr (!T::kMin) {
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            float c = acc[r];
                            c = __builtin_fmaf(a[r][2 * h], d[r][2 * h], c);
                            c = __builtin_fmaf(a[r][2 * h + 1], d[r][2 * h + 1], c);
                            acc[r] = c;
                        }
                    }
                }
            }
            if constexpr (T::kMin) {
                __syncthreads();                      // the sums of x are written
                if (u < U) {
                    const f32x4_t v = *reinterpret_cast<const f32x4_t *>(sxs + 4 * uc);
                    const float s4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        float c = acc[r];
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            c = __builtin_fmaf(a[r][k], d[r][k], c);
                            c = __builtin_fmaf(b[r][k], s4[k], c);
                        }
                        acc[r] = c;
                    }
                }
            }
        } else if (pass != xpass) {
            xpass = pass;
#pragma unroll
            for (int run = 0; run < 2; ++run) {
                const int f = T::xstart(uc, run) >> 2;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const f32x4_t v = xs[xslot(f + i)];
                    xv[32 * run + 4 * i] = v.x;
                    xv[32 * run + 4 * i + 1] = v.y;
                    xv[32 * run + 4 * i + 2] = v.z;
                    xv[32 * run + 4 * i + 3] = v.w;
                }
            }
            if constexpr (T::kMin) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    float t = 0.f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) t += xv[16 * k + i];
                    sx[k] = t;
                }
            }
        }
        if (!HALF && u < U) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float a[4], b[4];
                T::affine(raw[r], uc, a, b);
                float dk[4] = {0.f, 0.f, 0.f, 0.f};
                if constexpr (T::kDot)
                    T::dot(raw[r], uc, xv, dk);
                else
                    T::visit(raw[r], uc, [&](int e, float v) { dk[e >> 4] = __builtin_fmaf(v, xv[e], dk[e >> 4]); });
                float c = acc[r];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    c = __builtin_fmaf(a[k], dk[k], c);
                    if constexpr (T::kMin) c = __builtin_fmaf(b[k], sx[k], c);
                }
                acc[r] = c;
            }
        }
        if (pass == P - 1) {
            const int rb0 = blk * RPB + wave * RPW;
            if constexpr (LPR == 64) {
                constexpr int NQ = (R + 3) / 4;
                float out[NQ];
                q4::wave_reduce_rows<R>(acc, out);
                const int h = lane >> 4;
                if ((lane & 15) == 0 && (R >= 4 || (h & (R == 2 ? 1 : 3)) == 0)) {
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        const int row = rb0 + q4::reduced_row<R>(q, h);
                        if (row < N) y[row] = out[q];
                    }
                }
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float s = q4::group_sum<LPR>(acc[r]);
                    const int row = rb0 + r * RG + g;
                    if (ul == 0 && row < N) y[row] = s;
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = 0.f;
        }
    };

    if constexpr (ONE) {             // one item per workgroup: no second set of loads
        process(ra, 0);
        return;
    }
    for (int it = 0; it < nitems; it += 2) {
        if (it + 1 < nitems) load_item(rb, it + 1);
        process(ra, it);
        if (it + 1 >= nitems) break;
        if (it + 2 < nitems) load_item(ra, it + 2);
        process(rb, it + 1);
    }
}

// ---------------------------------------------------------------------------
// Dequantiser: one thread per unit, 256 consecutive units per workgroup.
// ---------------------------------------------------------------------------

constexpr int kDqBlock = 256;

template <class T>
__global__ __launch_bounds__(kDqBlock) void dequant_blk_kernel(const uint8_t *__restrict__ w,
                                                               float *__restrict__ out, int N, int K,
                                                               uint32_t RB) {
    const int64_t U = K >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * kDqBlock;
    const int64_t t = t0 + threadIdx.x;
    const int64_t n0 = t0 / U;
    const int64_t nl = std::min<int64_t>((t0 + kDqBlock - 1) / U, N - 1);
    const uint64_t byte0 = (uint64_t)n0 * RB;
    const uint32_t delta = (uint32_t)(byte0 & 15u);
    const uint64_t span = (uint64_t)(nl - n0 + 1) * RB + delta;
    const rsrc_t wr = raw_rsrc(w + (byte0 - delta), (uint32_t)std::min<uint64_t>(span, 0xFFFFFFFFull));
    if (t >= (int64_t)N * U) return;
    const int64_t n = t / U;
    const int u = (int)(t - n * U);
    typename T::Raw raw;
    T::load(raw, wr, delta + (uint32_t)(n - n0) * RB, u);
    float a[4], b[4];
    T::affine(raw, u, a, b);
    float v[64];
    T::visit(raw, u, [&](int e, float c) { v[e] = __builtin_fmaf(a[e >> 4], c, b[e >> 4]); });
#pragma unroll
    for (int run = 0; run < 2; ++run) {
        f32x4_t *dst = reinterpret_cast<f32x4_t *>(out + n * K + T::xstart(u, run));
#pragma unroll
        for (int i = 0; i < 8; ++i)
            dst[i] = f32x4_t{v[32 * run + 4 * i], v[32 * run + 4 * i + 1], v[32 * run + 4 * i + 2],
                             v[32 * run + 4 * i + 3]};
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------

constexpr int kMaxK = 32768;

struct Geo { int elems, bytes; };

bool geometry_of(int f, Geo &g) {
    switch (f) {
    case BLK_Q4_0: g = {32, 18}; return true;
    case BLK_Q8_0: g = {32, 34}; return true;
    case BLK_Q4_K: g = {256, 144}; return true;
    case BLK_Q5_K: g = {256, 176}; return true;
    case BLK_Q6_K: g = {256, 210}; return true;
    default: return false;
    }
}

// Launch geometry of one format: rows per lane slot count R, wavefronts
// per workgroup W, and workgroups per CU G (the grid is at most G * CUs
// workgroups; 0 = one workgroup per row block).
// Defaults (measured on the 4096 -> 14336 stream and 1024 -> 65536 shapes)
// apply to shapes of at least 2 * CUs row blocks; smaller ones, latency-
// bound, take one row slot and 4 wavefronts, the most workgroups.  One
// workgroup per row block (G = 0) runs the one-item kernel, whose small
// register footprint lets every wavefront of a CU be resident at once;
// every format takes it (at the stream shape Q5_K 11.7 -> 10.8 us, Q6_K
// 13.9 -> 12.2 us, Q8_0 12.9 -> 12.5 us against looping over row blocks).
// A configuration set through gemv_block_set_config applies to every shape.
struct Cfg { int R, W, G; bool forced; };
constexpr int kCUs = 256;
constexpr Cfg kDefault[6] = {{0, 0, 0, false}, {2, 4, 0, false}, {1, 8, 0, false},
                             {2, 4, 0, false}, {2, 4, 0, false}, {1, 8, 0, false}};
constexpr Cfg kSmall = {1, 4, 0, false};
// The setting of each format, packed into one word so that a launch reads
// it whole while gemv_block_set_config changes it on another thread:
// R (bits 0-3), W (4-7), G (8-15), forced (16).
constexpr uint32_t pack_cfg(Cfg c) {
    return (uint32_t)c.R | (uint32_t)c.W << 4 | (uint32_t)c.G << 8 | (c.forced ? 1u << 16 : 0u);
}
inline Cfg unpack_cfg(uint32_t v) {
    return {(int)(v & 15u), (int)((v >> 4) & 15u), (int)((v >> 8) & 255u), ((v >> 16) & 1u) != 0};
}
std::atomic<uint32_t> g_cfg[6] = {pack_cfg(kDefault[0]), pack_cfg(kDefault[1]), pack_cfg(kDefault[2]),
                                  pack_cfg(kDefault[3]), pack_cfg(kDefault[4]), pack_cfg(kDefault[5])};

// Lanes per row: the fewest of 64, 32, 16 that hold a row's units.
int lanes_per_row(int K);

Cfg config_for(int format, int N, int K) {
    const Cfg c = unpack_cfg(g_cfg[format].load(std::memory_order_acquire));
    if (c.forced) return c;
    const int rpb = c.R * (64 / lanes_per_row(K)) * c.W;
    return (N + rpb - 1) / rpb < 2 * kCUs ? kSmall : c;
}

bool cfg_ok(int format, int R, int W, int G) {
    const int max_r = (format == BLK_Q5_K || format == BLK_Q6_K) ? 2 : 4;
    return (R == 1 || R == 2 || R == 4) && R <= max_r && (W == 4 || W == 8) && G >= 0 && G <= 64;
}

// Lanes per row: the fewest of 64, 32, 16 that hold a row's units.
int lanes_per_row(int K) {
    const int U = K >> 6;
    return U > 32 ? 64 : (U > 16 ? 32 : 16);
}

template <class T, int R, int W, int LPR>
void launch_l(Cfg c, const float *x, const uint8_t *w, float *y, int N, int K, uint32_t RB,
              hipStream_t st) {
    constexpr int RPB = R * (64 / LPR) * W;
    const int nblk = (N + RPB - 1) / RPB;
    const int grid = c.G > 0 ? std::min(nblk, c.G * kCUs) : nblk;
    const size_t lds = (size_t)(K / 4 + K / 64) * 16 + (size_t)(K / 16) * 4;   // x, then its sums of 16
    if (grid == nblk && K / 64 <= LPR)   // every workgroup has exactly one item (one block, one pass)
        hipLaunchKernelGGL((gemv_blk_kernel<T, R, W, LPR, true>), dim3(grid), dim3(W * 64), lds, st, x, w, y, N,
                           K, RB);
    else
        hipLaunchKernelGGL((gemv_blk_kernel<T, R, W, LPR, false>), dim3(grid), dim3(W * 64), lds, st, x, w, y,
                           N, K, RB);
}

template <class T, int R, int W>
void launch_w(Cfg c, const float *x, const uint8_t *w, float *y, int N, int K, uint32_t RB,
              hipStream_t st) {
    switch (lanes_per_row(K)) {
    case 16: launch_l<T, R, W, 16>(c, x, w, y, N, K, RB, st); break;
    case 32: launch_l<T, R, W, 32>(c, x, w, y, N, K, RB, st); break;
    default: launch_l<T, R, W, 64>(c, x, w, y, N, K, RB, st); break;
    }
}

template <class T>
void launch_fmt(Cfg c, const float *x, const uint8_t *w, float *y, int N, int K, uint32_t RB,
                hipStream_t st) {
    if (c.R == 4) {
        if constexpr (T::kMaxR >= 4) {
            if (c.W == 8) launch_w<T, 4, 8>(c, x, w, y, N, K, RB, st);
            else launch_w<T, 4, 4>(c, x, w, y, N, K, RB, st);
        }
    } else if (c.W == 8) {
        if (c.R == 1) launch_w<T, 1, 8>(c, x, w, y, N, K, RB, st);
        else launch_w<T, 2, 8>(c, x, w, y, N, K, RB, st);
    } else {
        if (c.R == 1) launch_w<T, 1, 4>(c, x, w, y, N, K, RB, st);
        else launch_w<T, 2, 4>(c, x, w, y, N, K, RB, st);
    }
}

template <class T>
void launch_dq(const uint8_t *w, float *out, int N, int K, uint32_t RB, hipStream_t st) {
    const int64_t units = (int64_t)N * (K >> 6);
    const int grid = (int)((units + kDqBlock - 1) / kDqBlock);
    hipLaunchKernelGGL((dequant_blk_kernel<T>), dim3(grid), dim3(kDqBlock), 0, st, w, out, N, K, RB);
}

int check_k(int K) { return (K >= 256 && K <= kMaxK && K % 256 == 0) ? Q4_OK : Q4_EINVAL; }

}  // namespace

extern "C" int block_geometry(int format, int *elems, int *bytes) {
    if (!elems || !bytes) return Q4_ENULL;
    Geo g;
    if (!geometry_of(format, g)) return Q4_EINVAL;
    *elems = g.elems;
    *bytes = g.bytes;
    return Q4_OK;
}

extern "C" int gemv_block(int format, const float *x, const uint8_t *w, float *y, int M, int N,
                          int K, void *stream) {
    Geo g;
    if (!geometry_of(format, g)) return Q4_EINVAL;
    if (M != 1 || N < 0 || check_k(K) != Q4_OK) return Q4_EINVAL;
    if (N == 0) return Q4_OK;
    if (!x || !w || !y) return Q4_ENULL;
    if (!q4::aligned(x, 16) || !q4::aligned(w, 16) || !q4::aligned(y, 4)) return Q4_EALIGN;
    if (int st = q4::check_device(); st != Q4_OK) return st;
    const uint32_t RB = (uint32_t)(K / g.elems * g.bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Cfg c = config_for(format, N, K);
    switch (format) {
    case BLK_Q4_0: launch_fmt<FmtQ4_0>(c, x, w, y, N, K, RB, st); break;
    case BLK_Q8_0: launch_fmt<FmtQ8_0>(c, x, w, y, N, K, RB, st); break;
    case BLK_Q4_K: launch_fmt<FmtQ4_K>(c, x, w, y, N, K, RB, st); break;
    case BLK_Q5_K: launch_fmt<FmtQ5_K>(c, x, w, y, N, K, RB, st); break;
    default: launch_fmt<FmtQ6_K>(c, x, w, y, N, K, RB, st); break;
    }
    return q4::launch_status();
}

extern "C" int dequant_block(int format, const uint8_t *w, float *w_out, int N, int K, void *stream) {
    Geo g;
    if (!geometry_of(format, g)) return Q4_EINVAL;
    if (N < 0 || check_k(K) != Q4_OK) return Q4_EINVAL;
    if (N == 0) return Q4_OK;
    if (!w || !w_out) return Q4_ENULL;
    if (!q4::aligned(w, 16) || !q4::aligned(w_out, 16)) return Q4_EALIGN;
    if (int st = q4::check_device(); st != Q4_OK) return st;
    const uint32_t RB = (uint32_t)(K / g.elems * g.bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (format) {
    case BLK_Q4_0: launch_dq<FmtQ4_0>(w, w_out, N, K, RB, st); break;
    case BLK_Q8_0: launch_dq<FmtQ8_0>(w, w_out, N, K, RB, st); break;
    case BLK_Q4_K: launch_dq<FmtQ4_K>(w, w_out, N, K, RB, st); break;
    case BLK_Q5_K: launch_dq<FmtQ5_K>(w, w_out, N, K, RB, st); break;
    default: launch_dq<FmtQ6_K>(w, w_out, N, K, RB, st); break;
    }
    return q4::launch_status();
}

extern "C" int gemv_block_set_config(int format, int rows_per_lane, int waves_per_group,
                                     int groups_per_cu) {
    Geo g;
    if (!geometry_of(format, g)) return Q4_EINVAL;
    if (rows_per_lane == 0 && waves_per_group == 0 && groups_per_cu == 0) {
        g_cfg[format].store(pack_cfg(kDefault[format]), std::memory_order_release);
        return Q4_OK;
    }
    if (!cfg_ok(format, rows_per_lane, waves_per_group, groups_per_cu)) return Q4_EINVAL;
    g_cfg[format].store(pack_cfg({rows_per_lane, waves_per_group, groups_per_cu, true}), std::memory_order_release);
    return Q4_OK;
}

extern "C" int gemv_block_config(int format, int *rows_per_lane, int *waves_per_group,
                                 int *groups_per_cu) {
    if (!rows_per_lane || !waves_per_group || !groups_per_cu) return Q4_ENULL;
    Geo g;
    if (!geometry_of(format, g)) return Q4_EINVAL;
    const Cfg c = unpack_cfg(g_cfg[format].load(std::memory_order_acquire));
    *rows_per_lane = c.R;
    *waves_per_group = c.W;
    *groups_per_cu = c.G;
    return Q4_OK;
}
