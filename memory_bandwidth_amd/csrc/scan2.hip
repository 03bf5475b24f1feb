// scan2.hip -- the 2-bit corpus scan of the Refractometer page ("What each
// sweep measures", the scan sweep), for gfx950:
//
//     score[v, q] = sum_d lut[q, d, code(v, d)]
//
// over 2-bit codes packed 16 per little-endian u32 (see q4scan.h).
//
// Mapping onto CDNA4, following the page's knobs (workgroup size, the table
// in workgroup memory or in storage, vectors per thread):
//   * TPV adjacent threads share a vector, each scanning a contiguous 1/TPV
//     of its dimensions (the page's tail uses one thread per vector; on a
//     256-CU part 65,536 vectors then fill one wavefront per SIMD, too few
//     to hide LDS latency).  Codes come in 16-byte loads (64 dimensions),
//     the next chunk's load issued before the current chunk's lookups.
//   * With the table in LDS, every workgroup first stages it as
//     [d][code][query] float4 groups (queries padded to a multiple of 4), so
//     one ds_read_b128 returns four queries' entries for one (d, code).  The
//     lanes of one part of the dimensions are at the same dimension and
//     address at most four distinct 16-byte groups (broadcast reads); the
//     parts are offset from one another by padding, so that they fall in
//     different banks.
//   * With the table read from memory, each lookup is a 4-byte load that
//     the caches serve (the page's "storage" variant).
//   * Sums are fp32, per vector and query, in increasing d.
#include "q4_common.h"
#include "q4scan.h"

#include <algorithm>

namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Q4: groups of four queries (1 or 2).  VPT: vectors per thread.  TPV:
// threads per vector (each takes a contiguous 1/TPV of the dimensions; their
// partial sums meet through lane shuffles).  W: wavefronts per workgroup.
// LDS: table staged in LDS.
//
// LDS layout: part p of the dimensions (the range one of a vector's TPV
// threads scans) starts 256 / TPV bytes further into the bank rows than a
// plain [d][code][query] layout would put it, so that the TPV lanes of a
// vector, at the same position of their parts, read different banks.
template <int Q4, int VPT, int TPV, int W, bool LDS>
__global__ __launch_bounds__(W * 64) void scan2_kernel(const uint32_t *__restrict__ codes,
                                                       const float *__restrict__ lut,
                                                       float *__restrict__ scores, int V, int D,
                                                       int Q) {
    constexpr int T = W * 64;
    constexpr int QP = 4 * Q4;
    constexpr int PAD = 16 / TPV;         // float4s of padding before each part
    extern __shared__ f32x4_t slut[];     // [part][D/TPV][4][Q4] (+ padding) when LDS
    const int tid = threadIdx.x;
    const int DP = D / TPV;               // dimensions per part
    if constexpr (LDS) {
        // One float4 of lut (the four codes of one (q, d)) per step.
        const int n = Q * D;
        float *sl = reinterpret_cast<float *>(slut);
        for (int i = tid; i < n; i += T) {
            const int q = i / D, d = i - q * D;
            const f32x4_t v = reinterpret_cast<const f32x4_t *>(lut)[i];
            const int base = ((d * 4) * Q4 + (d / DP) * PAD) * 4 + q;   // float index of (d, code 0, q)
#pragma unroll
            for (int c = 0; c < 4; ++c) sl[base + c * Q4 * 4] = v[c];
        }
        if (Q % 4) {                      // padded queries read as zero
            for (int i = tid; i < D * 4; i += T) {
                const int d = i >> 2, c = i & 3;
                const int base = ((d * 4 + c) * Q4 + (d / DP) * PAD) * 4;
                for (int q = Q; q < QP; ++q) sl[base + q] = 0.f;
            }
        }
        __syncthreads();
    }

    const int WPV = D >> 4;               // code words per vector
    const int NCH = D >> 6;               // 16-byte chunks per vector
    const int CPP = NCH / TPV;            // chunks per part
    const int part = TPV == 1 ? 0 : tid % TPV;
    const int slot = TPV == 1 ? tid : tid / TPV;
    constexpr int SLOTS = T / TPV;        // vectors a workgroup scans per vector-per-thread step
    int vk[VPT];
    bool ok[VPT];
    const u32x4_t *src[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = ((int)blockIdx.x * VPT + k) * SLOTS + slot;
        ok[k] = v < V;
        vk[k] = min(v, V - 1);            // past V: re-read the last vector, store nothing
        src[k] = reinterpret_cast<const u32x4_t *>(codes + (size_t)vk[k] * WPV) + part * CPP;
    }
    float acc[VPT][QP];
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
        for (int q = 0; q < QP; ++q) acc[k][q] = 0.f;

    const int d0 = part * DP;
    const int sbase = part * PAD;         // this part's padding, in float4s
    u32x4_t cur[VPT], nxt[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) cur[k] = src[k][0];
    for (int ch = 0; ch < CPP; ++ch) {
        if (ch + 1 < CPP) {
#pragma unroll
            for (int k = 0; k < VPT; ++k) nxt[k] = src[k][ch + 1];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int d = d0 + ch * 64 + j * 16 + i;
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int c = (int)((cur[k][j] >> (2 * i)) & 3u);
                    if constexpr (LDS) {
#pragma unroll
                        for (int qq = 0; qq < Q4; ++qq) {
                            const f32x4_t t = slut[(d * 4 + c) * Q4 + qq + sbase];
                            acc[k][4 * qq] += t.x;
                            acc[k][4 * qq + 1] += t.y;
                            acc[k][4 * qq + 2] += t.z;
                            acc[k][4 * qq + 3] += t.w;
                        }
                    } else {
#pragma unroll
                        for (int q = 0; q < QP; ++q)
                            if (q < Q) acc[k][q] += lut[((size_t)q * D + d) * 4 + c];
                    }
                }
            }
        }
#pragma unroll
        for (int k = 0; k < VPT; ++k) cur[k] = nxt[k];
    }
    // Partial sums of a vector's TPV adjacent lanes meet by shuffles.
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
        for (int q = 0; q < QP; ++q)
#pragma unroll
            for (int m = 1; m < TPV; m <<= 1) acc[k][q] += __shfl_xor(acc[k][q], m);
    if (part != 0) return;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        if (!ok[k]) continue;
        float *out = scores + (size_t)vk[k] * Q;
#pragma unroll
        for (int q = 0; q < QP; ++q)
            if (q < Q) out[q] = acc[k][q];
    }
}

// tpv == 0: automatic, the fewest threads per vector (at most 8) that give
// 16 wavefronts per CU; more split a vector's lookups between lanes that
// contend for the same LDS banks, fewer leave LDS latency exposed.
struct ScanCfg { int lds, vpt, tpg, tpv; };
constexpr ScanCfg kScanDefault = {1, 1, 1024, 0};
constexpr int kCUs = 256;
ScanCfg g_scan = kScanDefault;

bool scan_cfg_ok(int lds, int vpt, int tpg, int tpv) {
    return (lds == 0 || lds == 1) && (vpt == 1 || vpt == 2) && (tpg == 64 || tpg == 256 || tpg == 1024) &&
           (tpv == 0 || tpv == 1 || tpv == 2 || tpv == 4 || tpv == 8);
}

int auto_tpv(int V, int vpt) {
    int t = 1;
    while (t < 8 && (int64_t)V * t / vpt < (int64_t)16 * 64 * kCUs) t <<= 1;
    return t;
}

// LDS bytes of the staged table: D * 4 float4 groups of Q4, plus the parts'
// padding.
size_t lut_lds_bytes(int D, int Q4, int tpv) { return ((size_t)D * 4 * Q4 + 16) * 16; }

template <int Q4, int VPT, int TPV, int W, bool LDS>
void launch_s(const uint32_t *codes, const float *lut, float *scores, int V, int D, int Q,
              hipStream_t st) {
    const int per = VPT * W * 64 / TPV;
    const int grid = (V + per - 1) / per;
    const size_t lds = LDS ? lut_lds_bytes(D, Q4, TPV) : 0;
    hipLaunchKernelGGL((scan2_kernel<Q4, VPT, TPV, W, LDS>), dim3(grid), dim3(W * 64), lds, st, codes,
                       lut, scores, V, D, Q);
}

template <int Q4, int VPT, int TPV, bool LDS>
void launch_w(int tpg, const uint32_t *codes, const float *lut, float *scores, int V, int D, int Q,
              hipStream_t st) {
    if (tpg == 64) launch_s<Q4, VPT, TPV, 1, LDS>(codes, lut, scores, V, D, Q, st);
    else if (tpg == 1024) launch_s<Q4, VPT, TPV, 16, LDS>(codes, lut, scores, V, D, Q, st);
    else launch_s<Q4, VPT, TPV, 4, LDS>(codes, lut, scores, V, D, Q, st);
}

template <int Q4, int VPT, bool LDS>
void launch_t(const ScanCfg &c, const uint32_t *codes, const float *lut, float *scores, int V, int D,
              int Q, hipStream_t st) {
    switch (c.tpv) {
    case 2: launch_w<Q4, VPT, 2, LDS>(c.tpg, codes, lut, scores, V, D, Q, st); break;
    case 4: launch_w<Q4, VPT, 4, LDS>(c.tpg, codes, lut, scores, V, D, Q, st); break;
    case 8: launch_w<Q4, VPT, 8, LDS>(c.tpg, codes, lut, scores, V, D, Q, st); break;
    default: launch_w<Q4, VPT, 1, LDS>(c.tpg, codes, lut, scores, V, D, Q, st); break;
    }
}

template <int Q4, bool LDS>
void launch_v(const ScanCfg &c, const uint32_t *codes, const float *lut, float *scores, int V, int D,
              int Q, hipStream_t st) {
    if (c.vpt == 2) launch_t<Q4, 2, LDS>(c, codes, lut, scores, V, D, Q, st);
    else launch_t<Q4, 1, LDS>(c, codes, lut, scores, V, D, Q, st);
}

}  // namespace

extern "C" int scan2(const uint32_t *codes, const float *lut, float *scores, int V, int D, int Q,
                     void *stream) {
    ScanCfg c = g_scan;
    if (Q < 1 || Q > 8 || V < 0 || D < 64 || D % 64 != 0 || D > (c.lds ? 1024 : 4096))
        return Q4_EINVAL;
    if (c.tpv == 0) c.tpv = auto_tpv(V, c.vpt);
    while ((D / 64) % c.tpv != 0) c.tpv >>= 1;    // the most threads per vector that split D evenly
    if (V == 0) return Q4_OK;
    if (!codes || !lut || !scores) return Q4_ENULL;
    if (!q4::aligned(codes, 16) || !q4::aligned(lut, 16) || !q4::aligned(scores, 16)) return Q4_EALIGN;
    if (int st = q4::check_device(); st != Q4_OK) return st;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (Q <= 4) {
        if (c.lds) launch_v<1, true>(c, codes, lut, scores, V, D, Q, st);
        else launch_v<1, false>(c, codes, lut, scores, V, D, Q, st);
    } else {
        if (c.lds) launch_v<2, true>(c, codes, lut, scores, V, D, Q, st);
        else launch_v<2, false>(c, codes, lut, scores, V, D, Q, st);
    }
    return q4::launch_status();
}

extern "C" int scan2_set_config(int lut_in_lds, int vectors_per_thread, int threads_per_group,
                                int threads_per_vector) {
    if (lut_in_lds == 0 && vectors_per_thread == 0 && threads_per_group == 0 && threads_per_vector == 0) {
        g_scan = kScanDefault;
        return Q4_OK;
    }
    if (!scan_cfg_ok(lut_in_lds, vectors_per_thread, threads_per_group, threads_per_vector))
        return Q4_EINVAL;
    g_scan = {lut_in_lds, vectors_per_thread, threads_per_group, threads_per_vector};
    return Q4_OK;
}

extern "C" int scan2_config(int *lut_in_lds, int *vectors_per_thread, int *threads_per_group,
                            int *threads_per_vector) {
    if (!lut_in_lds || !vectors_per_thread || !threads_per_group || !threads_per_vector) return Q4_ENULL;
    *lut_in_lds = g_scan.lds;
    *vectors_per_thread = g_scan.vpt;
    *threads_per_group = g_scan.tpg;
    *threads_per_vector = g_scan.tpv;
    return Q4_OK;
}
