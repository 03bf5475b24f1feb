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
//   * A workgroup serves one group of four queries; the two groups of the
//     same vectors are placed on one XCD, sharing its L2.  The grid holds
//     the workgroups that fit the chip at once, each looping over vector
//     blocks after building its table once.  With the table in LDS
//     it first builds, for every pair of dimensions and each of the 16 code
//     pairs, the float4 of its four queries' two-entry sums, so one
//     ds_read_b128 covers two dimensions (the scan is bound by these reads:
//     16 bytes of table per pair of dimensions and four queries, against
//     half a byte of codes).  The parts of a vector's dimensions are offset
//     from one another by padding, so that they fall in different banks.
//   * With the table read from memory, each lookup is a 4-byte load that
//     the caches serve (the page's "storage" variant).
//   * Sums are fp32, per vector and query, in increasing d (two dimensions
//     at a time from the LDS table: each entry is one fp32 sum of two table
//     values).
#include "q4_common.h"
#include "q4scan.h"

#include <algorithm>
#include <atomic>

namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One workgroup scores its vectors against one group of four queries (the
// two query groups of the same vectors run on the same XCD, so that the
// second read of the codes finds them in its L2).  VPT: vectors per thread.  TPV:
// threads per vector (each takes a contiguous 1/TPV of the dimensions; their
// partial sums meet through lane shuffles).  W: wavefronts per workgroup.
// LDS: the table staged in LDS; otherwise every lookup reads the caller's
// table from memory.
//
// LDS table: per pair of dimensions (2p, 2p + 1) and per 4-bit code pair
// c0 + 4 c1, the float4 of the four queries' lut[q, 2p, c0] + lut[q, 2p + 1,
// c1], so one ds_read_b128 covers two dimensions.  Part t of the pairs (the
// range one of a vector's TPV threads scans) starts 256 / TPV bytes further
// into the bank rows than a plain layout would put it, so that the TPV lanes
// of a vector, at the same position of their parts, read different banks.
template <int VPT, int TPV, int W, bool LDS>
__global__ __launch_bounds__(W * 64) void scan2_kernel(const uint32_t *__restrict__ codes,
                                                       const float *__restrict__ lut,
                                                       float *__restrict__ scores, int V, int D,
                                                       int Q) {
    constexpr int T = W * 64;
    constexpr int PAD = 16 / TPV;         // float4s of padding before each part
    extern __shared__ f32x4_t slut[];     // [pair][16] float4 (+ padding) when LDS
    const int tid = threadIdx.x;
    constexpr int SLOTS = T / TPV;        // vectors a workgroup scans per vector-per-thread step
    const int NQG = (Q + 3) >> 2;         // query groups
    // Workgroups stay resident and loop over vector blocks vb0, vb0 + vstride,
    // ..., building the table once.
    int qg = 0, vb0 = (int)blockIdx.x, vstride = (int)gridDim.x;
    if (NQG == 2) {
        // Workgroups are dealt to the eight XCDs in turn (workgroup b to XCD
        // b % 8), each with its own L2.  The two query groups of a vector
        // block take workgroups b and b + 8, on the same XCD, so that the
        // second read of the block's codes finds them in that L2.  The grid
        // is a multiple of 16; workgroups past the last vector block have
        // nothing to do.
        const int b = (int)blockIdx.x, r = b >> 3;
        qg = r & 1;
        vb0 = (r >> 1) * 8 + (b & 7);
        vstride = (int)gridDim.x / 2;
    }
    if ((int64_t)vb0 * VPT * SLOTS >= V) return;
    const int q0 = 4 * qg;
    const int NP = D >> 1;                // dimension pairs
    const int PP = NP / TPV;              // pairs per part
    if constexpr (LDS) {
        // One (pair, query) per step: two float4 of lut (the four codes of
        // each dimension) give that query's 16 sums.
        float *sl = reinterpret_cast<float *>(slut);
        for (int i = tid; i < NP * 4; i += T) {
            const int pr = i >> 2, j = i & 3, q = q0 + j;
            f32x4_t a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
            if (q < Q) {
                const f32x4_t *l = reinterpret_cast<const f32x4_t *>(lut) + (size_t)q * D + 2 * pr;
                a = l[0];
                b = l[1];
            }
            const int base = (pr * 16 + (pr / PP) * PAD) * 4 + j;
#pragma unroll
            for (int c1 = 0; c1 < 4; ++c1)
#pragma unroll
                for (int c0 = 0; c0 < 4; ++c0) sl[base + (c0 + 4 * c1) * 4] = a[c0] + b[c1];
        }
        __syncthreads();
    }

    const int WPV = D >> 4;               // code words per vector
    const int NCH = D >> 6;               // 16-byte chunks per vector
    const int CPP = NCH / TPV;            // chunks per part
    const int part = TPV == 1 ? 0 : tid % TPV;
    const int slot = TPV == 1 ? tid : tid / TPV;
    const int p0 = part * PP;             // first pair of this part
    const int sbase = part * PAD;         // this part's padding, in float4s
    for (int vb = vb0; (int64_t)vb * VPT * SLOTS < V; vb += vstride) {
        int vk[VPT];
        bool ok[VPT];
        const u32x4_t *src[VPT];
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int64_t v = ((int64_t)vb * VPT + k) * SLOTS + slot;
            ok[k] = v < V;
            vk[k] = (int)std::min<int64_t>(v, V - 1);   // past V: re-read the last vector, store nothing
            src[k] = reinterpret_cast<const u32x4_t *>(codes + (size_t)vk[k] * WPV) + part * CPP;
        }
        float acc[VPT][4];
#pragma unroll
        for (int k = 0; k < VPT; ++k)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[k][q] = 0.f;

        u32x4_t cur[VPT], nxt[VPT];
#pragma unroll
        for (int k = 0; k < VPT; ++k) cur[k] = src[k][0];
        for (int ch = 0; ch < CPP; ++ch) {
            if (ch + 1 < CPP) {
#pragma unroll
                for (int k = 0; k < VPT; ++k) nxt[k] = src[k][ch + 1];
            }
            if constexpr (LDS) {
                // The eight lookups of a code word are issued together, and with
                // one vector per thread those of the next word before the sums
                // of this one, so that 8 to 16 table reads per wavefront are in
                // flight (read by read, LDS latency would bound the scan).
                const f32x4_t *tb = slut + (p0 + ch * 32) * 16 + sbase;
                auto lookups = [&](f32x4_t (&t)[VPT][8], int j) {
#pragma unroll
                    for (int n = 0; n < 8; ++n)
#pragma unroll
                        for (int k = 0; k < VPT; ++k)
                            t[k][n] = tb[(j * 8 + n) * 16 + (int)((cur[k][j] >> (4 * n)) & 15u)];
                };
                auto sums = [&](const f32x4_t (&t)[VPT][8]) {
#pragma unroll
                    for (int n = 0; n < 8; ++n)
#pragma unroll
                        for (int k = 0; k < VPT; ++k) {
                            acc[k][0] += t[k][n].x;
                            acc[k][1] += t[k][n].y;
                            acc[k][2] += t[k][n].z;
                            acc[k][3] += t[k][n].w;
                        }
                };
                f32x4_t ta[VPT][8];
                if constexpr (VPT == 1) {
                    f32x4_t tn[VPT][8];
                    lookups(ta, 0);
#pragma unroll
                    for (int j = 0; j < 4; j += 2) {
                        lookups(tn, j + 1);
                        __builtin_amdgcn_sched_barrier(0);
                        sums(ta);
                        if (j + 2 < 4) lookups(ta, j + 2);
                        __builtin_amdgcn_sched_barrier(0);
                        sums(tn);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        lookups(ta, j);
                        __builtin_amdgcn_sched_barrier(0);
                        sums(ta);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
#pragma unroll
                    for (int n = 0; n < 8; ++n) {
                        const int pr = p0 + ch * 32 + j * 8 + n;     // dimensions 2 pr, 2 pr + 1
#pragma unroll
                        for (int k = 0; k < VPT; ++k) {
                            const int c4 = (int)((cur[k][j] >> (4 * n)) & 15u);
                            const int c0 = c4 & 3, c1 = c4 >> 2;
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                if (q0 + q < Q)
                                    acc[k][q] += lut[((size_t)(q0 + q) * D + 2 * pr) * 4 + c0] +
                                                 lut[((size_t)(q0 + q) * D + 2 * pr + 1) * 4 + c1];
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
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int m = 1; m < TPV; m <<= 1) acc[k][q] += __shfl_xor(acc[k][q], m);
        if (part == 0) {
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                if (!ok[k]) continue;
                float *out = scores + (size_t)vk[k] * Q + q0;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (q0 + q < Q) out[q] = acc[k][q];
        }
        }
    }
}

// tpv == 0: automatic, the fewest threads per vector (at most 8) that give
// 16 wavefronts per CU; more split a vector's lookups between lanes that
// contend for the same LDS banks, fewer leave LDS latency exposed.
struct ScanCfg { int lds, vpt, tpg, tpv; };
constexpr ScanCfg kScanDefault = {1, 1, 1024, 0};
constexpr int kCUs = 256;
constexpr int kMaxDLds = 4096;         // the largest D (the table in memory)
// The scan's setting packed into one word, so that a launch reads it whole
// while scan2_set_config changes it on another thread: lds (bit 0), vpt
// (bits 1-2), tpg (3-13), tpv (14-17).
constexpr uint32_t pack_scan(ScanCfg c) {
    return (uint32_t)c.lds | (uint32_t)c.vpt << 1 | (uint32_t)c.tpg << 3 | (uint32_t)c.tpv << 14;
}
inline ScanCfg unpack_scan(uint32_t v) {
    return {(int)(v & 1u), (int)((v >> 1) & 3u), (int)((v >> 3) & 2047u), (int)((v >> 14) & 15u)};
}
std::atomic<uint32_t> g_scan{pack_scan(kScanDefault)};

bool scan_cfg_ok(int lds, int vpt, int tpg, int tpv) {
    return (lds == 0 || lds == 1) && (vpt == 1 || vpt == 2) && (tpg == 64 || tpg == 256 || tpg == 1024) &&
           (tpv == 0 || tpv == 1 || tpv == 2 || tpv == 4 || tpv == 8);
}

int auto_tpv(int V, int Q, int vpt) {
    const int64_t groups = (Q + 3) / 4;
    int t = 1;
    while (t < 8 && (int64_t)V * groups * t / vpt < (int64_t)16 * 64 * kCUs) t <<= 1;
    return t;
}

// LDS bytes of the staged table: D / 2 pairs of 16 float4, plus the parts'
// padding.
size_t lut_lds_bytes(int D) { return ((size_t)D / 2 * 16 + 16) * 16; }

// Workgroups of one kernel that fit a CU at once with `lds` bytes of LDS
// each, from the occupancy calculator, cached per LDS size (D / 64 - 1).
template <int VPT, int TPV, int W, bool LDS>
int resident_per_cu(int D, size_t lds) {
    static int cache[kMaxDLds / 64];
    int &c = cache[(LDS ? D : 64) / 64 - 1];
    if (c == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, scan2_kernel<VPT, TPV, W, LDS>, W * 64, lds) !=
                hipSuccess || n < 1)
            n = 1;
        c = n;
    }
    return c;
}

template <int VPT, int TPV, int W, bool LDS>
void launch_s(const uint32_t *codes, const float *lut, float *scores, int V, int D, int Q,
              hipStream_t st) {
    const int per = VPT * W * 64 / TPV;
    const int64_t nvb = ((int64_t)V + per - 1) / per;
    const size_t lds = LDS ? lut_lds_bytes(D) : 0;
    // As many workgroups as fit the chip at once (each builds the table
    // once and loops over vector blocks), never more than there are blocks;
    // with two query groups a multiple of 16 (see the kernel's workgroup order).
    const int64_t cap = (int64_t)resident_per_cu<VPT, TPV, W, LDS>(D, lds) * kCUs;
    const int64_t grid = Q > 4 ? std::min((2 * nvb + 15) / 16, std::max<int64_t>(cap / 16, 1)) * 16
                               : std::min(nvb, cap);
    hipLaunchKernelGGL((scan2_kernel<VPT, TPV, W, LDS>), dim3((unsigned)grid), dim3(W * 64), lds, st,
                       codes, lut, scores, V, D, Q);
}

template <int VPT, int TPV, bool LDS>
void launch_w(int tpg, const uint32_t *codes, const float *lut, float *scores, int V, int D, int Q,
              hipStream_t st) {
    if (tpg == 64) launch_s<VPT, TPV, 1, LDS>(codes, lut, scores, V, D, Q, st);
    else if (tpg == 1024) launch_s<VPT, TPV, 16, LDS>(codes, lut, scores, V, D, Q, st);
    else launch_s<VPT, TPV, 4, LDS>(codes, lut, scores, V, D, Q, st);
}

template <int VPT, bool LDS>
void launch_t(const ScanCfg &c, const uint32_t *codes, const float *lut, float *scores, int V, int D,
              int Q, hipStream_t st) {
    switch (c.tpv) {
    case 2: launch_w<VPT, 2, LDS>(c.tpg, codes, lut, scores, V, D, Q, st); break;
    case 4: launch_w<VPT, 4, LDS>(c.tpg, codes, lut, scores, V, D, Q, st); break;
    case 8: launch_w<VPT, 8, LDS>(c.tpg, codes, lut, scores, V, D, Q, st); break;
    default: launch_w<VPT, 1, LDS>(c.tpg, codes, lut, scores, V, D, Q, st); break;
    }
}

template <bool LDS>
void launch_v(const ScanCfg &c, const uint32_t *codes, const float *lut, float *scores, int V, int D,
              int Q, hipStream_t st) {
    if (c.vpt == 2) launch_t<2, LDS>(c, codes, lut, scores, V, D, Q, st);
    else launch_t<1, LDS>(c, codes, lut, scores, V, D, Q, st);
}

}  // namespace

extern "C" int scan2(const uint32_t *codes, const float *lut, float *scores, int V, int D, int Q,
                     void *stream) {
    ScanCfg c = unpack_scan(g_scan.load(std::memory_order_acquire));
    if (Q < 1 || Q > 8 || V < 0 || D < 64 || D % 64 != 0 || D > (c.lds ? 1024 : 4096))
        return Q4_EINVAL;
    if (c.tpv == 0) c.tpv = auto_tpv(V, Q, c.vpt);
    while ((D / 64) % c.tpv != 0) c.tpv >>= 1;    // the most threads per vector that split D evenly
    if (V == 0) return Q4_OK;
    if (!codes || !lut || !scores) return Q4_ENULL;
    if (!q4::aligned(codes, 16) || !q4::aligned(lut, 16) || !q4::aligned(scores, 16)) return Q4_EALIGN;
    if (int st = q4::check_device(); st != Q4_OK) return st;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (c.lds) launch_v<true>(c, codes, lut, scores, V, D, Q, st);
    else launch_v<false>(c, codes, lut, scores, V, D, Q, st);
    return q4::launch_status();
}

extern "C" int scan2_set_config(int lut_in_lds, int vectors_per_thread, int threads_per_group,
                                int threads_per_vector) {
    if (lut_in_lds == 0 && vectors_per_thread == 0 && threads_per_group == 0 && threads_per_vector == 0) {
        g_scan.store(pack_scan(kScanDefault), std::memory_order_release);
        return Q4_OK;
    }
    if (!scan_cfg_ok(lut_in_lds, vectors_per_thread, threads_per_group, threads_per_vector))
        return Q4_EINVAL;
    g_scan.store(pack_scan({lut_in_lds, vectors_per_thread, threads_per_group, threads_per_vector}),
                 std::memory_order_release);
    return Q4_OK;
}

extern "C" int scan2_config(int *lut_in_lds, int *vectors_per_thread, int *threads_per_group,
                            int *threads_per_vector) {
    if (!lut_in_lds || !vectors_per_thread || !threads_per_group || !threads_per_vector) return Q4_ENULL;
    const ScanCfg c = unpack_scan(g_scan.load(std::memory_order_acquire));
    *lut_in_lds = c.lds;
    *vectors_per_thread = c.vpt;
    *threads_per_group = c.tpg;
    *threads_per_vector = c.tpv;
    return Q4_OK;
}
