// gemv_f32.hip -- dense fp32 control GEMV, y[M,N] = x[M,K] . w[N,K]^T, for gfx950.
//
// The control of cera 0.5.0 wgpu_gemv_bench.rs (the f32 kernel kept in the
// table to tell harness artefacts from kernel properties).  It shares the
// int4 kernel's geometry: a wavefront owns R rows, LPR lanes share a row and
// stream it with 16-byte non-temporal loads (four weights per lane-load; the
// weights are read once), x is staged in LDS (consecutive lanes read
// consecutive float4, so no swizzle is needed), and partial sums are reduced
// with DPP and cross-row shuffles, meeting in LDS only when S wavefronts
// split a row's K range.  Each lane keeps two batches of loads: the next
// batch is issued before the current one's arithmetic, so a wavefront's
// loads stay in flight across its whole row instead of one batch at a time.
#include "q4_common.h"
#include "q4_device.h"

namespace {

constexpr int kWaves = 4;
constexpr int kCUs = 256;                     // MI355X compute units
constexpr int kBlock = kWaves * q4::kWave;
constexpr int kLdsBytes = 64 * 1024;          // dynamic LDS budget per workgroup
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// A weight float4, read once: a non-temporal load.
__device__ __forceinline__ float4 ldnt(const float4 *p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
// float4 positions per lane in each of the two batches in flight: 2 at one
// or two activation rows (fewer registers, more wavefronts), 4 at more.
constexpr int batch(int M) { return M <= 2 ? 2 : 4; }

constexpr int row_slots(int M) { return M <= 2 ? 4 : (M <= 4 ? 2 : 1); }

template <int M, int LPR>
__global__ __launch_bounds__(kBlock) void gemv_f32_kernel(
    const float *__restrict__ x, const float4 *__restrict__ w, float *__restrict__ y, int N,
    int K, int S, int seg4) {
    constexpr int R = row_slots(M);
    constexpr int UB = batch(M);
    constexpr int RG = q4::kWave / LPR;
    constexpr int RPW = R * RG;
    extern __shared__ float lds[];
    float4 *xs = reinterpret_cast<float4 *>(lds);          // [M][seg4]
    float *comb = lds + M * seg4 * 4;                       // [waves][RPW][M]

    const int C4 = K >> 2;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int rb = wave / S;
    const int ks = wave - rb * S;
    const int row0 = (blockIdx.x * (kWaves / S) + rb) * RPW + lane / LPR;
    const int li = lane % LPR;

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

    for (int s0 = 0; s0 < C4; s0 += seg4) {
        const int segC = min(seg4, C4 - s0);
        if (s0 > 0) __syncthreads();
        for (int m = 0; m < M; ++m) {
            const float4 *src = reinterpret_cast<const float4 *>(x + (size_t)m * K) + s0;
            for (int i = tid; i < segC; i += kBlock) xs[m * segC + i] = src[i];
        }
        __syncthreads();
        const int part = (segC + S - 1) / S;
        const int lo = s0 + ks * part;
        const int hi = min(s0 + segC, lo + part);
        auto load = [&](float4 (&wv)[UB][R], int bs) {
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                const int c = bs + u * LPR;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int row = min(row0 + r * RG, N - 1);
                    wv[u][r] = c < hi ? ldnt(&w[(size_t)row * C4 + c])
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
        };
        auto comp = [&](const float4 (&wv)[UB][R], int bs) {
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                const int c = bs + u * LPR;
                if (c < hi) {
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const float4 xv = xs[m * segC + (c - s0)];
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            float a = acc[r][m];
                            a = __builtin_fmaf(wv[u][r].x, xv.x, a);
                            a = __builtin_fmaf(wv[u][r].y, xv.y, a);
                            a = __builtin_fmaf(wv[u][r].z, xv.z, a);
                            a = __builtin_fmaf(wv[u][r].w, xv.w, a);
                            acc[r][m] = a;
                        }
                    }
                }
            }
        };
        float4 wa[UB][R], wb[UB][R];
        int bs = lo + li;
        if (bs < hi) load(wa, bs);
        while (bs < hi) {
            const int n1 = bs + UB * LPR;
            if (n1 < hi) load(wb, n1);
            comp(wa, bs);
            bs = n1;
            if (bs >= hi) break;
            const int n2 = bs + UB * LPR;
            if (n2 < hi) load(wa, n2);
            comp(wb, bs);
            bs = n2;
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = q4::group_sum<LPR>(acc[r][m]);

    if (S == 1) {
        if (li == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int row = row0 + r * RG;
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
            for (int m = 0; m < M; ++m)
                comb[(wave * RPW + r * RG + lane / LPR) * M + m] = acc[r][m];
    }
    __syncthreads();
    if (ks == 0 && li == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = row0 + r * RG;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                float v = acc[r][m];
                for (int t = 1; t < S; ++t) v += comb[((wave + t) * RPW + r * RG + lane / LPR) * M + m];
                if (row < N) y[(size_t)m * N + row] = v;
            }
        }
    }
}

struct Geometry {
    int LPR, S, seg4, grid, lds;
};

Geometry plan(int M, int N, int K) {
    Geometry p{};
    const int C4 = K / 4;
    p.LPR = C4 <= 16 ? 16 : (C4 <= 32 ? 32 : 64);
    const int rpw = row_slots(M) * (q4::kWave / p.LPR);
    const long row_waves = ((long)N + rpw - 1) / rpw;
    // K split S: at least two wavefronts per SIMD where the rows allow it;
    // then, among the splits that stage x in no more segments, the one whose
    // workgroups spread most evenly over the CUs (896 workgroups of the
    // 4096 -> 14336 shape leave half the CUs a fourth one; 1792 do not).
    auto shape = [&](int S, Geometry &g) {
        g.S = S;
        const int comb = S > 1 ? kWaves * rpw * M * 4 : 0;
        const int max_seg = (kLdsBytes - comb) / (M * 16);
        g.seg4 = C4 < max_seg ? C4 : max_seg;
        const long rows_per_wg = (long)rpw * (kWaves / S);
        g.grid = (int)((N + rows_per_wg - 1) / rows_per_wg);
        g.lds = M * g.seg4 * 16 + comb;
    };
    int S = 1;
    while (S < kWaves && 2 * S * p.LPR <= C4 && row_waves * S < 2048) S *= 2;
    shape(S, p);
    const int segs = (C4 + p.seg4 - 1) / p.seg4;
    auto spread = [](long grid) {   // workgroups per CU over the most any CU gets
        const long per = (grid + kCUs - 1) / kCUs;
        return (double)grid / (double)(per * kCUs);
    };
    for (int s2 = S * 2; s2 <= kWaves && 2 * s2 * p.LPR <= C4; s2 *= 2) {
        Geometry g = p;
        shape(s2, g);
        if ((C4 + g.seg4 - 1) / g.seg4 > segs) break;
        if (spread(g.grid) > spread(p.grid) + 0.01) p = g;
    }
    return p;
}

template <int M>
void dispatch(const Geometry &p, const float *x, const float *w, float *y, int N, int K,
              hipStream_t st) {
    const float4 *w4 = reinterpret_cast<const float4 *>(w);
    switch (p.LPR) {
    case 16:
        hipLaunchKernelGGL((gemv_f32_kernel<M, 16>), dim3(p.grid), dim3(kBlock), p.lds, st,
                           x, w4, y, N, K, p.S, p.seg4);
        break;
    case 32:
        hipLaunchKernelGGL((gemv_f32_kernel<M, 32>), dim3(p.grid), dim3(kBlock), p.lds, st,
                           x, w4, y, N, K, p.S, p.seg4);
        break;
    default:
        hipLaunchKernelGGL((gemv_f32_kernel<M, 64>), dim3(p.grid), dim3(kBlock), p.lds, st,
                           x, w4, y, N, K, p.S, p.seg4);
        break;
    }
}

}  // namespace

extern "C" int gemv_f32(const float *x, const float *w, float *y, int M, int N, int K,
                        void *stream) {
    if (M < 1 || M > 8 || N < 0 || K < 4 || K % 4 != 0) return Q4_EINVAL;
    if (N == 0) return Q4_OK;
    if (!x || !w || !y) return Q4_ENULL;
    if (!q4::aligned(x, 16) || !q4::aligned(w, 16) || !q4::aligned(y, 4)) return Q4_EALIGN;
    const int dev = q4::check_device();
    if (dev != Q4_OK) return dev;
    const Geometry p = plan(M, N, K);
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (M) {
    case 1: dispatch<1>(p, x, w, y, N, K, st); break;
    case 2: dispatch<2>(p, x, w, y, N, K, st); break;
    case 3: dispatch<3>(p, x, w, y, N, K, st); break;
    case 4: dispatch<4>(p, x, w, y, N, K, st); break;
    case 5: dispatch<5>(p, x, w, y, N, K, st); break;
    case 6: dispatch<6>(p, x, w, y, N, K, st); break;
    case 7: dispatch<7>(p, x, w, y, N, K, st); break;
    default: dispatch<8>(p, x, w, y, N, K, st); break;
    }
    return q4::launch_status();
}
