// probes.hip -- bandwidth probes for gfx950.
//
// read_reduce streams a buffer with 16-byte loads folded by addition only
// and writes one partial sum per workgroup (webgpu-bench 0.1.0 README,
// read-bandwidth; Refractometer "What each sweep measures", bandwidth: vec4
// read-reduce).  copy_vec4 copies with 16-byte loads and stores (the same
// Refractometer sweep: vec4 copy).  write_fill stores a constant with
// 16-byte stores and reads nothing (webgpu-bench 0.1.0 README,
// write-bandwidth).  All walk the buffer grid-stride, so at every step the
// whole grid covers one contiguous span.  The read and copy probes can walk
// the buffer several times per launch: a buffer that fits a cache is then
// read from that cache, and the cost of the launch itself is spread over
// the passes.
#include "q4_common.h"
#include "q4_device.h"

namespace {

constexpr int kBlock = 256;
constexpr int kUnroll = 8;                     // 16-byte loads in flight per lane
constexpr int kDefaultFillBlocks = 4096;
constexpr int kMaxPasses = 4096;

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// A 16-byte load, marked non-temporal when NT.
template <bool NT>
__device__ __forceinline__ float4 load4(const float4 *p) {
    if constexpr (NT) {
        const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
        return make_float4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}

// NT: loads marked non-temporal (the data is read once).  The streaming
// probe takes them: they measured about 8% more bandwidth over 2 GiB than
// plain loads.  The multi-pass probe, which must find a small buffer in
// cache again, takes plain loads.
template <bool NT>
__global__ __launch_bounds__(kBlock) void read_reduce_kernel(const float4 *__restrict__ buf,
                                                             size_t n4, int passes,
                                                             float *__restrict__ partials) {
    __shared__ float wsum[kBlock / 64];
    const size_t stride = (size_t)gridDim.x * kBlock;
    float a[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) a[u] = 0.f;
    for (int p = 0; p < passes; ++p) {
        size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
        for (; i + (kUnroll - 1) * stride < n4; i += kUnroll * stride) {
            float4 v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                v[u] = load4<NT>(&buf[i + u * stride]);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) a[u] += (v[u].x + v[u].y) + (v[u].z + v[u].w);
        }
        for (; i < n4; i += stride) {
            const float4 v = load4<NT>(&buf[i]);
            a[0] += (v.x + v.y) + (v.z + v.w);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) s += a[u];
    s = q4::group_sum<64>(s);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < kBlock / 64; ++w) t += wsum[w];
        partials[blockIdx.x] = t;
    }
}

// Each pass copies the whole range again; the empty asm keeps the compiler
// from merging passes, whose stores it could otherwise prove redundant.
__global__ __launch_bounds__(kBlock) void copy_kernel(const float4 *__restrict__ src,
                                                      float4 *__restrict__ dst, size_t n4,
                                                      int passes) {
    const size_t stride = (size_t)gridDim.x * kBlock;
    for (int p = 0; p < passes; ++p) {
        size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
        for (; i + (kUnroll - 1) * stride < n4; i += kUnroll * stride) {
            float4 v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) dst[i + u * stride] = v[u];
        }
        for (; i < n4; i += stride) dst[i] = src[i];
        asm volatile("" ::: "memory");
    }
}

__global__ __launch_bounds__(kBlock) void write_fill_kernel(float4 *__restrict__ buf, size_t n4,
                                                            float value) {
    const float4 v = make_float4(value, value, value, value);
    const size_t stride = (size_t)gridDim.x * kBlock;
    for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < n4; i += stride) buf[i] = v;
}

}  // namespace

namespace {

int launch_read(bool nt, const float *buf, size_t n_floats, int passes, float *partials,
                int n_partials, void *stream) {
    if (n_floats % 4 != 0 || n_partials < 1 || n_partials > 65536 || passes < 1 ||
        passes > kMaxPasses)
        return Q4_EINVAL;
    if (!partials || (n_floats && !buf)) return Q4_ENULL;
    if ((buf && !q4::aligned(buf, 16)) || !q4::aligned(partials, 4)) return Q4_EALIGN;
    const int dev = q4::check_device();
    if (dev != Q4_OK) return dev;
    if (nt)
        hipLaunchKernelGGL(read_reduce_kernel<true>, dim3(n_partials), dim3(kBlock), 0,
                           static_cast<hipStream_t>(stream), reinterpret_cast<const float4 *>(buf),
                           n_floats / 4, passes, partials);
    else
        hipLaunchKernelGGL(read_reduce_kernel<false>, dim3(n_partials), dim3(kBlock), 0,
                           static_cast<hipStream_t>(stream), reinterpret_cast<const float4 *>(buf),
                           n_floats / 4, passes, partials);
    return q4::launch_status();
}

}  // namespace

extern "C" int read_reduce_passes(const float *buf, size_t n_floats, int passes, float *partials,
                                  int n_partials, void *stream) {
    return launch_read(false, buf, n_floats, passes, partials, n_partials, stream);
}

extern "C" int read_reduce(const float *buf, size_t n_floats, float *partials, int n_partials,
                           void *stream) {
    return launch_read(true, buf, n_floats, 1, partials, n_partials, stream);
}

extern "C" int copy_vec4(const float *src, float *dst, size_t n_floats, int passes, int n_blocks,
                         void *stream) {
    if (n_floats % 4 != 0 || n_blocks < 0 || n_blocks > 65536 || passes < 1 || passes > kMaxPasses)
        return Q4_EINVAL;
    if (n_floats == 0) return Q4_OK;
    if (!src || !dst) return Q4_ENULL;
    if (!q4::aligned(src, 16) || !q4::aligned(dst, 16)) return Q4_EALIGN;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    const uintptr_t bytes = (uintptr_t)n_floats * 4u;
    if (s0 < d0 + bytes && d0 < s0 + bytes) return Q4_EINVAL;   // the ranges overlap
    const int dev = q4::check_device();
    if (dev != Q4_OK) return dev;
    const size_t n4 = n_floats / 4;
    size_t blocks = n_blocks ? (size_t)n_blocks : (size_t)kDefaultFillBlocks;
    const size_t need = (n4 + kBlock - 1) / kBlock;
    if (blocks > need) blocks = need;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), reinterpret_cast<const float4 *>(src),
                       reinterpret_cast<float4 *>(dst), n4, passes);
    return q4::launch_status();
}

extern "C" int write_fill(float *buf, size_t n_floats, float value, int n_blocks, void *stream) {
    if (n_floats % 4 != 0 || n_blocks < 0 || n_blocks > 65536) return Q4_EINVAL;
    if (n_floats == 0) return Q4_OK;
    if (!buf) return Q4_ENULL;
    if (!q4::aligned(buf, 16)) return Q4_EALIGN;
    const int dev = q4::check_device();
    if (dev != Q4_OK) return dev;
    const size_t n4 = n_floats / 4;
    size_t blocks = n_blocks ? (size_t)n_blocks : (size_t)kDefaultFillBlocks;
    const size_t need = (n4 + kBlock - 1) / kBlock;
    if (blocks > need) blocks = need;
    hipLaunchKernelGGL(write_fill_kernel, dim3((unsigned)blocks), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), reinterpret_cast<float4 *>(buf), n4, value);
    return q4::launch_status();
}
