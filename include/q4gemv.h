/*
 * q4gemv.h -- C ABI of the MI355X (gfx950) int4 decode-GEMV library.
 *
 * The library computes the bandwidth-bound decode GEMV over block-quantised
 * 4-bit weights,
 *
 *     y[m, n] = sum_k x[m, k] * (q(n, k) - z(n, k / g)) * s(n, k / g),
 *
 * (gerbil "WGSL Kernel Reference", section 3 MatMulInt4: "Computes",
 * "INT4 Packing", "Dequantization"), plus a dense fp32 control GEMV, a
 * dequantiser for debugging and two HBM bandwidth probes (webgpu-bench 0.1.0
 * README, "What it measures": read-bandwidth and write-bandwidth).
 *
 * Storage format (all row-major, N-major weights W_q[N, K]):
 *   x       float32 [M, K]
 *   wq      uint8   [N, K/2]        code of (n, k) in byte n*K/2 + k/2:
 *                                   low nibble for even k, high for odd k
 *   scales  uint16  [N, G]          IEEE binary16 bit patterns, G = K / g
 *   zeros   uint8   [N, (G+1)/2]    zero point of group j of row n in byte
 *                                   n*((G+1)/2) + j/2: low nibble for even j
 *   y       float32 [M, N]
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors) owned
 *     by the caller.  The library never allocates, frees or keeps them.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL selects the
 *     default stream) and may be captured into a HIP graph.
 *   - Return value: Q4_OK (0) or a negative q4_status.  Arguments are fully
 *     validated before anything is launched; on an argument error nothing is
 *     launched and no output memory is touched.  A launch failure returns
 *     Q4_ELAUNCH.  No call ever returns Q4_OK without having launched its
 *     work, except where a size argument makes the output empty (N == 0 or
 *     n_floats == 0), which is documented per call.
 *   - The library runs on gfx950 only; any other device gives Q4_EDEVICE.
 */
#ifndef Q4GEMV_H
#define Q4GEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4GEMV_ABI_VERSION 1

enum q4_status {
    Q4_OK = 0,
    Q4_EINVAL = -1,  /* a size, shape or group-size argument is out of range */
    Q4_ENULL = -2,   /* a required pointer is NULL */
    Q4_EALIGN = -3,  /* a pointer breaks its alignment rule */
    Q4_EDEVICE = -4, /* no HIP device, or the current device is not gfx950 */
    Q4_ELAUNCH = -5  /* the kernel launch reported an error */
};

/* int4 decode GEMV: y[M, N] = x[M, K] . dequant(W_q[N, K])^T, fp32 accumulate
 * (gerbil "WGSL Kernel Reference", section 3 MatMulInt4, "Dequantization").
 * Two arithmetic paths (gemv_q4_path tells which one a shape takes):
 *   - fused multiply-add (2 to 8 rows; one row with K <= 512, or with K
 *     past the integer path's limit below): (q - z) formed exactly (in fp32
 *     for 2 to 8 rows, in binary16 for one row), multiplied by the fp32 x
 *     with fp32 fused multiply-adds, the group scale applied per 32-code
 *     chunk;
 *   - integer (M == 1: 512 < K <= 19232, or <= 19264 where N is small
 *     enough for 4-wavefront workgroups, as the LDS must hold the chunk
 *     records of all of x; 2 to 8 rows with K > 1024 only when fixed with
 *     gemv_q4_set_geometry): every chunk of 32 values
 *     of an x row (x[m][32c .. 32c+31]) is written as X + r with
 *     X = rint(x * 2^sh) an integer, |X| <= 2^26 (2^(25-sh) <= max|x| over
 *     the chunk < 2^(26-sh)), and r the exact residual; the sum of (q - z) * X
 *     is formed exactly in int32, and for every element whose |r| exceeds
 *     2^-14 of |x * 2^sh| (values far below the chunk's largest) (q - z) * r
 *     is added in fp32, so each product is carried to within 2^-14 of itself;
 *     then one conversion per chunk, a multiply by 2^-sh and the group scale.
 *     q == z gives exactly 0; a chunk of x row m holding Inf or NaN makes
 *     every output of row m NaN.
 * Accuracy, on either path, for every finite x whose products and sums stay
 * inside the fp32 range: each output y[m, n] satisfies
 *     |y - y_ref| <= 1e-4 * sum_k |x[m, k] w[n, k]| + 1e-6,
 * with y_ref the exact sum and w = (q - z) * s the dequantised weight.
 *   1 <= M <= 8;  N >= 0 (N == 0 launches nothing);  group_size in {32, 128};
 *   K >= group_size, K % group_size == 0 and K <= 16777216 (2^24: every
 *   byte offset of the kernels' 32-bit buffer addressing then fits; a
 *   longer K returns Q4_EINVAL rather than reading short).
 *   x and wq 16-byte aligned; scales 2-byte aligned; y 4-byte aligned.
 *   y must not overlap any input. */
int gemv_q4(const float *x, const uint8_t *wq, const uint16_t *scales,
            const uint8_t *zeros, float *y, int M, int N, int K, int group_size,
            void *stream);

/* gemv_q4 with a caller-provided device workspace, which lets the 2-8 row
 * multiply-add path split K over workgroups where x would otherwise be
 * staged in several LDS segments (a long K at several rows: each CU would
 * read all of x for the weights of a few rows).  The workgroups then write
 * partial sums into the workspace and a second launch on the same stream adds
 * them, in a fixed order, into y.  Same computation, rules and errors as
 * gemv_q4 (gerbil "WGSL Kernel Reference", section 3 MatMulInt4); the result
 * may differ from gemv_q4's in the last bits (another summation order), both
 * within the stated bound.
 *   workspace        device memory, 16-byte aligned, not overlapping any
 *                    argument; NULL, or fewer bytes than
 *                    gemv_q4_workspace_size reports, runs gemv_q4's plan.
 *                    Its contents need no initialisation and are
 *                    meaningless after the call.  The caller owns it; the
 *                    library keeps no pointer to it after the call (a graph
 *                    that captured the call keeps using it when replayed).
 *   workspace_bytes  its size in bytes.
 * Calls that use the same workspace must not overlap in time (stream order
 * serialises calls on one stream).  Q4_EALIGN for a misaligned workspace. */
int gemv_q4_ws(const float *x, const uint8_t *wq, const uint16_t *scales,
               const uint8_t *zeros, float *y, int M, int N, int K, int group_size,
               void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes gemv_q4_ws uses for a shape: 4 * ks * M * N (ks the
 * workgroups splitting K, 2 to 8) where it splits K, 0 where it does not.
 * Host-only; launches nothing and needs no device.  Q4_EINVAL for an invalid
 * shape, Q4_ENULL for a NULL bytes. */
int gemv_q4_workspace_size(int M, int N, int K, int group_size, size_t *bytes);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): gemv_q4_ws with the
 * library's own workspace, a static 512 KiB device array on each GPU (enough
 * for every K split gemv_q4_ws makes), so the call allocates nothing.  Same
 * arguments, results, rules and errors as gemv_q4_ws with a large enough
 * workspace (bit-identical to it); Q4_EINVAL should a shape ever need more
 * than the array holds.  The first call on a device looks up the array's
 * address there (no allocation).  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (from different streams or
 * threads) race and may return wrong results; calls on one stream are
 * ordered and safe.  Nothing in the array needs clearing between calls. */
int gemv_q4_static(const float *x, const uint8_t *wq, const uint16_t *scales,
                   const uint8_t *zeros, float *y, int M, int N, int K, int group_size,
                   void *stream);

/* SwiGLU block of a decoder layer on int4 weights: the gate and up
 * projections, each a gemv_q4 of the same x, combined as
 *   y[m, n] = silu(g[m, n]) * u[m, n],   silu(v) = v / (1 + e^-v)
 * (gerbil "WGSL Kernel Reference", section 9 SiLU for silu, section 12 Mul
 * for the combine, which the page notes could be fused with the SiLU).
 * With one activation row on the integer path without a K-split, one launch
 * converts x once and streams the gate matrix, then the up matrix, and
 * combines in registers.  Otherwise two launches: u is written to y, then
 * the gate GEMV combines in its store.  Either way there is no separate
 * element-wise pass and no intermediate buffer.
 * Arguments, rules and the arithmetic path of each projection are those of
 * gemv_q4 (both matrices [N, K] with the same group_size); y must not overlap
 * any input.  Each output is within |u| * 1.1 * t_g + |silu(g)| * t_u plus
 * second-order and rounding terms of the exact value, t_g and t_u being the
 * gemv_q4 error bounds of the two projections. */
int gemv_q4_swiglu(const float *x, const uint8_t *wq_gate, const uint16_t *scales_gate,
                   const uint8_t *zeros_gate, const uint8_t *wq_up, const uint16_t *scales_up,
                   const uint8_t *zeros_up, float *y, int M, int N, int K, int group_size,
                   void *stream);

/* Dense fp32 control GEMV, y[M, N] = x[M, K] . w[N, K]^T (cera 0.5.0
 * wgpu_gemv_bench.rs: the f32 kernel kept in the table as the control).
 *   1 <= M <= 8;  N >= 0 (N == 0 launches nothing);  K >= 4, K % 4 == 0.
 *   x and w 16-byte aligned; y 4-byte aligned. */
int gemv_f32(const float *x, const float *w, float *y, int M, int N, int K, void *stream);

/* Debug dequantiser (gerbil "WGSL Kernel Reference", section 3 MatMulInt4,
 * "INT4 Packing" and "Dequantization").  Writes, for every (n, k):
 *   w_out[n*K + k]     = (float)(q - z) * s      (bit-exact; may be NULL)
 *   codes_out[n*K + k] = q                        (0..15;   may be NULL)
 * At least one output must be non-NULL.
 *   N >= 0 (N == 0 launches nothing); group_size in {32, 128}; K >= group_size,
 *   K % group_size == 0.  wq 16-byte aligned, scales 2-byte aligned, w_out
 *   16-byte aligned, codes_out 8-byte aligned. */
int dequant_q4(const uint8_t *wq, const uint16_t *scales, const uint8_t *zeros,
               float *w_out, uint8_t *codes_out, int N, int K, int group_size,
               void *stream);

/* Read-bandwidth probe (webgpu-bench 0.1.0 README, read-bandwidth; Refractometer
 * "What each sweep measures", bandwidth: vec4 read-reduce).  Streams buf with
 * 16-byte non-temporal loads folded by addition only and writes one partial
 * sum per workgroup: exactly n_partials workgroups are launched and
 * partials[0 .. n_partials) are all written.  The caller adds the partials.
 *   buf 16-byte aligned, n_floats % 4 == 0 (n_floats == 0 writes zeros);
 *   1 <= n_partials <= 65536; partials 4-byte aligned. */
int read_reduce(const float *buf, size_t n_floats, float *partials, int n_partials,
                void *stream);

/* read_reduce walking buf `passes` times in one launch (1 <= passes <= 4096);
 * each partial is the sum over all passes.  A buffer that fits a cache is
 * then re-read from it, which the bandwidth sweep uses to find the caches'
 * knees: unlike read_reduce, whose loads are marked non-temporal (the data
 * is read once), these loads are plain.  Other arguments and errors as
 * read_reduce. */
int read_reduce_passes(const float *buf, size_t n_floats, int passes, float *partials,
                       int n_partials, void *stream);

/* Copy-bandwidth probe (Refractometer "What each sweep measures", bandwidth:
 * vec4 copy): dst[i] = src[i] for i < n_floats with 16-byte loads and
 * stores, the whole range copied `passes` times in one launch.
 *   src, dst 16-byte aligned and not overlapping (Q4_EINVAL if they do);
 *   n_floats % 4 == 0 (n_floats == 0 launches nothing); 1 <= passes <= 4096;
 *   0 <= n_blocks <= 65536 workgroups of 256 threads (0 picks the default
 *   grid; never more than the range needs). */
int copy_vec4(const float *src, float *dst, size_t n_floats, int passes, int n_blocks,
              void *stream);

/* Write-bandwidth probe (webgpu-bench 0.1.0 README, write-bandwidth): stores
 * `value` to every element with 16-byte stores and no reads.
 *   buf 16-byte aligned, n_floats % 4 == 0 (n_floats == 0 launches nothing);
 *   0 <= n_blocks <= 65536 (0 picks the default grid). */
int write_fill(float *buf, size_t n_floats, float value, int n_blocks, void *stream);

/* Launch geometry that gemv_q4 would use for a shape, for reporting and
 * tests; host-only, launches nothing and needs no device.  Any output
 * pointer may be NULL.  Returns Q4_EINVAL for an invalid shape.
 *   grid         workgroups launched
 *   block        threads per workgroup
 *   rows_per_wave output rows one wavefront owns (the integer path: at most;
 *                a workgroup owns ceil(N / grid) rows, dealt evenly to its
 *                row groups)
 *   lanes_per_row lanes that share one row's K range (16, 32 or 64)
 *   ksplit       wavefronts that split one row block's K range
 *   segments     x segments staged through LDS one after another */
int gemv_q4_geometry(int M, int N, int K, int group_size, int *grid, int *block,
                     int *rows_per_wave, int *lanes_per_row, int *ksplit, int *segments);

/* Which arithmetic path gemv_q4 takes for a shape (see gemv_q4): returns
 * Q4_PATH_FMA or Q4_PATH_INTEGER, or Q4_EINVAL for an invalid shape.
 * Host-only; launches nothing and needs no device. */
#define Q4_PATH_FMA 0
#define Q4_PATH_INTEGER 1
int gemv_q4_path(int M, int N, int K, int group_size);

/* Human-readable text for a q4_status value (never NULL). */
const char *q4_strerror(int status);

/* Q4GEMV_ABI_VERSION of the built library. */
int q4_abi_version(void);

/* Fixes the launch geometry gemv_q4 (and each projection of gemv_q4_swiglu)
 * uses for one exact shape (M, N, K, group_size), for autotuning and for
 * applying a tuned profile (Refractometer, "What each sweep measures", q4
 * GEMV: columns per workgroup, K-splits and rows are the swept knobs; the
 * best configuration per device is kept as a profile).
 *   path     Q4_PATH_FMA or Q4_PATH_INTEGER
 *   waves    wavefronts per workgroup: 4, 8 or 16, or 0 for the plan's choice
 *            (the multiply-add path has 4 for one row and 8 for 2 to 8 rows;
 *            the integer path for 2 to 8 rows has 8, or 16 above 4 rows)
 *   ksplit   wavefronts splitting one row's K range: 1, 2 or 4, or 0 for the
 *            plan's choice
 * Returns Q4_EINVAL for an invalid shape or knob, or a combination the
 * kernels cannot run (e.g. the integer path at K <= 512 or with a K-split at
 * K <= 1024, or more than 3 chunk positions per lane); the previous setting
 * for the shape then stays.
 * Setting a shape again replaces its entry; up to 256 shapes.  Host-only:
 * needs no device and launches nothing.  The table is process-wide (every
 * caller's launches of that shape take the setting) and safe to change
 * while other threads call into the library: a launch reads a shape's
 * setting whole, either before or after a concurrent change. */
int gemv_q4_set_geometry(int M, int N, int K, int group_size, int path, int waves, int ksplit);

/* Forgets every geometry set by gemv_q4_set_geometry (process-wide, safe
 * beside concurrent calls like gemv_q4_set_geometry).  Returns Q4_OK. */
int gemv_q4_clear_geometry(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4GEMV_H */
