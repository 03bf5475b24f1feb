/*
 * q4blocks.h -- C ABI of the decode GEMV over the block quantisation formats
 * named on the cera page (crate cera 0.5.0, examples/wgpu_gemv_bench.rs: the
 * kernel table and the block-geometry table of its decode-GEMV benchmark).
 *
 * A matrix W[N, K] in a block format is N rows stored one after another;
 * row n is its K / elems blocks in order, row_bytes = K / elems * bytes.
 * The page gives each format's geometry; the decoding is the published
 * definition of the GGML formats of these names (all fields little-endian):
 *
 *   BLK_Q4_0  32 elements, 18 bytes: d (binary16), 16 bytes of codes.
 *             Element i < 16 is the low nibble of code byte i, element
 *             16 + i its high nibble; w = d * (nibble - 8).
 *   BLK_Q8_0  32 elements, 34 bytes: d, 32 int8 codes; w = d * q.
 *   BLK_Q4_K  256 elements, 144 bytes: d, dmin (binary16), 12 bytes of
 *             packed 6-bit scale s_j and min m_j for eight sub-blocks of 32
 *             (j < 4: s_j = b[j] & 63, m_j = b[j+4] & 63; j >= 4: the low
 *             nibble, resp. high nibble, of b[j+4] below the top two bits of
 *             b[j-4], resp. b[j]), 128 code bytes: byte 32p + l holds
 *             element 64p + l (low nibble) and 64p + 32 + l (high nibble);
 *             w = d * s_j * q - dmin * m_j, j = element / 32.
 *   BLK_Q5_K  256 elements, 176 bytes: as BLK_Q4_K with 32 bytes qh before
 *             the codes; element 32j + l adds 16 * bit j of qh[l].
 *   BLK_Q6_K  256 elements, 210 bytes: 128 bytes ql, 64 bytes qh, 16 int8
 *             scales, d.  Element 128h + 32t + l: low nibble from nibble
 *             t / 2 of ql[64h + 32(t % 2) + l], top two bits from bits 2t,
 *             2t + 1 of qh[32h + l]; w = d * scale[element / 16] * (q - 32).
 *
 * Conventions are those of q4gemv.h: device pointers owned by the caller,
 * asynchronous on `stream` (a hipStream_t; NULL = default stream), return
 * Q4_OK or a negative q4_status, arguments validated before any launch, and
 * nothing launched or written on an error.
 */
#ifndef Q4BLOCKS_H
#define Q4BLOCKS_H

#include <stddef.h>
#include <stdint.h>

#include "q4gemv.h"

#ifdef __cplusplus
extern "C" {
#endif

enum blk_format { BLK_Q4_0 = 1, BLK_Q8_0 = 2, BLK_Q4_K = 3, BLK_Q5_K = 4, BLK_Q6_K = 5 };

/* Elements and bytes of one block of `format` (the cera page's geometry
 * table).  Q4_ENULL if an output pointer is NULL, Q4_EINVAL for an unknown
 * format.  Host only; launches nothing. */
int block_geometry(int format, int *elems, int *bytes);

/* Decode GEMV over a block-format matrix (the GEMV of the cera page's
 * decode benchmark): y[0, n] = sum_k x[0, k] * W(n, k), fp32 accumulate.
 *   x  float32 [M, K], 16-byte aligned      w  uint8 [N, row_bytes], 16-byte aligned
 *   y  float32 [M, N]
 * Limits: M == 1 (one activation row), N >= 0, K a multiple of 256 (the
 * page's own rule: the K-format super-block, and a multiple of every other
 * block size) with 256 <= K <= 32768.  N == 0 returns Q4_OK with nothing
 * launched, before any pointer check.  Each weight is formed as an exact
 * small integer (the code minus its offset: 8, 32, or none) times x, summed
 * in fp32 per 16 or 32 elements and scaled once per group; the min term of Q4_K/Q5_K is applied per
 * sub-block as dmin * m_j * sum(x).  Accuracy: |y - y_exact| <= 1e-4 * B +
 * 1e-6, with B = sum_k |x_k| * |W(n, k)|, and for Q4_K/Q5_K B = sum_k |x_k|
 * (|d s_j q| + |dmin m_j|).  A weight that decodes to Inf or NaN makes its
 * output row NaN or infinite; an x that is Inf or NaN makes every output NaN
 * or infinite. */
int gemv_block(int format, const float *x, const uint8_t *w, float *y, int M, int N, int K,
               void *stream);

/* Debug dequantiser: w_out[n * K + k] = W(n, k), each the single rounding of
 * the exact decoded value (bit-exact).  w 16-byte aligned, w_out float32
 * [N, K] 16-byte aligned; K as for gemv_block.  N == 0 returns Q4_OK with
 * nothing launched. */
int dequant_block(int format, const uint8_t *w, float *w_out, int N, int K, void *stream);

/* Launch geometry of gemv_block for one format: row slots per lane (1, 2 or
 * 4), wavefronts per workgroup (4 or 8) and workgroups per compute unit
 * (0..64; 0 = one workgroup per row block, otherwise the grid is at most
 * that many per CU and each workgroup loops over row blocks).  A set
 * geometry applies to every shape; 0, 0, 0 restores the default, a
 * per-format geometry for shapes of at least 512 row blocks and 1 row slot
 * with 4 wavefronts below that.  Process-wide (every caller's launches of
 * the format take it); safe beside concurrent calls on other threads: a
 * launch reads the setting whole, before or after a change.  Q4_EINVAL for
 * an unknown format or an unsupported combination. */
int gemv_block_set_config(int format, int rows_per_lane, int waves_per_group, int groups_per_cu);

/* The geometry gemv_block uses now for `format`. */
int gemv_block_config(int format, int *rows_per_lane, int *waves_per_group, int *groups_per_cu);

#ifdef __cplusplus
}
#endif

#endif /* Q4BLOCKS_H */
