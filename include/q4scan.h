/*
 * q4scan.h -- C ABI of the 2-bit corpus scan (Refractometer, "What each
 * sweep measures", the scan sweep: 65,536 vectors x 8 queries, the lookup
 * table in workgroup memory or in storage, a workgroup size and a number of
 * vectors per thread).
 *
 * Each corpus vector holds D two-bit codes; a query is given as its lookup
 * table, one value per (dimension, code).  The scan scores every vector
 * against every query:
 *
 *     score[v, q] = sum_d lut[q, d, code(v, d)]
 *
 * (for a table built as lut[q, d, c] = query[q, d] * level[d, c] this is the
 * dot product of the query with the vector's reconstruction).
 *
 *   codes   uint32  [V, D/16]   16 codes per little-endian word: dimension
 *                               16w + i in bits 2i, 2i+1 of word w
 *   lut     float32 [Q, D, 4]
 *   scores  float32 [V, Q]
 *
 * Conventions are those of q4gemv.h: device pointers owned by the caller,
 * asynchronous on `stream` (a hipStream_t; NULL = default stream), Q4_OK or
 * a negative q4_status, arguments validated before any launch, nothing
 * launched or written on an error.
 */
#ifndef Q4SCAN_H
#define Q4SCAN_H

#include <stddef.h>
#include <stdint.h>

#include "q4gemv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The scan above.  Limits: 1 <= Q <= 8; D a multiple of 64 with
 * 64 <= D <= 1024 (the table is staged whole in LDS) or, with the table
 * read from memory (scan2_set_config), D <= 4096; V >= 0, V == 0 returns
 * Q4_OK with nothing launched.  codes, lut and scores 16-byte aligned.
 * Sums in fp32 in increasing d per vector; accuracy
 * |score - exact| <= 1e-4 * sum_d |lut term| + 1e-6. */
int scan2(const uint32_t *codes, const float *lut, float *scores, int V, int D, int Q,
          void *stream);

/* The page's knobs: the table in LDS (1) or read from memory (0), vectors
 * per thread (1 or 2) and threads per workgroup (64, 256 or 1024); and
 * threads per vector (1, 2, 4 or 8: at most that many threads share a
 * vector, each scanning a contiguous part of its dimensions; the largest
 * power of two not above it that divides D / 64 is used; 0 = the fewest that
 * give 16 wavefronts per compute unit).  The page's own tail runs 256
 * threads per workgroup, one vector per thread; the default here is the
 * table in LDS, 1 vector per thread, 1024 threads, automatic threads per
 * vector.  All zero restores the default.  Process-wide (every caller's
 * scans take it); safe beside concurrent calls on other threads: a launch
 * reads the setting whole, before or after a change.  Q4_EINVAL for any
 * other value. */
int scan2_set_config(int lut_in_lds, int vectors_per_thread, int threads_per_group,
                     int threads_per_vector);

/* The configuration scan2 uses now. */
int scan2_config(int *lut_in_lds, int *vectors_per_thread, int *threads_per_group,
                 int *threads_per_vector);

#ifdef __cplusplus
}
#endif

#endif /* Q4SCAN_H */
