/*
 * scanref.c -- plain CPU oracle for the 2-bit corpus scan of the
 * Refractometer page ("What each sweep measures", the scan sweep: 65,536
 * vectors x 8 queries, a lookup table in workgroup memory or in storage).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, link or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the
 * HIP library; the two meet only through the seeded input arrays.
 *
 * What is computed (the page names the scan, its sizes and its lookup
 * table, not its arithmetic; this is the plainest reading of a lookup-table
 * scan over 2-bit codes):
 *
 *   code(v, d)   = bits 2(d % 16), 2(d % 16) + 1 of codes[v * D/16 + d / 16]
 *                  (16 two-bit codes per little-endian u32, the 2-bit form of
 *                  the int4 packing of the gerbil kernel reference)
 *   score[v, q]  = sum_d lut[(q * D + d) * 4 + code(v, d)]
 *   bound[v, q]  = sum_d |lut[(q * D + d) * 4 + code(v, d)]|
 *
 * in f64, one term at a time in increasing d.
 *
 * Pins (tests/test_oracle_scan.py): constant codes reduce the score to a
 * plain sum of one table column; a one-hot table counts the vectors whose
 * code at one dimension equals one value; hand-packed words; a table of the
 * form query * level gives the dot product of the query with the dequantised
 * vector, checked against exact integer arithmetic.
 */
#include <math.h>
#include <stdint.h>

static int code_at(const uint32_t *codes, int64_t D, int64_t v, int64_t d)
{
    uint32_t w = codes[v * (D / 16) + d / 16];
    return (int)((w >> (2 * (d % 16))) & 3u);
}

/* scores[i * Q + q] and bound[i * Q + q] for each listed vector rows[i]. */
void scanref_rows(const uint32_t *codes, int64_t V, int64_t D, const float *lut, int64_t Q,
                  const int64_t *rows, int64_t R, double *scores, double *bound)
{
    (void)V;
    for (int64_t i = 0; i < R; ++i) {
        int64_t v = rows[i];
        for (int64_t q = 0; q < Q; ++q) {
            double s = 0.0, b = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                double t = (double)lut[(q * D + d) * 4 + code_at(codes, D, v, d)];
                s += t;
                b += fabs(t);
            }
            scores[i * Q + q] = s;
            bound[i * Q + q] = b;
        }
    }
}
