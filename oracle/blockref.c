/*
 * blockref.c -- plain CPU oracle for the decode GEMV over the block
 * quantisation formats named on the cera page (wgpu_gemv_bench, the
 * block-geometry table: Q4_0 32 elements in 18 bytes, Q8_0 32 in 34, Q4_K 256
 * in 144, Q5_K 256 in 176, Q6_K 256 in 210).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, link or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the
 * HIP library; the two meet only through the seeded input arrays.
 *
 * The page gives each format's geometry, not its decoding.  The formats are
 * the GGML block formats of those names; the decoding below is their
 * published definition, restated (one block, little-endian fields):
 *
 *   Q4_0  d:f16 | qs[16]       element i < 16: low nibble of qs[i];
 *                              element 16 + i: high nibble of qs[i];
 *                              w = d * (nibble - 8)
 *   Q8_0  d:f16 | qs[32] int8  w = d * qs[i]
 *   Q4_K  d:f16 | dmin:f16 | sc[12] | qs[128]
 *         eight sub-blocks of 32 with 6-bit scale s_j and 6-bit min m_j:
 *           j < 4:  s_j = sc[j] & 63,  m_j = sc[j+4] & 63
 *           j >= 4: s_j = (sc[j+4] & 15) | (sc[j-4] >> 6) << 4,
 *                   m_j = (sc[j+4] >> 4) | (sc[j] >> 6) << 4
 *         qs[32p + l] (p < 4, l < 32): low nibble is element 64p + l
 *         (sub-block 2p), high nibble element 64p + 32 + l (sub-block 2p+1);
 *         w = d * s_j * q - dmin * m_j
 *   Q5_K  d:f16 | dmin:f16 | sc[12] | qh[32] | qs[128]
 *         as Q4_K, with a fifth bit: element 64p + l adds 16 * bit 2p of
 *         qh[l], element 64p + 32 + l adds 16 * bit 2p+1 of qh[l]
 *   Q6_K  ql[128] | qh[64] | sc[16] int8 | d:f16
 *         element e = 128h + 32t + l (h < 2, t < 4, l < 32):
 *           low 4 bits: nibble (t >> 1) of ql[64h + 32(t & 1) + l]
 *           high 2 bits: bits 2t, 2t+1 of qh[32h + l]
 *         w = d * sc[e / 16] * (q - 32)
 *
 * Every function is the definition written out in f64, one element at a
 * time, in increasing index order, with no blocking or reordering.  Every
 * product above is exact in f64 (at most 11 + 8 + 7 significant bits), so
 * the f64 weight is the exact value and its float conversion rounds once.
 *
 * Pins (tests/test_oracle_blocks.py): the page's geometry table; blocks
 * packed from random integer fields decode to the value those fields define;
 * hand-written blocks with every 6-bit scale and min position exercised;
 * Q4_0 against the int4 oracle (g = 32, zero point 8); Q5_K with no fifth
 * bits against Q4_K, and with all of them; Q8_0 with d = 1 against exact
 * integer arithmetic.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

enum { BF_Q4_0 = 1, BF_Q8_0 = 2, BF_Q4_K = 3, BF_Q5_K = 4, BF_Q6_K = 5 };

/* Elements and bytes of one block; 0 for an unknown format. */
int blockref_geometry(int fmt, int64_t *elems, int64_t *bytes)
{
    switch (fmt) {
    case BF_Q4_0: *elems = 32; *bytes = 18; return 1;
    case BF_Q8_0: *elems = 32; *bytes = 34; return 1;
    case BF_Q4_K: *elems = 256; *bytes = 144; return 1;
    case BF_Q5_K: *elems = 256; *bytes = 176; return 1;
    case BF_Q6_K: *elems = 256; *bytes = 210; return 1;
    default: *elems = 0; *bytes = 0; return 0;
    }
}

/* IEEE 754 binary16 stored little-endian at p. */
static double f16_at(const uint8_t *p)
{
    unsigned h = (unsigned)p[0] | (unsigned)p[1] << 8;
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* 6-bit scale and min of sub-block j of a Q4_K / Q5_K block. */
static void scale_min(const uint8_t *sc, int j, int *s, int *m)
{
    if (j < 4) {
        *s = sc[j] & 63;
        *m = sc[j + 4] & 63;
    } else {
        *s = (sc[j + 4] & 15) | ((sc[j - 4] >> 6) << 4);
        *m = (sc[j + 4] >> 4) | ((sc[j] >> 6) << 4);
    }
}

/* Element e of the block at b: its exact weight w, and a, the magnitude the
 * tolerance is built from: |w|, except for the formats with a min term,
 * where the weight is the difference of two products and a is the sum of
 * their magnitudes. */
static void element(int fmt, const uint8_t *b, int e, double *w, double *a)
{
    switch (fmt) {
    case BF_Q4_0: {
        int i = e & 15;
        int q = (e < 16) ? (b[2 + i] & 15) : (b[2 + i] >> 4);
        *w = f16_at(b) * (double)(q - 8);
        *a = fabs(*w);
        return;
    }
    case BF_Q8_0: {
        int q = (int8_t)b[2 + e];
        *w = f16_at(b) * (double)q;
        *a = fabs(*w);
        return;
    }
    case BF_Q4_K:
    case BF_Q5_K: {
        const uint8_t *sc = b + 4;
        const uint8_t *qh = b + 16;
        const uint8_t *qs = b + (fmt == BF_Q4_K ? 16 : 48);
        int p = e / 64, r = e % 64, hi = r >= 32, l = r % 32;
        int j = 2 * p + hi;
        int q = hi ? (qs[32 * p + l] >> 4) : (qs[32 * p + l] & 15);
        if (fmt == BF_Q5_K)
            q += 16 * ((qh[l] >> j) & 1);
        int s, m;
        scale_min(sc, j, &s, &m);
        double t1 = f16_at(b) * (double)s * (double)q;
        double t2 = f16_at(b + 2) * (double)m;
        *w = t1 - t2;
        *a = fabs(t1) + fabs(t2);
        return;
    }
    case BF_Q6_K: {
        const uint8_t *ql = b, *qh = b + 128;
        const int8_t *sc = (const int8_t *)(b + 192);
        int h = e / 128, t = (e % 128) / 32, l = e % 32;
        int lo = ql[64 * h + 32 * (t & 1) + l];
        lo = (t >> 1) ? (lo >> 4) : (lo & 15);
        int hb = (qh[32 * h + l] >> (2 * t)) & 3;
        int q = lo | hb << 4;
        *w = f16_at(b + 208) * (double)sc[e / 16] * (double)(q - 32);
        *a = fabs(*w);
        return;
    }
    default:
        *w = NAN;
        *a = NAN;
    }
}

/* Weights of row n, element k, of an [N, K] matrix stored row after row,
 * each row K / elems blocks. */
static void weight(int fmt, const uint8_t *w, int64_t K, int64_t n, int64_t k,
                   double *wv, double *a)
{
    int64_t be, bb;
    blockref_geometry(fmt, &be, &bb);
    const uint8_t *blk = w + (n * (K / be) + k / be) * bb;
    element(fmt, blk, (int)(k % be), wv, a);
}

/* out[n*K + k] = (float) W(n, k); a single rounding of the exact value. */
void blockref_dequant(int fmt, const uint8_t *w, int64_t N, int64_t K, float *out)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            double v, a;
            weight(fmt, w, K, n, k, &v, &a);
            out[n * K + k] = (float)v;
        }
}

/* For each listed row n and activation row m:
 *   y[m, i]     = sum_k x[m,k] * W(n,k)        in f64, increasing k
 *   bound[m, i] = sum_k |x[m,k]| * a(n,k)      (a as in element()) */
void blockref_gemv_rows(int fmt, const float *x, const uint8_t *w, int64_t M,
                        int64_t N, int64_t K, const int64_t *rows, int64_t R,
                        double *y, double *bound)
{
    (void)N;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t i = 0; i < R; ++i) {
            int64_t n = rows[i];
            double s = 0.0, b = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double v, a;
                weight(fmt, w, K, n, k, &v, &a);
                double xv = (double)x[m * K + k];
                s += xv * v;
                b += fabs(xv) * a;
            }
            y[m * R + i] = s;
            bound[m * R + i] = b;
        }
}
