/*
 * q4ref.c -- plain CPU oracle for the int4 decode GEMV, its dense control,
 * the dequantiser and the two bandwidth probes.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, link or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the
 * HIP library; the two meet only through the seeded input arrays.
 *
 * Every function is the plain definition written out, in f64, one element at
 * a time, in increasing index order, with no blocking or reordering.
 *
 * Storage format (gerbil "WGSL Kernel Reference", section 3 MatMulInt4,
 * "INT4 Packing" and "Dequantization"; weights read N-major, W_q[N, K]):
 *   wq[n*(K/2) + k/2]        holds code q(n,k): low nibble for even k,
 *                            high nibble for odd k
 *   scales[n*G + j]          binary16 bits of the scale of group j = k / g
 *   zeros[n*ZB + j/2]        zero point z(n,j): low nibble for even j,
 *                            high nibble for odd j, ZB = ceil(G/2)
 *   W(n,k) = (q(n,k) - z(n, k/g)) * s(n, k/g)        (same section, "Dequantization")
 *   y[m,n] = sum_k x[m,k] * W(n,k)                   (section 3, "Computes")
 *
 * Parity status of each function (what pins it, outside itself):
 *   q4ref_f16_to_f64   all 65536 patterns against numpy's binary16
 *   q4ref_dequant      one-hot and u32-packed brute force written from the
 *                      page's flat-index group formula; z = 8 closed form;
 *                      round trip with q4ref_quantize on exact weights
 *   q4ref_gemv_q4      q = z gives exactly 0; z = 8, q = c, x = 1 closed form;
 *                      numpy float64 matmul of an independently dequantised W;
 *                      integer-exact inputs against Python integer arithmetic
 *   q4ref_gemv_f32     numpy float64 matmul; integer-exact inputs
 *   q4ref_sum          all-ones buffer sums to n; numpy float64 sum
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

/* IEEE 754 binary16: sign bit 15, 5-bit biased exponent (bias 15) in bits
 * 14..10, 10-bit fraction.  Exponent 0 encodes zero and subnormals
 * (f * 2^-24); exponent 31 encodes infinities (f = 0) and NaNs. */
double q4ref_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);  /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

static int code_at(const uint8_t *wq, int64_t K, int64_t n, int64_t k)
{
    uint8_t b = wq[n * (K / 2) + k / 2];
    return (k & 1) ? (b >> 4) : (b & 0x0F);
}

static int zero_at(const uint8_t *zeros, int64_t G, int64_t n, int64_t j)
{
    int64_t zb = (G + 1) / 2;
    uint8_t b = zeros[n * zb + j / 2];
    return (j & 1) ? (b >> 4) : (b & 0x0F);
}

/* The exact dequantised weight.  |q - z| <= 15 needs 4 bits and a binary16
 * scale carries 11 significant bits, so the product is exact in f64 and in
 * f32 alike. */
static double weight_at(const uint8_t *wq, const uint16_t *scales,
                        const uint8_t *zeros, int64_t K, int64_t g,
                        int64_t n, int64_t k)
{
    int64_t G = K / g;
    int64_t j = k / g;
    int q = code_at(wq, K, n, k);
    int z = zero_at(zeros, G, n, j);
    double s = q4ref_f16_to_f64(scales[n * G + j]);
    return (double)(q - z) * s;
}

/* W[n,k] as float and/or the raw codes q(n,k), both [N, K] row-major.
 * Either output may be NULL. */
void q4ref_dequant(const uint8_t *wq, const uint16_t *scales, const uint8_t *zeros,
                   int64_t N, int64_t K, int64_t g, float *w_out, uint8_t *codes_out)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            if (w_out)
                w_out[n * K + k] = (float)weight_at(wq, scales, zeros, K, g, n, k);
            if (codes_out)
                codes_out[n * K + k] = (uint8_t)code_at(wq, K, n, k);
        }
}

/* y[m,r] = sum_k x[m,k] W(rows[r],k) in f64, and bound[m,r] = sum_k |x W|,
 * for the rows listed (all rows when rows == NULL, then nrows = N).
 * Outputs are [M, nrows] row-major. */
void q4ref_gemv_q4_rows(const float *x, const uint8_t *wq, const uint16_t *scales,
                        const uint8_t *zeros, int64_t M, int64_t N, int64_t K,
                        int64_t g, const int64_t *rows, int64_t nrows,
                        double *y, double *bound)
{
    (void)N;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t n = rows ? rows[r] : r;
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double t = (double)x[m * K + k] * weight_at(wq, scales, zeros, K, g, n, k);
                acc += t;
                mag += fabs(t);
            }
            y[m * nrows + r] = acc;
            if (bound)
                bound[m * nrows + r] = mag;
        }
}

void q4ref_gemv_q4(const float *x, const uint8_t *wq, const uint16_t *scales,
                   const uint8_t *zeros, int64_t M, int64_t N, int64_t K, int64_t g,
                   double *y, double *bound)
{
    q4ref_gemv_q4_rows(x, wq, scales, zeros, M, N, K, g, NULL, N, y, bound);
}

/* Dense control: y[m,r] = sum_k x[m,k] w[rows[r],k] with w f32 [N, K]. */
void q4ref_gemv_f32_rows(const float *x, const float *w, int64_t M, int64_t N,
                         int64_t K, const int64_t *rows, int64_t nrows,
                         double *y, double *bound)
{
    (void)N;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t n = rows ? rows[r] : r;
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double t = (double)x[m * K + k] * (double)w[n * K + k];
                acc += t;
                mag += fabs(t);
            }
            y[m * nrows + r] = acc;
            if (bound)
                bound[m * nrows + r] = mag;
        }
}

void q4ref_gemv_f32(const float *x, const float *w, int64_t M, int64_t N, int64_t K,
                    double *y, double *bound)
{
    q4ref_gemv_f32_rows(x, w, M, N, K, NULL, N, y, bound);
}

/* Read probe reference: the f64 sum and absolute sum of a float buffer. */
void q4ref_sum(const float *buf, int64_t n, double *sum, double *abssum)
{
    double s = 0.0, a = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        s += (double)buf[i];
        a += fabs((double)buf[i]);
    }
    *sum = s;
    *abssum = a;
}

/* Test helper, not part of the method on the pages: the inverse map
 * q = clamp(round_half_even(w / s) + z, 0, 15), packed back into wq.
 * Used only to check that dequantisation round-trips exactly. */
void q4ref_quantize(const float *w, const uint16_t *scales, const uint8_t *zeros,
                    int64_t N, int64_t K, int64_t g, uint8_t *wq_out)
{
    int64_t G = K / g;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t j = k / g;
            double s = q4ref_f16_to_f64(scales[n * G + j]);
            double t = nearbyint((double)w[n * K + k] / s) + zero_at(zeros, G, n, j);
            int q = t < 0.0 ? 0 : (t > 15.0 ? 15 : (int)t);
            uint8_t *b = &wq_out[n * (K / 2) + k / 2];
            if (k & 1)
                *b = (uint8_t)((*b & 0x0F) | (q << 4));
            else
                *b = (uint8_t)((*b & 0xF0) | q);
        }
}
