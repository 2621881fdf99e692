/*
 * CPU oracle for the fused LiteLinear forward -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline
 * leg load this file's library.  The HIP library never links, includes or
 * calls it, and this file includes nothing from the HIP library.
 *
 * What it computes (LiteLinear README, page "moonmath-ai/LiteLinear", the
 * equation in the introduction, with the layouts of the Features list and of
 * SVDLinearLayer on the tt_compressor page, "Forward: y = (x @ B.T) @ A.T"):
 *
 *     T[m,k] = sum_j x[m,j] * B[k,j]
 *     y[m,n] = sum_k T[m,k] * A[n,k] + scale * sum_j x[m,j] * dec(Q[n,j]) + bias[n]
 *
 * Every input is turned into a double exactly (bf16 and float32 are subsets
 * of double, and so is every e4m3fn value), every sum runs in double in
 * plain index order, and nothing is rounded to a narrower type.  The result
 * is the exact value up to double rounding of the sums.
 *
 * dec() is the OCP 8-bit floating point e4m3fn format that the README names
 * for the residual (Features: "Q_fp8 in e4m3fn"): sign s = b>>7, exponent
 * field e = (b>>3)&15 with bias 7, mantissa field f = b&7;
 *   e == 0            : (-1)^s * (f/8) * 2^-6       (zero and subnormals)
 *   0x7F and 0xFF     : NaN (the format has no infinities)
 *   otherwise         : (-1)^s * (1 + f/8) * 2^(e-7) (largest: 448)
 *
 * ORACLE_PLANT selects a deliberately wrong variant; only the pin tests build
 * it, to show that each pin catches a plausible mistake.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_PLANT
#define ORACLE_PLANT 0
#endif

double oracle_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16; /* bf16 is the top half of a float32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_e4m3fn_to_f64(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 15, f = b & 7;
    double mag;
    if (e == 15 && f == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)f, -9); /* f/8 * 2^-6 */
    else
#if ORACLE_PLANT == 4
        mag = ldexp(8.0 + f, e - 9); /* planted: exponent bias off by one */
#else
        mag = ldexp(8.0 + f, e - 10); /* (1 + f/8) * 2^(e-7) */
#endif
#if ORACLE_PLANT == 3
    if (e == 0) return mag; /* planted: sign lost on subnormals */
#endif
    return s ? -mag : mag;
}

void oracle_decode_e4m3fn(const uint8_t *codes, int64_t n, double *outv)
{
    for (int64_t i = 0; i < n; ++i)
        outv[i] = oracle_e4m3fn_to_f64(codes[i]);
}

/*
 * Forward for a list of rows of x.
 *   x     bf16 bits [M, in] row-major        A bf16 bits [out, r] row-major
 *   B     bf16 bits [r, in] row-major        Q e4m3fn codes [out, in] row-major
 *   scale float32 dequant multiplier          bias bf16 bits [out] or NULL
 *   rows  nrows row indices into x (NULL: rows 0..nrows-1)
 *   y     double [nrows, out] (output)        T double [nrows, r] or NULL (output)
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_forward_rows(const uint16_t *x, const uint16_t *A, const uint16_t *B,
                        const uint8_t *Q, float scale, const uint16_t *bias,
                        int64_t M, int64_t in, int64_t out, int64_t r,
                        const int64_t *rows, int64_t nrows, double *y, double *T,
                        int nthreads)
{
    double dec[256];
    double s = (double)scale;
    int bad = 0;
    if (M < 0 || in < 0 || out < 0 || r < 0 || nrows < 0 || !y)
        return -1;
    if (nrows > 0 && (!x || (out > 0 && in > 0 && !Q) || (r > 0 && (!A || !B))))
        return -1;
    for (int i = 0; i < 256; ++i)
        dec[i] = oracle_e4m3fn_to_f64((uint8_t)i);
    if (nthreads < 1)
        nthreads = 1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t m = rows ? rows[i] : i;
        double *xr, *tr;
        if (m < 0 || m >= M) {
            bad = 1;
            continue;
        }
        xr = (double *)malloc(sizeof(double) * (size_t)(in > 0 ? in : 1));
        tr = (double *)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
        if (!xr || !tr) {
            free(xr);
            free(tr);
            bad = 1;
            continue;
        }
        for (int64_t j = 0; j < in; ++j)
            xr[j] = oracle_bf16_to_f64(x[m * in + j]);
        /* low-rank projection T = x B^T */
        for (int64_t k = 0; k < r; ++k) {
            double acc = 0.0;
            for (int64_t j = 0; j < in; ++j)
#if ORACLE_PLANT == 6
                acc += xr[j] * oracle_bf16_to_f64(B[j * r + k]); /* planted: B transposed */
#else
                acc += xr[j] * oracle_bf16_to_f64(B[k * in + j]);
#endif
            tr[k] = acc;
            if (T)
                T[i * r + k] = acc;
        }
        for (int64_t n = 0; n < out; ++n) {
            double lr = 0.0, res = 0.0, v;
            for (int64_t k = 0; k < r; ++k)
#if ORACLE_PLANT == 5
                lr += tr[k] * oracle_bf16_to_f64(A[k * out + n]); /* planted: A transposed */
#else
                lr += tr[k] * oracle_bf16_to_f64(A[n * r + k]);
#endif
            for (int64_t j = 0; j < in; ++j)
                res += xr[j] * dec[Q[n * in + j]];
#if ORACLE_PLANT == 2
            v = lr + res; /* planted: scale ignored */
#elif ORACLE_PLANT == 7
            v = s * res; /* planted: low-rank term dropped */
#else
            v = lr + s * res;
#endif
#if ORACLE_PLANT != 1 /* planted 1: bias dropped */
            if (bias)
                v += oracle_bf16_to_f64(bias[n]);
#endif
            y[i * out + n] = v;
        }
        free(xr);
        free(tr);
    }
    return bad ? -1 : 0;
}

/* Reports how many OpenMP threads a parallel region actually gets. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
