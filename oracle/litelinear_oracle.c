/*
 * CPU oracle for the fused LiteLinear forward -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline
 * leg load this file's library.  The HIP library never links, includes or
 * calls it, and this file includes nothing from the HIP library.
 *
 * What it computes (LiteLinear README, page "moonmath-ai/LiteLinear", the
 * equation in the introduction, with the layouts of the Features list and of
 * SVDLinearLayer on the tt_compressor page, whose forward projects x onto B's
 * rows first and then applies A, with A [out, r] and B [r, in]):
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
 * e4m3fnuz, the residual's format on AMD hardware in the README's Features
 * list: the same fields, exponent bias 8, no negative zero and no
 * infinities.  0x80 (the would-be negative zero) is the only NaN;
 *   e == 0            : (-1)^s * f * 2^-10          (zero and subnormals)
 *   otherwise         : (-1)^s * (1 + f/8) * 2^(e-8) (largest: 0x7F = 240)
 */
double oracle_e4m3fnuz_to_f64(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 15, f = b & 7;
    double mag;
    if (b == 0x80)
        return NAN;
    if (e == 0)
        mag = ldexp((double)f, -10);
    else
#if ORACLE_PLANT == 13
        mag = ldexp(8.0 + f, e - 10); /* planted: the e4m3fn exponent bias */
#else
        mag = ldexp(8.0 + f, e - 11); /* (1 + f/8) * 2^(e-8) */
#endif
    return s ? -mag : mag;
}

void oracle_decode_e4m3fnuz(const uint8_t *codes, int64_t n, double *outv)
{
    for (int64_t i = 0; i < n; ++i)
        outv[i] = oracle_e4m3fnuz_to_f64(codes[i]);
}

/*
 * Forward for a list of rows of x.
 *   x     bf16 bits [M, in] row-major        A bf16 bits [out, r] row-major
 *   B     bf16 bits [r, in] row-major        Q 8-bit codes [out, in] row-major
 *   scale float32 dequant multiplier          bias bf16 bits [out] or NULL
 *   rows  nrows row indices into x (NULL: rows 0..nrows-1)
 *   y     double [nrows, out] (output)        T double [nrows, r] or NULL (output)
 *   q_format  0: Q holds e4m3fn codes; 1: e4m3fnuz codes
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_forward_rows_q(const uint16_t *x, const uint16_t *A, const uint16_t *B,
                          const uint8_t *Q, float scale, const uint16_t *bias,
                          int64_t M, int64_t in, int64_t out, int64_t r,
                          const int64_t *rows, int64_t nrows, double *y, double *T,
                          int nthreads, int q_format)
{
    double dec[256];
    double s = (double)scale;
    int bad = 0;
    if (M < 0 || in < 0 || out < 0 || r < 0 || nrows < 0 || !y || q_format < 0 || q_format > 1)
        return -1;
    if (nrows > 0 && (!x || (out > 0 && in > 0 && !Q) || (r > 0 && (!A || !B))))
        return -1;
    for (int i = 0; i < 256; ++i)
        dec[i] = q_format ? oracle_e4m3fnuz_to_f64((uint8_t)i) : oracle_e4m3fn_to_f64((uint8_t)i);
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

/* oracle_forward_rows_q for e4m3fn codes. */
int oracle_forward_rows(const uint16_t *x, const uint16_t *A, const uint16_t *B,
                        const uint8_t *Q, float scale, const uint16_t *bias,
                        int64_t M, int64_t in, int64_t out, int64_t r,
                        const int64_t *rows, int64_t nrows, double *y, double *T,
                        int nthreads)
{
    return oracle_forward_rows_q(x, A, B, Q, scale, bias, M, in, out, r, rows, nrows, y, T, nthreads, 0);
}

/*
 * Activations in e4m3fn (the optional fp8-activation mode).  Each row of x
 * gets a power-of-two scale 2^e, e the smallest integer with
 * max_j |x[m,j]| <= 448 * 2^e (and e >= -126; e = -126 for an all-zero row),
 * and every element becomes the e4m3fn code nearest to x[m,j] / 2^e, ties to
 * the even code.  x[m,j] / 2^e is exact (a power-of-two scaling of a bf16
 * value), so the only rounding is the one to e4m3fn.  A row holding a NaN or
 * an infinity gets e = 0 and every code 0x7F (NaN).
 */

/* Nearest e4m3fn code to a finite v with |v| <= 448, ties to even. */
static uint8_t e4m3fn_nearest(double v)
{
    int sign = v < 0 || (v == 0 && signbit(v));
    double a = fabs(v), q;
    int code, ex;
    if (a < ldexp(1.0, -6)) {
        /* zero and subnormals: multiples of 2^-9 (a result of 8 is 2^-6) */
        q = a * 512.0;
        double fl = floor(q);
        double fr = q - fl;
        int k = (int)fl;
        if (fr > 0.5 || (fr == 0.5 && (k & 1)))
            k += 1;
        code = k; /* k == 8 is the code of 2^-6 */
    } else {
        /* normal: a = (1 + f/8) 2^ex with ex in [-6, 8] */
        double mant = frexp(a, &ex); /* a = mant 2^ex, mant in [0.5, 1) */
        ex -= 1;
        mant *= 2.0;                 /* [1, 2) */
        q = (mant - 1.0) * 8.0;      /* [0, 8) */
        double fl = floor(q);
        double fr = q - fl;
        int f = (int)fl;
#if ORACLE_PLANT == 8
        if (fr >= 0.5) /* planted: ties away from zero */
#else
        if (fr > 0.5 || (fr == 0.5 && (f & 1)))
#endif
            f += 1;
        if (f == 8) {
            f = 0;
            ex += 1;
        }
        code = ((ex + 7) << 3) | f;
    }
    return (uint8_t)(code | (sign << 7));
}

/* Scale exponent of a row (see above); returns 0 and sets *nonfinite for a
 * row holding a NaN or an infinity. */
static int row_scale_exp(const uint16_t *xr, int64_t in, int *nonfinite)
{
    double amax = 0.0;
    int ex, e;
    *nonfinite = 0;
    for (int64_t j = 0; j < in; ++j) {
        double v = oracle_bf16_to_f64(xr[j]);
        if (!isfinite(v)) {
            *nonfinite = 1;
            return 0;
        }
        if (fabs(v) > amax)
            amax = fabs(v);
    }
    if (amax == 0.0)
        return -126;
    /* amax = mant 2^ex, mant in [0.5, 1); 448 2^e = 0.875 2^(e + 9) */
    double mant = frexp(amax, &ex);
#if ORACLE_PLANT == 9
    e = ex - 9; /* planted: the scale may leave amax above 448 */
#else
    e = mant <= 0.875 ? ex - 9 : ex - 8;
#endif
    return e < -126 ? -126 : e;
}

/*
 * x bf16 bits [M, in] -> codes [M, in] and exponents e[M] (scale 2^e).
 */
void oracle_quantize_rows(const uint16_t *x, int64_t M, int64_t in, uint8_t *codes, int32_t *exps)
{
    for (int64_t m = 0; m < M; ++m) {
        int nonfinite;
        int e = row_scale_exp(x + m * in, in, &nonfinite);
        exps[m] = e;
        for (int64_t j = 0; j < in; ++j)
            codes[m * in + j] = nonfinite ? 0x7F : e4m3fn_nearest(ldexp(oracle_bf16_to_f64(x[m * in + j]), -e));
    }
}

/*
 * Forward of the fp8-activation mode for a list of rows: as
 * oracle_forward_rows, but the residual product reads x as
 * 2^e[m] * dec(codes[m, j]) (the row's quantised activations); the low-rank
 * projection T = x B^T still reads the bf16 x.
 */
int oracle_forward_rows_act8(const uint16_t *x, const uint16_t *A, const uint16_t *B,
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
        double *xr, *xq, *tr;
        uint8_t *cr;
        int32_t e;
        if (m < 0 || m >= M) {
            bad = 1;
            continue;
        }
        xr = (double *)malloc(sizeof(double) * (size_t)(in > 0 ? in : 1));
        xq = (double *)malloc(sizeof(double) * (size_t)(in > 0 ? in : 1));
        tr = (double *)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
        cr = (uint8_t *)malloc((size_t)(in > 0 ? in : 1));
        if (!xr || !xq || !tr || !cr) {
            free(xr);
            free(xq);
            free(tr);
            free(cr);
            bad = 1;
            continue;
        }
        oracle_quantize_rows(x + m * in, 1, in, cr, &e);
        for (int64_t j = 0; j < in; ++j) {
            xr[j] = oracle_bf16_to_f64(x[m * in + j]);
            xq[j] = ldexp(dec[cr[j]], e);
        }
        for (int64_t k = 0; k < r; ++k) {
            double acc = 0.0;
            for (int64_t j = 0; j < in; ++j)
#if ORACLE_PLANT == 10
                acc += xq[j] * oracle_bf16_to_f64(B[k * in + j]); /* planted: T from the quantised x */
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
                lr += tr[k] * oracle_bf16_to_f64(A[n * r + k]);
            for (int64_t j = 0; j < in; ++j)
                res += xq[j] * dec[Q[n * in + j]];
            v = lr + s * res;
            if (bias)
                v += oracle_bf16_to_f64(bias[n]);
            y[i * out + n] = v;
        }
        free(xr);
        free(xq);
        free(tr);
        free(cr);
    }
    return bad ? -1 : 0;
}

/*
 * Decomposition side (the step upstream of the forward: LiteLinear README,
 * *Usage*, "From a dense nn.Linear": LiteLinear.from_dense, SVD-based;
 * *Features*: W ~ A.B + Q_fp8 with a per-tensor Q_scale_inv).
 *
 * Residual: R = W - A B in double, W bf16 [out, in], A bf16 [out, r],
 * B bf16 [r, in].
 */
void oracle_residual(const uint16_t *W, const uint16_t *A, const uint16_t *B, int64_t out, int64_t in,
                     int64_t r, double *R)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < out; ++n)
        for (int64_t j = 0; j < in; ++j) {
            double ab = 0.0;
            for (int64_t k = 0; k < r; ++k)
#if ORACLE_PLANT == 11
                ab += oracle_bf16_to_f64(A[n * r + k]) * oracle_bf16_to_f64(B[j * r + k]); /* planted: B read transposed */
#else
                ab += oracle_bf16_to_f64(A[n * r + k]) * oracle_bf16_to_f64(B[k * in + j]);
#endif
            R[n * in + j] = oracle_bf16_to_f64(W[n * in + j]) - ab;
        }
}

/*
 * Per-tensor e4m3fn quantiser of a float32 residual: s = amax / 448 in
 * float32 (1 when amax is 0), and each code the e4m3fn value nearest to
 * the float32 quotient R / s clamped to +-448 (ties to even).  R must be
 * finite.  Returns s; the dequantised residual is s * dec(code).
 */
float oracle_quantize_tensor(const float *R, int64_t n, uint8_t *codes)
{
    float amax = 0.0f, s;
    for (int64_t i = 0; i < n; ++i)
        if (fabsf(R[i]) > amax)
            amax = fabsf(R[i]);
#if ORACLE_PLANT == 12
    s = amax > 0.0f ? amax / 240.0f : 1.0f; /* planted: the fnuz maximum */
#else
    s = amax > 0.0f ? amax / 448.0f : 1.0f;
#endif
    for (int64_t i = 0; i < n; ++i) {
        float q = R[i] / s;
        if (q > 448.0f)
            q = 448.0f;
        if (q < -448.0f)
            q = -448.0f;
        codes[i] = e4m3fn_nearest((double)q);
    }
    return s;
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
