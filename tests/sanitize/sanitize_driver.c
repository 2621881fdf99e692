/*
 * Host-only driver for the sanitizer build (test infrastructure): exercises
 * the oracle's functions and the C ABI's host-only argument checks on small
 * and edge-case inputs, so that an address or undefined-behaviour
 * sanitizer sees every path.  Built and run by tests/test_sanitizers.py with
 * gcc -fsanitize=address,undefined; exits 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* oracle (oracle/litelinear_oracle.c) */
double oracle_e4m3fn_to_f64(uint8_t b);
double oracle_e4m3fnuz_to_f64(uint8_t b);
double oracle_bf16_to_f64(uint16_t h);
int oracle_forward_rows_q(const uint16_t *x, const uint16_t *A, const uint16_t *B, const uint8_t *Q, float scale,
                          const uint16_t *bias, int64_t M, int64_t in, int64_t out, int64_t r, const int64_t *rows,
                          int64_t nrows, double *y, double *T, int nthreads, int q_format);
int oracle_forward_rows_act8(const uint16_t *x, const uint16_t *A, const uint16_t *B, const uint8_t *Q, float scale,
                             const uint16_t *bias, int64_t M, int64_t in, int64_t out, int64_t r,
                             const int64_t *rows, int64_t nrows, double *y, double *T, int nthreads);
void oracle_quantize_rows(const uint16_t *x, int64_t M, int64_t in, uint8_t *codes, int32_t *exps);
void oracle_residual(const uint16_t *W, const uint16_t *A, const uint16_t *B, int64_t out, int64_t in, int64_t r,
                     double *R);
float oracle_quantize_tensor(const float *R, int64_t n, uint8_t *codes);

/* host-only argument checks of the C ABI (rank_fp8_residual_amd/csrc/check.cpp) */
int litelinear_check_args(const void *x, const void *A, const void *B, const void *Q, const void *bias,
                          const void *y, int64_t M, int64_t in, int64_t out, int64_t r, int y_bytes_per_elem);

static int failures = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

static uint16_t bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16); /* exact for the small integers used here */
}

int main(void) {
    /* decodes over every code */
    for (int c = 0; c < 256; ++c) {
        double a = oracle_e4m3fn_to_f64((uint8_t)c), b = oracle_e4m3fnuz_to_f64((uint8_t)c);
        CHECK(isnan(a) == (c == 0x7F || c == 0xFF));
        CHECK(isnan(b) == (c == 0x80));
    }
    /* forward on a small case, every row, T requested, both formats, act8 */
    enum { M = 5, IN = 48, OUT = 7, R = 3 };
    uint16_t x[M * IN], A[OUT * R], B[R * IN], bias[OUT];
    uint8_t Q[OUT * IN];
    for (int i = 0; i < M * IN; ++i) x[i] = bf16((float)((i * 7) % 9 - 4));
    for (int i = 0; i < OUT * R; ++i) A[i] = bf16((float)((i % 3) - 1));
    for (int i = 0; i < R * IN; ++i) B[i] = bf16((float)((i * 5) % 3 - 1));
    for (int i = 0; i < OUT; ++i) bias[i] = bf16(0.25f * (float)(i - 3));
    for (int i = 0; i < OUT * IN; ++i) Q[i] = (uint8_t)((i * 37) & 0x77);
    double y[M * OUT], T[M * R], y2[M * OUT];
    int64_t rows[3] = {4, 0, 2};
    CHECK(oracle_forward_rows_q(x, A, B, Q, 0.5f, bias, M, IN, OUT, R, NULL, M, y, T, 2, 0) == 0);
    CHECK(oracle_forward_rows_q(x, A, B, Q, 0.5f, bias, M, IN, OUT, R, rows, 3, y2, NULL, 1, 1) == 0);
    CHECK(oracle_forward_rows_act8(x, A, B, Q, 0.5f, NULL, M, IN, OUT, R, rows, 3, y2, NULL, 2) == 0);
    CHECK(oracle_forward_rows_q(x, NULL, NULL, Q, 1.0f, NULL, M, IN, OUT, 0, NULL, M, y, NULL, 1, 0) == 0);
    int64_t bad_rows[1] = {M};
    CHECK(oracle_forward_rows_q(x, A, B, Q, 1.0f, bias, M, IN, OUT, R, bad_rows, 1, y, NULL, 1, 0) == -1);
    CHECK(oracle_forward_rows_q(x, A, B, Q, 1.0f, bias, M, IN, OUT, R, NULL, M, y, NULL, 1, 2) == -1);
    /* quantisers and the residual */
    uint8_t codes[M * IN];
    int32_t exps[M];
    oracle_quantize_rows(x, M, IN, codes, exps);
    double Rd[OUT * IN];
    oracle_residual(x, A, B, 1, IN, R, Rd); /* x's first row as a 1 x IN weight */
    float Rf[OUT * IN];
    for (int i = 0; i < OUT * IN; ++i) Rf[i] = (float)((i % 11) - 5) * 0.01f;
    CHECK(oracle_quantize_tensor(Rf, OUT * IN, Q) > 0.0f);
    CHECK(oracle_quantize_tensor(Rf, 0, Q) == 1.0f);
    /* host-only argument checks: valid, edge and refused cases (fake,
     * aligned addresses: nothing is dereferenced) */
    const uintptr_t a16 = (uintptr_t)1 << 20;
    const void *px = (const void *)a16, *pA = (const void *)(2 * a16), *pB = (const void *)(3 * a16),
               *pQ = (const void *)(4 * a16), *pb = (const void *)(5 * a16), *py = (const void *)(64 * a16);
    CHECK(litelinear_check_args(px, pA, pB, pQ, pb, py, 4, 32, 8, 2, 2) == 0);
    CHECK(litelinear_check_args(px, pA, pB, pQ, pb, py, 0, 32, 8, 2, 2) == 0);
    CHECK(litelinear_check_args(px, pA, pB, pQ, pb, py, -1, 32, 8, 2, 2) == 1);
    CHECK(litelinear_check_args(px, pA, pB, pQ, pb, py, 4, 24, 8, 2, 2) == 2);
    CHECK(litelinear_check_args(px, pA, pB, pQ, pb, px, 4, 32, 8, 2, 2) == 1);
    CHECK(litelinear_check_args(px, pA, pB, pQ, pb, py, (int64_t)1 << 41, 32, 8, 2, 2) == 1);
    CHECK(litelinear_check_args(px, pA, pB, pQ, pb, py, INT64_MAX, INT64_MAX, INT64_MAX, INT64_MAX, 4) == 1);
    CHECK(litelinear_check_args(px, pA, pB, pQ, pb, py, 4, 32, 8, 2, 3) == 1);
    CHECK(litelinear_check_args(NULL, NULL, NULL, NULL, NULL, py, 4, 0, 8, 0, 2) == 0);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("sanitizer driver: all checks passed\n");
    return 0;
}
