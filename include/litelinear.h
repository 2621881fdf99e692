/*
 * litelinear.h -- C ABI of the fused LiteLinear forward for AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (LiteLinear README, page "moonmath-ai/LiteLinear": the
 * equation in the introduction, and the Features list):
 *
 *     y = (x B^T) A^T + scale * (x dec(Q)^T) + bias
 *
 * i.e. a linear layer whose weight is held as W ~ A B + scale * dec(Q): a
 * bf16 rank-r pair A [out, r], B [r, in] (the layout of SVDLinearLayer on the
 * tt_compressor page) plus a residual Q stored as OCP e4m3fn codes with one
 * per-tensor dequantisation multiplier `scale` (the README's state key
 * Q_scale_inv).  Activations x are bf16 [M, in] (all leading dimensions of
 * the caller's tensor flattened into M rows); y is bf16 [M, out].
 *
 * Conventions for every entry point:
 *   - All matrices are dense, row-major, with leading dimension equal to the
 *     row length.  Pointers are device pointers on the handle's device.
 *   - The caller owns every tensor.  The library never frees them and does
 *     not keep them past the point where the stream passes the call.
 *   - Nothing throws or aborts across this ABI; every call returns a status.
 *   - A kernel fault shows up as a HIP error at the caller's next
 *     synchronisation, not as a status of the call that queued it.
 *   - Work-groups of one forward launch hand T = x B^T to each other through
 *     device counters.  Their waits rely on work-groups being dispatched in
 *     id order (producers first) and are bounded; a wait that gives up sets
 *     the handle's error word, and the next forward call on the handle (or
 *     litelinear_device_status) returns LITELINEAR_ERR_SYNC.
 *   - Graph capture: every forward entry point may be captured into a HIP
 *     graph and replayed, once a call of the same or a larger shape has run
 *     on the handle outside capture (so that its workspace exists).  The
 *     counters are back at zero after every launch, and a captured call
 *     queues no allocation, memset or event.  A call under capture that
 *     would have to grow the workspace returns LITELINEAR_ERR_UNSUPPORTED.
 */
#ifndef LITELINEAR_H
#define LITELINEAR_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct litelinear_ctx *litelinear_handle_t; /* opaque, library-owned */

typedef enum {
    LITELINEAR_OK = 0,
    LITELINEAR_ERR_INVALID_ARG = 1, /* NULL required pointer, negative size, y overlapping an input */
    LITELINEAR_ERR_UNSUPPORTED = 2, /* in % 16 != 0, or x / Q / B / y not 16-byte aligned */
    LITELINEAR_ERR_HIP = 3,         /* a HIP runtime call or kernel launch failed */
    LITELINEAR_ERR_OOM = 4,         /* workspace allocation failed */
    LITELINEAR_ERR_SYNC = 5,        /* an earlier launch on this handle gave up waiting for other
                                       work-groups of the launch: its output is undefined (see
                                       litelinear_device_status) */
    LITELINEAR_ERR_SCRATCH = 6      /* litelinear_forward_noalloc: the call needs more workspace than
                                       the fixed scratch holds (nothing was queued) */
} litelinear_status_t;

/* Options set per handle with litelinear_set_option(). */
typedef enum {
    /* Kernel family.  0 = choose from the shape (default): the skinny
     * kernels for M <= 64 (but for tiny problems, 32 < M, in <= 256 and
     * M * in * out <= 2^22, where the tiled kernel computes T inside each
     * output tile), else the tiled kernel; 1 = the skinny kernels (HBM-bound
     * on Q, for small M: up to 16 rows with 2048 < in <= 8192 and at least
     * 192 groups of 32 output columns, and no K-split hint, each work-group
     * streams its columns over all of `in`; otherwise work-groups split `in`
     * into slices whose partial sums the last one of each column tile adds);
     * 2 = the tiled kernel (MFMA-bound, for large M).  All compute the same
     * operation; a kernel that does not take the shape returns UNSUPPORTED. */
    LITELINEAR_OPT_PATH = 1,
    /* Output type.  0 = bf16 y (default, rounded to nearest even);
     * 1 = float32 y [M, out] (no output rounding; y must hold 4*M*out bytes). */
    LITELINEAR_OPT_OUTPUT_F32 = 2,
    /* Skinny path K-split hint.  0 = choose automatically, else the wanted
     * number of slices of `in`; each slice is a power of two from 512 to
     * 4096 elements of `in` (at most 4096 / ceil(M / 16)), the smallest that
     * does not give more slices than the hint. */
    LITELINEAR_OPT_SPLIT_K = 3,
    /* Per-kernel timing.  1 = record a HIP event pair around every kernel
     * the handle launches, on the caller's stream; read the totals with
     * litelinear_kernel_time().  0 = off (default). */
    LITELINEAR_OPT_PROFILE = 4,
    /* Tiled path: K slices per 64-column block of T = x B^T.  0 = choose
     * automatically (default); n > 0 = n slices (at most the number of
     * 64-element steps of `in`), computed by separate work-groups and summed
     * in slice order. */
    LITELINEAR_OPT_T_SPLITS = 5,
    /* Activations of the residual product.  0 = bf16 x (default); 1 = x
     * quantised to e4m3fn with one power-of-two scale per row (exactly as
     * litelinear_quantize_rows() does, on the handle's workspace) and the
     * residual product run on the fp8 matrix cores:
     *     y = (x B^T) A^T + scale * diag(2^e) (dec(codes) dec(Q)^T) + bias
     * T = x B^T still reads the bf16 x.  This is an approximation of the
     * forward (the pages run the fp8 residual against bf16 activations).
     * On normally distributed activations (with or without outlier
     * channels) it was measured within 0.13 RMS(y) of the exact y
     * element-wise and within 2.4e-2 in relative L1; its tests allow 0.25
     * RMS(y) and 4e-2.  Runs on the tiled kernel only (with
     * LITELINEAR_OPT_PATH = 1 the forward returns UNSUPPORTED). */
    LITELINEAR_OPT_ACT_FP8 = 6,
    /* Activation fused into the epilogue, for activation projections such
     * as the feed-forward input projections of the LTX-Video transformer
     * whose shapes the LiteLinear README benchmarks (*Performance Benchmark
     * on shapes captured from LTX-Video*).  0 = none (default); 1 = GELU in
     * its tanh approximation (Hendrycks and Gimpel, "Gaussian Error Linear
     * Units (GELUs)", 2016) applied to every element of y after the bias:
     *     y = gelu(v) = 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))),
     * v the forward's float32 value, before the one rounding to bf16 (or
     * none with LITELINEAR_OPT_OUTPUT_F32).  Both paths, the fp8-activation
     * mode and both outputs of litelinear_forward_pair().
     * 2 = GEGLU, the gated activation of a projection that a GEGLU module
     * wraps (the README's *Integration guide* passes such an activation
     * projection through LiteLinear; Shazeer, "GLU Variants Improve
     * Transformer", 2020): Q, A and bias hold out = 2F rows, the hidden half
     * first and then the gate, and
     *     y [M, F] = v[:, :F] * GELU(v[:, F:]),  GELU(u) = u Phi(u) exactly
     *     (0.5 u (1 + erf(u / sqrt(2))), the device library's erff),
     * v the forward's float32 value [M, 2F], rounded once at the end.  out
     * must be even; y has out / 2 columns.  Both paths and the
     * fp8-activation mode; litelinear_forward_pair() returns UNSUPPORTED. */
    LITELINEAR_OPT_ACTIVATION = 7,
    /* Test hook for the error path.  0 = off (default); n > 0 = every bounded
     * wait of the following forward launches looks for one count more than
     * the launch produces and gives up after n polls, so the kernels finish
     * normally and the error word gets set (the outputs are undefined). */
    LITELINEAR_OPT_TEST_WAIT_TIMEOUT = 8,
    /* Format of the residual codes Q.  0 = OCP e4m3fn (default: bias 7, max
     * 448, NaN 0x7F/0xFF); 1 = e4m3fnuz, the format the LiteLinear README's
     * Features list names for AMD hardware (bias 8, max 240 at 0x7F, no
     * negative zero, no infinities, 0x80 the only NaN).  Every code is
     * decoded exactly either way.  e4m3fnuz runs with bf16 activations only
     * (with LITELINEAR_OPT_ACT_FP8 the forward returns UNSUPPORTED) and on
     * output tiles of at most 256 x 128. */
    LITELINEAR_OPT_Q_FORMAT = 9,
    /* Tiled path: how T = x B^T is computed.  0 = choose automatically
     * (default); 1 = by producer work-groups inside the output tiles' launch
     * (they hold back some output tiles until T is done); 2 = by a launch of
     * its own queued just before, where the shape allows it: r <= 128,
     * in <= 8192 (4096 for r > 64), T handed over through memory in
     * 64-column blocks (not for ranks that are multiples of 256 on 256 x 256
     * tiles, nor where tiny problems compute T inside each output tile);
     * otherwise as 1.  Automatic: a launch of its own for
     * grids of fewer than four rounds of one output tile per compute unit
     * whose last round has no free slots for the producers.  Either way T'
     * is the same float32 sum rounded once; only its order of additions
     * differs. */
    LITELINEAR_OPT_T_LAUNCH = 10
} litelinear_option_t;

/* Kernels whose time litelinear_kernel_time() reports. */
typedef enum {
    LITELINEAR_KERNEL_PAD_A = 0,  /* copy of A into a zero-padded [out, r_pad] buffer (either path,
                                     only when r % 8 != 0 or A is not 16-byte aligned) */
    LITELINEAR_KERNEL_MAIN = 1,   /* tiled path: T = x B^T, residual, rank-r product and bias */
    LITELINEAR_KERNEL_SKINNY = 2, /* skinny path (either skinny kernel): the same in one launch */
    LITELINEAR_KERNEL_QUANT = 3,  /* activations to e4m3fn (LITELINEAR_OPT_ACT_FP8, litelinear_quantize_rows) */
    LITELINEAR_KERNEL_CONVERT = 4 /* decomposition side: litelinear_quantize_tensor, litelinear_residual_quantize
                                     (both passes of one call count as one launch) */
} litelinear_kernel_t;

/*
 * Create a handle bound to HIP device `device_ordinal`.  The handle owns the
 * workspace (the T = x B^T buffer and per-row-tile counters of the tiled
 * path, a padded copy of A for ranks that are not a multiple of 8, the
 * split-K partial sums and counters of the skinny path, the e4m3fn codes and
 * row scales of x in the fp8-activation mode); it grows on demand
 * inside the forward calls, stream-ordered on the call's stream
 * (hipMallocAsync / hipFreeAsync: no other stream or device-wide wait).
 * Calls on one handle must be ordered (one stream at a time, or streams the
 * caller orders with events): they share the workspace.  The handle also
 * owns one word of pinned host memory, mapped into the device, in which
 * kernels report a wait that gave up.
 * Errors: INVALID_ARG (out == NULL or no such device), HIP, OOM.
 */
litelinear_status_t litelinear_create(litelinear_handle_t *out, int device_ordinal);

/*
 * y = (x B^T) A^T + scale * (x dec(Q)^T) + bias, queued on `stream`.
 *
 *   x     bf16  [M, in]   16-byte aligned.
 *   A     bf16  [out, r]  may be NULL iff r == 0.
 *   B     bf16  [r, in]   16-byte aligned; may be NULL iff r == 0.
 *   Q     uint8 [out, in] OCP e4m3fn codes (bias 7, max 448, NaN 0x7F/0xFF),
 *                         16-byte aligned.  Every code is decoded exactly.
 *   scale float32 dequantisation multiplier: residual = scale * dec(Q).
 *   bias  bf16  [out] or NULL (no bias).
 *   y     bf16  [M, out] (float32 with LITELINEAR_OPT_OUTPUT_F32),
 *                         16-byte aligned; must not overlap any input.
 *   M, in, out, r  sizes; M == 0 or out == 0 returns OK without a launch.
 *   stream  HIP stream of the handle's device (NULL = default stream).
 *
 * Precision: products in bf16 x bf16 (every e4m3fn value is exact in bf16)
 * with float32 accumulation; T = x B^T is rounded once to bf16 before the
 * rank-r product; y is rounded once (nearest even) to bf16.
 * The call returns without synchronising; inputs must stay valid until the
 * stream passes it.  Errors: INVALID_ARG, UNSUPPORTED, HIP, OOM, and SYNC
 * (returned instead of queueing anything when an earlier launch's wait gave
 * up; the call after it runs normally).
 */
litelinear_status_t litelinear_forward(litelinear_handle_t h,
                                       const void *x, const void *A, const void *B,
                                       const void *Q, float scale, const void *bias,
                                       void *y, int64_t M, int64_t in, int64_t out,
                                       int64_t r, hipStream_t stream);

/*
 * litelinear_forward() for callers that cannot allocate memory: code under
 * HIP graph capture that must not add allocation nodes, tight serving loops,
 * harnesses that forbid hipMalloc.  The same kernels, options and results
 * as litelinear_forward(), but the workspace (T' blocks, partial sums,
 * counters, a padded copy of A, e4m3fn activations) is carved out of a
 * fixed scratch array of 32 MiB per device, a file-scope device array of
 * the library that each device holds until the process ends; the call
 * allocates nothing (no hipMalloc, hipFree or event), and queues a small
 * kernel that clears the counters it uses, then the forward.
 *
 *   Arguments, layouts and ownership as litelinear_forward().
 *   Every call on one device shares that device's scratch: calls that can
 *   overlap on one device (different streams, or different handles without
 *   ordering between them) race and must be ordered by the caller.
 *   The workspace needed: counters (at most 64 KiB), plus 2 M r_pad bytes of
 *   T' (tiled path), up to 4 t_splits M r_pad bytes of T partial sums, for
 *   the skinny path 4 splits M out bytes of partial sums, 2 out r_pad bytes
 *   for a padded A, and M (in + 4) bytes with e4m3fn activations, each
 *   rounded up to 256 bytes.
 * Errors: those of litelinear_forward(), and SCRATCH (nothing queued) when
 * the call needs more than the scratch holds (for example the 16384 x 4096
 * e4m3fn-activation forward, whose activation codes alone take 64 MiB).
 */
litelinear_status_t litelinear_forward_noalloc(litelinear_handle_t h,
                                               const void *x, const void *A, const void *B,
                                               const void *Q, float scale, const void *bias,
                                               void *y, int64_t M, int64_t in, int64_t out,
                                               int64_t r, hipStream_t stream);

/*
 * litelinear_forward() on activations whose rows are `ldx` elements apart:
 * x is a row slice of a wider bf16 tensor (for example one part of a fused
 * projection's output, or every other token of a sequence), read in place
 * with no copy.  ldx = in is litelinear_forward().
 *
 *   x     bf16, row m at x + m * ldx elements, `in` of them used; 16-byte
 *         aligned, ldx >= in and ldx % 8 == 0 (every row 16-byte aligned).
 *   the other arguments as in litelinear_forward(); y does not overlap
 *   x's extent, (M - 1) * ldx + in elements.
 * Errors: INVALID_ARG (ldx < in), UNSUPPORTED (ldx % 8 != 0), and those of
 * litelinear_forward().
 */
litelinear_status_t litelinear_forward_strided(litelinear_handle_t h,
                                               const void *x, int64_t ldx, const void *A,
                                               const void *B, const void *Q, float scale,
                                               const void *bias, void *y, int64_t M, int64_t in,
                                               int64_t out, int64_t r, hipStream_t stream);

/*
 * Activations to e4m3fn with one power-of-two scale per row, queued on
 * `stream` (the first step of LITELINEAR_OPT_ACT_FP8, also usable alone).
 *
 *   x       bf16    [M, in]  16-byte aligned.
 *   codes   uint8   [M, in]  8-byte aligned; OCP e4m3fn codes.
 *   scales  float32 [M]      4-byte aligned; scales[m] = 2^e[m].
 *
 * e[m] is the smallest integer, at least -126, with
 * max_j |x[m,j]| <= 448 * 2^e[m] (-126 for an all-zero row), and codes[m,j]
 * is the e4m3fn value nearest to x[m,j] / 2^e[m] (an exact quotient), ties
 * to the even code, with x's sign (so -0 and small negatives give 0x80).  A
 * row holding a NaN or an infinity gets scales[m] = 1 and every code 0x7F.
 * The outputs must not overlap x or each other.  M == 0 returns OK without a
 * launch.  Errors: INVALID_ARG, UNSUPPORTED (in % 16 != 0, misaligned
 * pointer, in >= 2^30), HIP.
 */
litelinear_status_t litelinear_quantize_rows(litelinear_handle_t h, const void *x, int64_t M, int64_t in,
                                             void *codes, float *scales, hipStream_t stream);

/*
 * Decomposition side (LiteLinear README, *Usage*: LiteLinear.from_dense
 * builds the pair by an SVD of the dense weight; *Features*:
 * W ~ A B + Q_fp8 with Q_fp8 in e4m3fn and a per-tensor Q_scale_inv).
 *
 * litelinear_quantize_tensor: per-tensor e4m3fn codes of a float32 array.
 *   R          float32 [n]  16-byte aligned, finite; n % 4 == 0.
 *   codes      uint8   [n]  4-byte aligned.
 *   scale_out  float32 device pointer: s = max|R| / 448 (1 when R is all
 *              zero), a correctly rounded float32 division.
 *   codes[i] is the e4m3fn value nearest to clamp(R[i] / s, -448, 448), the
 *   quotient a correctly rounded float32 division, ties to the even code;
 *   R ~ s * dec(codes) (the forward's Q and scale).
 *
 * litelinear_residual_quantize: the same for R = W - A B, computed on the
 * device in float32 (bf16 products, float32 sums) and never stored.
 *   W      bf16 [out, in] 16-byte aligned, in % 16 == 0.
 *   A      bf16 [out, r]  16-byte aligned, r % 8 == 0 (may be NULL iff r == 0).
 *   B      bf16 [r, in]   16-byte aligned (may be NULL iff r == 0).
 *   codes  uint8 [out, in] 16-byte aligned; scale_out as above.
 *
 * Both read their input twice (max |R|, then the codes) in two launches
 * queued on `stream`, and use one word of the handle's workspace per
 * work-group of the first (at most 4096 words for litelinear_quantize_tensor,
 * one per 128 x 128 tile of W for litelinear_residual_quantize), which the
 * handle grows as for litelinear_forward (so a captured call must follow an
 * uncaptured one of at least its size).  Outputs must not overlap the
 * inputs.  Errors: INVALID_ARG, UNSUPPORTED (alignment, the multiples above,
 * tensors of 2^31 bytes or more, workspace growth under capture), HIP, OOM.
 */
litelinear_status_t litelinear_quantize_tensor(litelinear_handle_t h, const float *R, int64_t n, void *codes,
                                               float *scale_out, hipStream_t stream);
litelinear_status_t litelinear_residual_quantize(litelinear_handle_t h, const void *W, const void *A, const void *B,
                                                 int64_t out, int64_t in, int64_t r, void *codes, float *scale_out,
                                                 hipStream_t stream);

/*
 * Two outputs that share x and B, and so T = x B^T (a gate/up pair; the
 * modegpt_compressor page's shared factors are the analogue on the other
 * side of the product):
 *     y1 = T A1^T + scale1 * (x dec(Q1)^T) + bias1      y1 [M, out1]
 *     y2 = T A2^T + scale2 * (x dec(Q2)^T) + bias2      y2 [M, out2]
 * Each output's tensors follow litelinear_forward's rules; the outputs must
 * not overlap each other or any input.  Large M runs one tiled launch that
 * computes T once for both; with M in the skinny regime (or out1 or out2 0)
 * it runs one forward per output.  Options as for litelinear_forward.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP, OOM.
 */
litelinear_status_t litelinear_forward_pair(litelinear_handle_t h, const void *x, const void *B, const void *A1,
                                            const void *Q1, float scale1, const void *bias1, void *y1, int64_t out1,
                                            const void *A2, const void *Q2, float scale2, const void *bias2, void *y2,
                                            int64_t out2, int64_t M, int64_t in, int64_t r, hipStream_t stream);

/* Frees the handle and its workspace (synchronising the device first).
 * NULL is accepted. */
litelinear_status_t litelinear_destroy(litelinear_handle_t h);

/* Host-only validation of litelinear_forward's arguments, with the same
 * result codes; touches no device (usable without a GPU).  y_bytes_per_elem
 * is 2 for bf16 output, 4 for float32 output. */
litelinear_status_t litelinear_check_args(const void *x, const void *A, const void *B,
                                          const void *Q, const void *bias, const void *y,
                                          int64_t M, int64_t in, int64_t out, int64_t r,
                                          int y_bytes_per_elem);

/* Set an option (litelinear_option_t).  Errors: INVALID_ARG for an unknown
 * key or value. */
litelinear_status_t litelinear_set_option(litelinear_handle_t h, int key, int64_t value);

/* Accumulated GPU time and launch count of one kernel kind since the last
 * reset, measured with HIP events while LITELINEAR_OPT_PROFILE is on.
 * Synchronises on the recorded events.  reset != 0 clears the totals. */
litelinear_status_t litelinear_kernel_time(litelinear_handle_t h, int kernel,
                                           double *total_ms, int64_t *launches, int reset);

/* LITELINEAR_ERR_SYNC if a bounded wait inside a launch on this handle has
 * given up since the last report (that launch's output is undefined), else
 * OK.  It reads the handle's error word without synchronising: synchronise
 * the stream first to cover every queued call.  Reporting clears the word,
 * and the next forward call first resets the handle's counters on its
 * stream.  Errors: INVALID_ARG (h == NULL). */
litelinear_status_t litelinear_device_status(litelinear_handle_t h);

/* Diagnostic, not part of the forward: the HBM read ceiling that the skinny
 * path (which streams Q once) is measured against.  Reads `bytes` (a
 * multiple of 16, src 16-byte aligned) of device memory once with
 * `work_groups` work-groups of 256 threads, each over one contiguous span,
 * `unroll` (4, 8 or 16) 16-byte loads in flight per lane, non-temporal when
 * `nontemporal` != 0; XORs one word per work-group into sink[0 ..
 * work_groups) (so the reads are not optimised away).  Queued on `stream`.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
litelinear_status_t litelinear_read_probe(litelinear_handle_t h, const void *src, int64_t bytes, int work_groups,
                                          int unroll, int nontemporal, unsigned *sink, hipStream_t stream);

/* Static text for a status code. */
const char *litelinear_status_string(litelinear_status_t s);

/* Version string of the library ("major.minor.patch"). */
const char *litelinear_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LITELINEAR_H */
