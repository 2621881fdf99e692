// Internal launch interface between the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ll {

// Tiled path: one launch whose first work-groups compute T' = x B^T / scale
// into a bf16 workspace [M, r_pad] and whose other work-groups each produce
// one output tile y = scale * (x dec(Q)^T + T' A^T) + bias.
struct TiledProblem {
    const void *x, *A, *B, *Q, *bias;
    void *y;
    void *t_ws;          // bf16 [M, r_pad]; unused when r == 0
    float *t_part;       // float32 [t_splits, M, r_pad] partial sums of T (t_splits > 1)
    float scale;
    int64_t M, K, N, r, r_pad;
    int64_t ldx;         // elements between rows of x (>= K, multiple of 8)
    int t_splits;        // K slices per T block (tiled_t_splits())
    int t_launch;        // K slices of T's launch of its own (tiled_t_launch()),
                         // 0: T producers inside the output tiles' launch
    unsigned *err;       // host-visible error word (a bounded wait gave up)
    unsigned wait_limit; // polls before a bounded wait gives up (> 0)
    unsigned wait_extra; // added to every wait's target: 0, or 1 to make the
                         // waits give up (a test of the error path)
    bool out_f32;
    bool gelu;           // GELU (tanh approximation) on y before its rounding, both outputs
    int q_format;        // Q codes: 0 e4m3fn, 1 e4m3fnuz (bf16 activations only)
    bool act8;           // the fp8-activation mode will run (xq, xs set before the launch)
    bool glu;            // gated epilogue: N = 2F rows of Q/A/bias (hidden then gate),
                         // y [M, F] = hidden * GELU_erf(gate); one output only
    // fp8-activation mode (both set, or both null): e4m3fn codes of x [M, K]
    // and the rows' scales 2^e [M] from launch_quant_rows; the residual
    // product reads these, T still reads x.
    const void *xq;
    const float *xs;
    // Optional second output sharing x and B (N2 > 0): its Q [N2, K], A
    // [N2, r], bias, scale and y [M, N2], and a second T' workspace.
    const void *Q2, *A2, *bias2;
    void *y2;
    void *t_ws2;
    float scale2;
    int64_t N2;
};

// x bf16 [M, K] with rows ldx elements apart (K % 8 == 0, ldx % 8 == 0) ->
// e4m3fn codes [M, K] and one power-of-two scale per row [M] (see quant.hip).
hipError_t launch_quant_rows(const void *x, int64_t ldx, void *codes, float *scales, int64_t M, int64_t K,
                             hipStream_t s);

// Decomposition side (convert.hip).  part: workspace of *_slots() words
// (one per work-group of the first pass), written before it is read in
// each call, so it needs no clearing.
int64_t quant_tensor_slots(int64_t n);
int64_t residual_quant_slots(int64_t N, int64_t K);
// float32 R [n] (n % 4 == 0) -> codes [n], *scale_out = max|R| / 448.
hipError_t launch_quant_tensor(const float *R, int64_t n, void *codes, unsigned *part, float *scale_out,
                               hipStream_t s);
// R = W - A B (W bf16 [N, K], A bf16 [N, r], B bf16 [r, K]; K % 16 == 0,
// r % 8 == 0) -> codes [N, K], *scale_out = max|R| / 448.
hipError_t launch_residual_quant(const void *W, const void *A, const void *B, int64_t N, int64_t K, int64_t r,
                                 void *codes, unsigned *part, float *scale_out, hipStream_t s);

// HBM read ceiling probe (probe.hip): reads bytes (a multiple of 16) of src
// once with `wgs` work-groups of 256 threads, `unroll` (4, 8 or 16) 16-byte
// loads in flight per lane, optionally non-temporal; XORs one word per
// work-group into sink[0 .. wgs).
hipError_t launch_read_probe(const void *src, int64_t bytes, int wgs, int unroll, bool nontemporal, unsigned *sink,
                             hipStream_t s);

// Fixed device scratch of litelinear_forward_noalloc (noalloc.hip): a
// file-scope device array of kScratchBytes per device.  scratch_init()
// returns its device address on `device`, which must be the current device;
// the address is looked up once per device and kept.
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr size_t kScratchSyncBytes = (size_t)64 << 10;  // counters at its start
hipError_t scratch_init(int device, void **ptr);

// Tile configuration of one launch (work-group tile BM x BN).
struct TileCfg {
    int bm, bn;
};

// True when the tiled path divides T by scale before rounding it, so that
// scale is applied in the epilogue (see tiled.hip).
bool scale_foldable(float scale);
TileCfg choose_main_tile(const TiledProblem &p);
// A's rows must be whole 16-byte chunks (r % 8 == 0, 16-byte aligned base);
// otherwise it is first copied into a zero-padded [N, r_pad] workspace.
bool a_needs_padding(int64_t r, const void *A);
bool tiled_shape_ok(const TiledProblem &p, TileCfg c);
int tiled_row_tiles(const TiledProblem &p, TileCfg c);
hipError_t launch_pad_a(const void *A, void *a_pad, int64_t N, int64_t r, int64_t r_pad, hipStream_t s);
// p[0 .. n) = v, queued on s as a kernel (never a memset node).
hipError_t launch_fill_u32(unsigned *p, int64_t n, unsigned v, hipStream_t s);
// K slices per block of T: T is computed by tiled_row_tiles() x (blocks per
// row tile: 2 of 128 rows for 256-row tiles with 64-column T blocks, else 1) x (r_pad /
// tiled_t_cols()) x t_splits producer work-groups, enough of them to finish
// early but few enough to leave most CUs to the output tiles.
// hint > 0 asks for that many slices (capped at the number of K steps).
int tiled_t_splits(const TiledProblem &p, TileCfg c, int64_t hint);
// T in a launch of its own, queued before the output tiles' launch, instead
// of producer work-groups inside it: for grids of fewer than four rounds
// whose last round has no free slots for the producers.  Needs 64-column T
// blocks, r_pad <= 128 and in <= 8192 (4096 for r_pad = 128).  Returns its
// K slices (t_part holds that many partial sums when more than one), or 0
// for in-launch producers.  hint: 0 = automatic, 1 = in-launch producers,
// 2 = a launch of its own wherever the shape allows it.
int tiled_t_launch(const TiledProblem &p, TileCfg c, int64_t hint);
// sync: tiled_sync_words() counters, zero before the launch and zero again
// after it: per row tile the T blocks finished (tiled_flag_step() of them
// complete the row tile's T) and the consumers done reading T' (the last one
// clears both), per T block the finished K slices (the last slice clears it).
// Covers both ways of computing T (p.t_launch).
int64_t tiled_sync_words(const TiledProblem &p, TileCfg c);
unsigned tiled_flag_step(const TiledProblem &p, TileCfg c);
// True when the output work-groups compute T themselves (no producers, no
// T workspace or counters): 128 x 128 tiles of tiny, latency-bound problems
// (tiled_tiny_shape(), which also sends such problems with M <= 64 to the
// tiled kernel when the path is chosen automatically).
bool tiled_tiny_shape(int64_t M, int64_t K, int64_t N, int64_t r);
bool tiled_self_t(const TiledProblem &p, TileCfg c);
// Columns of T per producer block (64, or 256 for ranks that are multiples
// of 256 with 256-wide output tiles).
int tiled_t_cols(const TiledProblem &p, TileCfg c);
hipError_t launch_tiled(const TiledProblem &p, TileCfg c, const void *a_eff, const void *a_eff2, unsigned *sync,
                        hipStream_t s);

// Skinny path (M <= 64): T producers plus output work-groups of 128
// columns over K slices (see skinny.hip).
struct SkinnyPlan {
    int mb;          // row blocks of 16 (1, 2 or 4)
    int k_slice;     // K elements per output work-group (512 .. 4096)
    int splits;      // K slices
    int tiles_n;     // column tiles
    int groups;      // 16-rank fragments of T (r_pad / 16)
    int t_kslice;    // K elements of a T piece
    int t_splits;    // K ranges of T pieces (over all slices)
    int pps;         // T pieces per K slice
    int pwg;         // work-groups per slice that compute pieces
    int producers;   // pwg * splits when r > 0: the pieces' work-groups
    int fullk;       // 1: all of K per 32-column work-group (skinny_fullk_kernel)
    int nq;          // fullk: ring stages per wave (K quarter = 256 nq)
};

struct SkinnyProblem {
    const void *x, *A, *B, *Q, *bias;
    void *y;
    float *partials;     // float32 [splits, M, N] (splits > 1)
    unsigned *sync;      // skinny_sync_words() counters, zero before the
                         // launch and left at zero by it
    unsigned long long *gen;  // plan.fullk and r > 0: 33 x 256 bytes of counters
                              // that only grow (zero when allocated)
    unsigned *err;       // host-visible error word (a bounded wait gave up)
    unsigned wait_limit; // polls before a bounded wait gives up (> 0)
    unsigned wait_extra; // added to the T wait's target (1: a test of the error path)
    float *t_part;       // T pieces, float32 [t_splits, M, r_pad] (r > 0)
    float scale;
    int64_t M, K, N, r, r_pad;
    int64_t ldx;         // elements between rows of x (>= K, multiple of 8)
    bool out_f32;
    bool gelu;           // GELU (tanh approximation) on y before its rounding
    int q_format;        // Q codes: 0 e4m3fn, 1 e4m3fnuz
    bool glu;            // gated epilogue: N = 2F (hidden, then gate), y [M, F]
    SkinnyPlan plan;
};

bool skinny_supports(int64_t M);  // row counts the skinny kernel takes
// splits_hint > 0 asks for about that many K slices.
// glu: N counts the rows of Q (hidden and gate).
SkinnyPlan skinny_plan(int64_t M, int64_t K, int64_t N, int64_t r_pad, int64_t splits_hint, bool glu);
int64_t skinny_sync_words(const SkinnyPlan &pl);
// ldx: elements between rows of x.
bool skinny_shape_ok(int64_t M, int64_t K, int64_t N, int64_t r_pad, const SkinnyPlan &pl, int64_t ldx);
// a_eff: A itself, or its zero-padded [N, r_pad] copy (see a_needs_padding).
hipError_t launch_skinny(const SkinnyProblem &p, const void *a_eff, hipStream_t s);

}  // namespace ll
