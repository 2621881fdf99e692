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
    int t_splits;        // K slices per T block (tiled_t_splits())
    bool out_f32;
};

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
// K slices per 64-column block of T: T is computed by tiled_row_tiles() x
// (r_pad / 64) x t_splits producer work-groups, enough of them to finish
// early but few enough to leave most CUs to the output tiles.
// hint > 0 asks for that many slices (capped at the number of K steps).
int tiled_t_splits(const TiledProblem &p, TileCfg c, int64_t hint);
// sync: tiled_sync_words() counters, zero before the launch and left at zero
// by it (per row tile: T blocks done, consumers past their wait; per T block:
// slices done).
int64_t tiled_sync_words(const TiledProblem &p, TileCfg c);
hipError_t launch_tiled(const TiledProblem &p, TileCfg c, const void *a_eff, unsigned *sync, hipStream_t s);

// Skinny path: split-K over `in`; every work-group computes its own slice of
// T, and the last work-group of each column tile sums the slices in order.
struct SkinnyProblem {
    const void *x, *A, *B, *Q, *bias;
    void *y;
    float *partials;     // float32 [splits, M, N] (used when splits > 1)
    unsigned *counters;  // one per column tile, zero between calls
    float scale;
    int64_t M, K, N, r, r_pad;
    int splits;          // number of K slices
    int64_t k_slice;     // elements of K per slice: 64 * skinny_slice_steps()
    bool out_f32;
};

int skinny_col_tile();                        // columns per work-group
bool skinny_supports(int64_t M, int64_t r_pad);  // shapes the skinny kernel takes
bool skinny_shape_ok(int64_t M, int64_t K, int64_t N, int64_t r_pad, int64_t splits);
// Steps of 64 per K slice (4, 8 or 16; the kernel unrolls them), aiming at
// about one work-group per CU, or at `splits_hint` slices when it is > 0.
int skinny_slice_steps(int64_t K, int64_t N, int64_t splits_hint);
// a_eff: A itself, or its zero-padded [N, r_pad] copy (see a_needs_padding).
hipError_t launch_skinny(const SkinnyProblem &p, const void *a_eff, hipStream_t s);

}  // namespace ll
