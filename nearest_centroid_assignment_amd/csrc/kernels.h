// kernels.h - internal launchers shared by the C-ABI layer (api.hip) and the
// kernel files. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace km {

// Rows of the stable counting sort handled by one block of the update.
constexpr int64_t kSortTileRows = 1024;

// Workspace sections used by the update (all device pointers, caller-owned).
struct UpdateScratch {
    int *tile_hist;  // k * n_tiles: per (cluster, row tile) counts, then their
                     // exclusive prefix over tiles
    int *cnt;        // k: rows per cluster
    int *seg_start;  // k: first position of each cluster in perm
    int *perm;       // n: row indices grouped by cluster, increasing within one
    int64_t n_tiles; // ceil(n / kSortTileRows)
};

// out[r] = sum_t A[r, t]^2 for r < rows (float64 accumulation, rounded once).
hipError_t launch_row_sqnorms(const float *A, int64_t rows, int64_t d, float *out,
                              hipStream_t stream);

// keys[i] = UINT64_MAX for i < n (the identity of the packed-key minimum).
hipError_t launch_fill_keys(unsigned long long *keys, int64_t n, hipStream_t stream);

// Fused Gram product + argmin epilogue: for every sample, atomically lowers
// keys[i] to the packed (distance', index) of its best centroid per tile.
hipError_t launch_assign_tiles(const float *X, const float *C, const float *cn, int64_t n,
                               int64_t k, int64_t d, unsigned long long *keys,
                               hipStream_t stream);

// Turns packed keys into int64 labels in place; if min_dist != NULL it holds
// ||x_i||^2 on entry and the clamped full squared distance on exit.
hipError_t launch_finalize(unsigned long long *keys, float *min_dist, int64_t n,
                           hipStream_t stream);

// The whole update: counts, stable grouping of rows by label, segmented sums
// in float64 and the mean (old centre kept for empty clusters).
hipError_t launch_update(const float *X, const int64_t *labels, const float *C_old, int64_t n,
                         int64_t k, int64_t d, float *C_new, int64_t *counts,
                         const UpdateScratch &ws, hipStream_t stream);

// Upper limits of the launch grids (blocks); checked by the C-ABI layer.
int64_t assign_grid_blocks(int64_t n, int64_t k);
int64_t update_grid_blocks(int64_t n, int64_t k, int64_t d);

}  // namespace km
