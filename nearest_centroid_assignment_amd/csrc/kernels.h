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
    int *tile_hist;          // n_tiles * k: [b * k + j] = rows of tile b with label j,
                             // then their exclusive prefix over tiles
    unsigned short *rank;    // n: rank of a row among the rows of its tile with the
                             // same label and a lower index
    int *cnt;                // k: rows per cluster
    int *seg_start;          // k: first position of each cluster in perm
    int *perm;               // n: row indices grouped by cluster, increasing within one
    int *big;                // k + 1: the number of clusters with more than the split
                             // size, then their indices in increasing order
    int *order;              // k: the other clusters, grouped by load rounds (most first)
    int *no_empty;           // 1: set by a count that reports empty clusters: 1 when
                             // there are none
    int64_t n_tiles;         // ceil(n / kSortTileRows)
};

// A kernel given a Gate returns at once, in every block, when either flag it
// points to is non-zero (NULL pointers count as zero). kmeans_fit gates the
// kernels of iterations enqueued after convergence, and the recount after a
// relocation that moved nothing.
struct Gate {
    const int *a = nullptr;
    const int *b = nullptr;
};

__device__ __forceinline__ bool gated(const Gate &g) {
    return (g.a != nullptr && *g.a != 0) || (g.b != nullptr && *g.b != 0);
}

// Inverse of the assignment's order-preserving map of a float to 32 bits
// (the distance half of a packed key).
__device__ __forceinline__ float key_distance(unsigned long long key) {
    const uint32_t u = (uint32_t)(key >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// out[r] = sum_t A[r, t]^2 for r < rows (float64 accumulation, rounded once).
hipError_t launch_row_sqnorms(const float *A, int64_t rows, int64_t d, float *out,
                              hipStream_t stream, Gate gate = Gate{});

// keys[i] = UINT64_MAX for i < n (the identity of the packed-key minimum).
hipError_t launch_fill_keys(unsigned long long *keys, int64_t n, hipStream_t stream,
                            Gate gate = Gate{});

// Fused Gram product + argmin epilogue: for every sample, atomically lowers
// keys[i] to the packed (distance', index) of its best centroid per tile,
// or, at k <= 64 (one pass over all centroids), stores it outright.
// With stop != NULL every block returns at once if *stop is non-zero.
hipError_t launch_assign_tiles(const float *X, const float *C, const float *cn, int64_t n,
                               int64_t k, int64_t d, unsigned long long *keys,
                               hipStream_t stream, const int *stop = nullptr);

// Whether launch_assign_tiles with these arguments stores every sample's key
// outright (then the identity fill before it is not needed).
bool assign_stores_keys(const float *X, const float *C, int64_t n, int64_t k, int64_t d);

// Turns packed keys into int64 labels in place. min_dist (nullable): with
// add_norm it holds ||x_i||^2 on entry and the clamped full squared distance
// on exit; without, it receives the best ||c||^2 - 2 x.c, to which
// launch_add_norms later adds the norms gathered by the update.
hipError_t launch_finalize(unsigned long long *keys, float *min_dist, bool add_norm, int64_t n,
                           int64_t k, hipStream_t stream);

// Clusters of more rows than this are summed in parts by the mean kernel;
// smaller ones by one wave in sample order: 64, or 128 when X has at least
// 2^26 elements and clusters average 32 rows or more (then clusters of 65 to
// 128 rows are common, and a wave summing one alone is still far from the
// critical path, while the split's per-part barrier and merge are not).
int split_rows(int64_t n, int64_t k, int64_t d);

// Counting phase of the update, first step, on labels: per tile of
// kSortTileRows rows, the histogram column tile_hist[b * k + .] and the
// stable ranks of the rows. Rows with a label outside [0, k) are skipped.
hipError_t launch_rank_hist(const int64_t *labels, int64_t n, int64_t k, const UpdateScratch &ws,
                            Gate gate, hipStream_t stream);

// The same step fused with the assignment's finalize: packed keys become int64
// labels in place (and min_dist as in launch_finalize), then the histogram
// and the ranks of those labels.
hipError_t launch_finalize_rank_hist(unsigned long long *keys, float *min_dist, bool add_norm,
                                     int64_t n, int64_t k, const UpdateScratch &ws, Gate gate,
                                     hipStream_t stream);

// Counting phase, second step (after one of the two above, on the same
// labels): per-cluster sizes (ws.cnt, counts), segment starts, the tiles'
// prefixes, and the split of the clusters by split_rows(n, k, d); num_empty
// (nullable) receives the number of empty clusters and ws.no_empty whether
// there are none. For k <= 1024 and n <= 64 * kSortTileRows it also groups
// the rows (ws.perm), which launch_group_and_mean then leaves as it is.
hipError_t launch_scan(const int64_t *labels, int64_t n, int64_t k, int64_t d, int64_t *counts,
                       int *num_empty, const UpdateScratch &ws, Gate gate, hipStream_t stream);

// Both steps on labels.
hipError_t launch_count(const int64_t *labels, int64_t n, int64_t k, int64_t d, int64_t *counts,
                        int *num_empty, const UpdateScratch &ws, Gate gate, hipStream_t stream);

// Second phase: stable grouping of rows by label and the float64 segmented
// sums and means (old centre kept for an empty cluster). If shift_partial is
// not NULL, mean_blocks(k, d) partial sums of (new - old)^2 are written there.
// If xn_part is not NULL (only when every label lies in [0, k), so that every
// row is grouped), it receives norm_parts(d) x n float32 partial squared
// norms of the rows, in grouped order: [c * n + p] is chunk c of row
// ws.perm[p]. shift_partial and xn_part are not both set.
// mean_blocks counts the blocks of both mean kernels (small and big clusters).
hipError_t launch_group_and_mean(const float *X, const int64_t *labels, const float *C_old,
                                 int64_t n, int64_t k, int64_t d, float *C_new,
                                 double *shift_partial, float *xn_part, const UpdateScratch &ws,
                                 Gate gate, hipStream_t stream);
int64_t mean_blocks(int64_t k, int64_t d);
// Column chunks of the mean kernel: partial norms per row.
int64_t norm_parts(int64_t d);

// The whole update: counts, stable grouping of rows by label, segmented sums
// in float64 and the mean (old centre kept for empty clusters); xn_part as in
// launch_group_and_mean. With counted = true the first counting step has
// already run (launch_finalize_rank_hist on these labels).
hipError_t launch_update(const float *X, const int64_t *labels, const float *C_old, int64_t n,
                         int64_t k, int64_t d, float *C_new, int64_t *counts, float *xn_part,
                         bool counted, const UpdateScratch &ws, hipStream_t stream);

// min_dist[i] = max(0, ||x_i||^2 + min_dist[i]), ||x_i||^2 the float64 sum of
// the row's partial norms from the update (xn_part and the grouping ws.perm
// of that update), rounded once to float32.
hipError_t launch_add_norms(float *min_dist, const float *xn_part, int64_t n, int64_t d,
                            const UpdateScratch &ws, hipStream_t stream);

// Workspace sections of the empty-cluster relocation (device pointers).
struct RelocScratch {
    double *dist;                  // n: float64 distance of each sample to its centre
    int *empty;                    // k: empty clusters in increasing index
    unsigned long long *sort_key;  // reloc_sort_cap(n, k)
    int *sort_idx;                 // reloc_sort_cap(n, k)
    int *num_empty;                // 1: empty clusters after the assignment
};

// Size of the relocation sort buffers: the power of two >= min(n, k).
int64_t reloc_sort_cap(int64_t n, int64_t k);

// Relocation of the clusters left empty by the assignment (counts already
// taken into ws.cnt with num_empty set): relabels the moved samples.
hipError_t launch_relocate(const float *X, const float *C_old, int64_t *labels, int64_t n,
                           int64_t k, int64_t d, const RelocScratch &rs, const UpdateScratch &ws,
                           hipStream_t stream, Gate gate = Gate{});

// Unless *converged is already set (then nothing happens): shift_out = sum of
// the first `blocks` partials (fixed order); converged = (shift_out <= tol);
// ++*iterations.
hipError_t launch_shift(const double *partial, int64_t blocks, double tol, double *shift_out,
                        int *converged, int *iterations, hipStream_t stream);

// p[0 .. count) = 0 (a kernel, so that the call can be captured in a graph).
hipError_t launch_zero_i32(int *p, int64_t count, hipStream_t stream);

// *dst = (double)*count.
hipError_t launch_store_count(double *dst, const int *count, hipStream_t stream);

// out = sum of min_dist[0 .. n) in float64 (fixed order).
hipError_t launch_inertia(const float *min_dist, int64_t n, double *out, hipStream_t stream);

hipError_t launch_copy_f32(float *dst, const float *src, int64_t count, hipStream_t stream);

// Workspace sections of the k-means++ seeding (device pointers).
struct PPScratch {
    double *buf_a, *buf_b;      // trials * n: D of each candidate (alternating)
    double *parts_a, *parts_b;  // trials * pp_blocks(n): per-block sums of those
    int64_t *cand_a, *cand_b;   // trials: candidate sample indices (alternating)
    void *state;                // pp_state_bytes(): winner and its potential
    double *xnorm;              // n: |x_i|^2 in float64
};
int64_t pp_blocks(int64_t n);
int pp_max_trials();
int pp_block_threads();  // threads per block of the distance kernel
size_t pp_state_bytes();

// Greedy k-means++ seeding: chosen[0] = first, then k - 1 centres drawn with
// rand ((k - 1) * trials uniforms); centres[c] = X[chosen[c]].
hipError_t launch_kmeanspp(const float *X, int64_t n, int64_t d, int64_t k, int64_t first,
                           int trials, const double *rand, float *centres, int64_t *chosen,
                           const PPScratch &ws, hipStream_t stream);

// Largest launch grids, in work-items; checked by the C-ABI layer against the
// 2^32 - 1 limit of one dispatch dimension.
// The assignment launch (the tile the launcher will choose).
int64_t assign_grid_threads(int64_t n, int64_t k, int64_t d);
// The largest launch of the update (count, group, mean).
int64_t update_grid_threads(int64_t n, int64_t k, int64_t d);

}  // namespace km
