// update.hip - Lloyd centroid update on gfx950.
//
// The update of "Three shapes that fit an eager Gram assignment", section Full
// Lloyd step, is a one-hot (n, k) membership matrix times X; the Cython kernel
// of "004 - tile sizes ...", section Cython reference, scatters each sample
// into per-thread centre buffers instead. Here the samples are first grouped
// by label with a stable counting sort, then every (cluster, column chunk)
// block adds its cluster's rows in increasing sample order:
//
//   tile_hist_kernel     counts per (cluster, tile of 1024 rows)
//   tile_scan_kernel     exclusive prefix over tiles, per cluster; cluster sizes
//   cluster_scan_kernel  exclusive prefix over clusters -> segment starts; counts
//   scatter_kernel       perm[segment start + rows of the cluster in earlier
//                        tiles + rank within the tile] = row   (stable)
//   segment_mean_kernel  float64 sums over each segment, coalesced row chunks,
//                        then the mean rounded once to float32, or the old
//                        centre for an empty cluster
//
// No float atomics: every sum has one fixed order, so results are
// deterministic, and the float64 sum in increasing sample order followed by a
// float64 divide is exactly the plain definition of the mean.
#include "kernels.h"

namespace km {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = (int)kSortTileRows;  // rows per sort tile
constexpr int kChunk = 1024;               // columns per segment_mean block (256 x 4)

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

__global__ __launch_bounds__(256) void fill_i32_kernel(int *__restrict__ p, int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
        p[i] = 0;
}

// One block per tile of kTile rows. Rows with a label outside [0, k) are skipped.
__global__ __launch_bounds__(256) void tile_hist_kernel(const int64_t *__restrict__ labels,
                                                        int64_t n, int64_t k, int64_t n_tiles,
                                                        int *__restrict__ tile_hist) {
    const int64_t b = blockIdx.x;
#pragma unroll
    for (int q = 0; q < kTile / 256; ++q) {
        const int64_t i = b * kTile + q * 256 + threadIdx.x;
        if (i < n) {
            const int64_t l = labels[i];
            if (l >= 0 && l < k) atomicAdd(tile_hist + l * n_tiles + b, 1);
        }
    }
}

// One wave per cluster: exclusive scan of its n_tiles counters, in place.
__global__ __launch_bounds__(256) void tile_scan_kernel(int *__restrict__ tile_hist, int64_t k,
                                                        int64_t n_tiles, int *__restrict__ cnt) {
    const int lane = threadIdx.x & 63;
    const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (j >= k) return;
    int *h = tile_hist + j * n_tiles;
    int carry = 0;
    for (int64_t base = 0; base < n_tiles; base += 64) {
        const int64_t t = base + lane;
        const int v = t < n_tiles ? h[t] : 0;
        int incl = v;
        for (int off = 1; off < 64; off <<= 1) {
            const int up = __shfl_up(incl, off);
            if (lane >= off) incl += up;
        }
        if (t < n_tiles) h[t] = carry + incl - v;
        carry += __shfl(incl, 63);
    }
    if (lane == 0) cnt[j] = carry;
}

// A single block of 1024 threads: exclusive scan over the k cluster sizes.
__global__ __launch_bounds__(1024) void cluster_scan_kernel(const int *__restrict__ cnt, int64_t k,
                                                            int *__restrict__ seg_start,
                                                            int64_t *__restrict__ counts) {
    __shared__ int wave_tot[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int carry = 0;
    for (int64_t base = 0; base < k; base += 1024) {
        const int64_t j = base + tid;
        const int v = j < k ? cnt[j] : 0;
        int incl = v;
        for (int off = 1; off < 64; off <<= 1) {
            const int up = __shfl_up(incl, off);
            if (lane >= off) incl += up;
        }
        if (lane == 63) wave_tot[wave] = incl;
        __syncthreads();
        int before = 0, total = 0;
        for (int w = 0; w < 16; ++w) {
            const int wt = wave_tot[w];
            before += w < wave ? wt : 0;
            total += wt;
        }
        if (j < k) {
            seg_start[j] = carry + before + incl - v;
            counts[j] = v;
        }
        carry += total;
        __syncthreads();  // wave_tot is rewritten by the next chunk
    }
}

// One block per tile. The rank of a row among the rows of the same tile with
// the same label and a smaller index is counted directly from the tile's
// labels in LDS, which keeps the grouping stable (increasing row order inside
// every cluster) and independent of thread timing.
__global__ __launch_bounds__(256) void scatter_kernel(const int64_t *__restrict__ labels, int64_t n,
                                                      int64_t k, int64_t n_tiles,
                                                      const int *__restrict__ tile_prefix,
                                                      const int *__restrict__ seg_start,
                                                      int *__restrict__ perm) {
    __shared__ int lab[kTile];
    const int64_t b = blockIdx.x;
    const int64_t row0 = b * kTile;
    const int rows = (int)min((int64_t)kTile, n - row0);
    for (int r = threadIdx.x; r < kTile; r += 256) {
        int l = -1;
        if (r < rows) {
            const int64_t v = labels[row0 + r];
            l = (v >= 0 && v < k) ? (int)v : -1;
        }
        lab[r] = l;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < rows; r += 256) {
        const int l = lab[r];
        if (l < 0) continue;
        int rank = 0;
        for (int q = 0; q < r; ++q) rank += lab[q] == l;
        const int64_t pos = (int64_t)seg_start[l] + tile_prefix[(int64_t)l * n_tiles + b] + rank;
        perm[pos] = (int)(row0 + r);
    }
}

// Block (cluster j, column chunk c); thread t owns 4 columns. The segment's
// rows are added in increasing sample order in float64.
template <bool kVec>
__global__ __launch_bounds__(256) void segment_mean_kernel(
    const float *__restrict__ X, const int *__restrict__ perm, const int *__restrict__ seg_start,
    const int *__restrict__ cnt, const float *C_old, int64_t k, int64_t d, int64_t chunks,
    float *C_new) {
    // C_old and C_new may be the same array: each element is read and written
    // by the same thread only, so they carry no __restrict__.
    const int64_t j = blockIdx.x / chunks;
    const int64_t c = blockIdx.x % chunks;
    const int64_t count = cnt[j];
    const int64_t start = seg_start[j];
    int64_t col[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        col[e] = kVec ? c * kChunk + 4 * threadIdx.x + e : c * kChunk + threadIdx.x + 256 * e;
    double s[4] = {0.0, 0.0, 0.0, 0.0};
    if (kVec) {
        if (col[0] < d) {
#pragma unroll 4
            for (int64_t p = 0; p < count; ++p) {
                const int64_t i = perm[start + p];
                const f32x4 v = *reinterpret_cast<const f32x4 *>(X + i * d + col[0]);
                s[0] += (double)v.x;
                s[1] += (double)v.y;
                s[2] += (double)v.z;
                s[3] += (double)v.w;
            }
        }
    } else {
#pragma unroll 4
        for (int64_t p = 0; p < count; ++p) {
            const int64_t i = perm[start + p];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (col[e] < d) s[e] += (double)X[i * d + col[e]];
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (col[e] < d) {
            const int64_t o = j * d + col[e];
            C_new[o] = count > 0 ? (float)(s[e] / (double)count) : C_old[o];
        }
    }
}

inline unsigned grid_stride_blocks(int64_t n) {
    int64_t b = cdiv(n, 256);
    if (b > 4096) b = 4096;
    if (b < 1) b = 1;
    return (unsigned)b;
}

}  // namespace

int64_t update_grid_blocks(int64_t n, int64_t k, int64_t d) {
    const int64_t a = k * cdiv(d, kChunk);
    const int64_t b = cdiv(n, kTile);
    const int64_t c = cdiv(k, 4);
    return a > b ? (a > c ? a : c) : (b > c ? b : c);
}

hipError_t launch_update(const float *X, const int64_t *labels, const float *C_old, int64_t n,
                         int64_t k, int64_t d, float *C_new, int64_t *counts,
                         const UpdateScratch &ws, hipStream_t stream) {
    const int64_t hist_words = k * ws.n_tiles;
    if (hist_words > 0) {
        fill_i32_kernel<<<grid_stride_blocks(hist_words), 256, 0, stream>>>(ws.tile_hist,
                                                                           hist_words);
        if (n > 0)
            tile_hist_kernel<<<(unsigned)ws.n_tiles, 256, 0, stream>>>(labels, n, k, ws.n_tiles,
                                                                       ws.tile_hist);
        tile_scan_kernel<<<(unsigned)cdiv(k, 4), 256, 0, stream>>>(ws.tile_hist, k, ws.n_tiles,
                                                                   ws.cnt);
    } else {
        // n == 0: every cluster is empty.
        fill_i32_kernel<<<grid_stride_blocks(k), 256, 0, stream>>>(ws.cnt, k);
    }
    cluster_scan_kernel<<<1, 1024, 0, stream>>>(ws.cnt, k, ws.seg_start, counts);
    if (n > 0)
        scatter_kernel<<<(unsigned)ws.n_tiles, 256, 0, stream>>>(labels, n, k, ws.n_tiles,
                                                                 ws.tile_hist, ws.seg_start,
                                                                 ws.perm);
    const int64_t chunks = cdiv(d, kChunk);
    const unsigned blocks = (unsigned)(k * chunks);
    const bool vec = (d % 4 == 0) && ((uintptr_t)X % 16 == 0) && ((uintptr_t)C_old % 16 == 0) &&
                     ((uintptr_t)C_new % 16 == 0);
    if (vec)
        segment_mean_kernel<true><<<blocks, 256, 0, stream>>>(X, ws.perm, ws.seg_start, ws.cnt,
                                                              C_old, k, d, chunks, C_new);
    else
        segment_mean_kernel<false><<<blocks, 256, 0, stream>>>(X, ws.perm, ws.seg_start, ws.cnt,
                                                               C_old, k, d, chunks, C_new);
    return hipGetLastError();
}

}  // namespace km
