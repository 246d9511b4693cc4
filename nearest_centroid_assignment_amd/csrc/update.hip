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
//                        centre for an empty cluster: a wave per cluster of at
//                        most 64 rows, sixteen waves per larger one; in a
//                        Lloyd step also the rows' partial squared norms
//   add_norms_kernel     min_dist = max(0, ||x||^2 + best ||c||^2 - 2 x.c)
//                        from those partial norms
//
// No float atomics: every sum has one fixed order, so results are
// deterministic. For a cluster of at most 64 rows that order is increasing
// sample order, so the float64 sum and divide are exactly the plain definition
// of the mean; larger clusters add sixteen contiguous parts of their rows.
#include "kernels.h"

namespace km {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = (int)kSortTileRows;  // rows per sort tile
constexpr int kCols = 256;                 // columns per segment_mean block (64 lanes x 4)
constexpr int kSplitSmall = 64;            // larger clusters are split in kBigWaves parts ...
constexpr int kSplitLarge = 128;           // ... or larger than this, on big inputs
constexpr int kBigWaves = 16;              // waves (parts) per big-cluster block
constexpr int kBigBlocks = 256;            // segment_mean blocks that take the large clusters

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

__global__ __launch_bounds__(256) void fill_i32_kernel(int *__restrict__ p, int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
        p[i] = 0;
}

// kParts blocks of 256 threads per tile of kTile rows, one row per thread
// (one block per tile left most CUs idle). Rows with a label outside [0, k)
// are skipped.
constexpr int kParts = kTile / 256;
__global__ __launch_bounds__(256) void tile_hist_kernel(const int64_t *__restrict__ labels,
                                                        int64_t n, int64_t k, int64_t n_tiles,
                                                        int *__restrict__ tile_hist) {
    const int64_t b = blockIdx.x / kParts;
    const int64_t i = b * kTile + (blockIdx.x % kParts) * 256 + threadIdx.x;
    if (i < n) {
        const int64_t l = labels[i];
        if (l >= 0 && l < k) atomicAdd(tile_hist + l * n_tiles + b, 1);
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

// Load-round classes of the clusters summed by one wave (at most kSplit
// rows): class ceil(count / 8), 0 .. kSplit / 8.
template <int kSplit>
__device__ __forceinline__ int round_class(int count) {
    return count <= kSplit ? (count + 7) / 8 : -1;
}

// A single block of 1024 threads: exclusive scan over the k cluster sizes.
// If num_empty != NULL it receives the number of clusters of size 0. big[0]
// receives the number of clusters with more than kSplit rows and big[1 ..]
// their indices in increasing order. order[0 .. k - big[0]) receives the
// other clusters grouped by load-round class, most rounds first, increasing
// index within a class (a stable partition: every rank comes from ballots, so
// the order is the same on every run). The mean kernel gives 16 consecutive
// entries of `order` to one block, so a block's waves run the same number of
// load rounds instead of all waiting for the block's largest cluster.
template <int kSplit>
__global__ __launch_bounds__(1024) void cluster_scan_kernel(const int *__restrict__ cnt, int64_t k,
                                                            int *__restrict__ seg_start,
                                                            int64_t *__restrict__ counts,
                                                            int *__restrict__ num_empty,
                                                            int *__restrict__ big,
                                                            int *__restrict__ order) {
    constexpr int kClasses = kSplit / 8 + 1;
    __shared__ int wave_tot[16];
    __shared__ int wave_big[16];
    __shared__ int wave_empty[16];
    __shared__ int wave_cls[16][kClasses];
    __shared__ int cls_next[kClasses];  // next free slot of each class in order
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const unsigned long long below = (1ull << lane) - 1ull;
    int carry = 0, empties = 0, big_carry = 0;
    int cls_total = 0;  // thread c < kClasses: clusters of class c so far
    for (int64_t base = 0; base < k; base += 1024) {
        const int64_t j = base + tid;
        const int v = j < k ? cnt[j] : 0;
        empties += (j < k && v == 0);
        int incl = v;
        for (int off = 1; off < 64; off <<= 1) {
            const int up = __shfl_up(incl, off);
            if (lane >= off) incl += up;
        }
        const bool is_big = j < k && v > kSplit;
        const unsigned long long bm = __ballot(is_big);
        const int cls = j < k ? round_class<kSplit>(v) : -1;
        if (lane == 63) wave_tot[wave] = incl;
        if (lane == 0) wave_big[wave] = __popcll(bm);
#pragma unroll
        for (int c = 0; c < kClasses; ++c) {
            const unsigned long long cm = __ballot(cls == c);
            if (lane == 0) wave_cls[wave][c] = __popcll(cm);
        }
        __syncthreads();
        int before = 0, total = 0, big_before = 0, big_total = 0;
        for (int w = 0; w < 16; ++w) {
            const int wt = wave_tot[w], wb = wave_big[w];
            before += w < wave ? wt : 0;
            total += wt;
            big_before += w < wave ? wb : 0;
            big_total += wb;
        }
        if (tid < kClasses)
            for (int w = 0; w < 16; ++w) cls_total += wave_cls[w][tid];
        if (j < k) {
            seg_start[j] = carry + before + incl - v;
            counts[j] = v;
        }
        if (is_big) big[1 + big_carry + big_before + __popcll(bm & below)] = (int)j;
        carry += total;
        big_carry += big_total;
        __syncthreads();  // wave_tot, wave_big and wave_cls are rewritten by the next chunk
    }
    // Class c starts after every class with more rounds.
    if (tid < kClasses) wave_cls[0][tid] = cls_total;
    __syncthreads();
    if (tid < kClasses) {
        int start = 0;
        for (int c = kClasses - 1; c > tid; --c) start += wave_cls[0][c];
        cls_next[tid] = start;
    }
    __syncthreads();
    for (int64_t base = 0; base < k; base += 1024) {
        const int64_t j = base + tid;
        const int cls = j < k ? round_class<kSplit>(cnt[j]) : -1;
        int rank = 0;
#pragma unroll
        for (int c = 0; c < kClasses; ++c) {
            const unsigned long long cm = __ballot(cls == c);
            if (cls == c) rank = __popcll(cm & below);
            if (lane == 0) wave_cls[wave][c] = __popcll(cm);
        }
        __syncthreads();
        if (cls >= 0) {
            int pos = cls_next[cls] + rank;
            for (int w = 0; w < wave; ++w) pos += wave_cls[w][cls];
            order[pos] = (int)j;
        }
        __syncthreads();  // every thread has read cls_next and wave_cls
        if (tid < kClasses) {
            int t = 0;
            for (int w = 0; w < 16; ++w) t += wave_cls[w][tid];
            cls_next[tid] += t;
        }
        __syncthreads();
    }
    if (tid == 0) big[0] = big_carry;
    if (num_empty) {
        for (int off = 32; off > 0; off >>= 1) empties += __shfl_xor(empties, off);
        if (lane == 0) wave_empty[wave] = empties;
        __syncthreads();
        if (tid == 0) {
            int t = 0;
            for (int w = 0; w < 16; ++w) t += wave_empty[w];
            *num_empty = t;
        }
    }
}

// kParts blocks of 256 threads per tile, one thread per row: part p takes
// rows 256p .. 256p + 255 of the tile and loads the tile's labels up to its
// last row into LDS. The rank of a row among the rows of the same tile with
// the same label and a smaller index is counted directly from those labels,
// which keeps the grouping stable (increasing row order inside every
// cluster) and independent of thread timing. A wave first counts over the
// whole chunks of 64 rows before its own, four labels per (broadcast) LDS
// read with no divergence, then over the earlier rows of its own chunk.
// (One 1024-thread block per tile used a quarter of the CUs at n = 65536.)
static_assert(kTile == 1024 && kParts == 4, "scatter_kernel splits 1024-row tiles in 4 parts");
__global__ __launch_bounds__(256) void scatter_kernel(const int64_t *__restrict__ labels, int64_t n,
                                                      int64_t k, int64_t n_tiles,
                                                      const int *__restrict__ tile_prefix,
                                                      const int *__restrict__ seg_start,
                                                      int *__restrict__ perm) {
    __shared__ __align__(16) int lab[kTile];
    const int64_t b = blockIdx.x / kParts;
    const int part = blockIdx.x % kParts;
    const int64_t row0 = b * kTile;
    const int rows = (int)min((int64_t)kTile, n - row0);
    for (int q = threadIdx.x; q < (part + 1) * 256; q += 256) {
        int l = -1;
        if (q < rows) {
            const int64_t v = labels[row0 + q];
            l = (v >= 0 && v < k) ? (int)v : -1;
        }
        lab[q] = l;
    }
    __syncthreads();
    const int r = part * 256 + threadIdx.x;
    const int l = lab[r];
    if (l < 0) return;
    const int chunk0 = r & ~63;
    const int4 *lab4 = reinterpret_cast<const int4 *>(lab);
    int rank = 0;
    for (int q = 0; q < chunk0; q += 4) {
        const int4 v = lab4[q >> 2];
        rank += (v.x == l) + (v.y == l) + (v.z == l) + (v.w == l);
    }
    for (int q = chunk0; q < r; ++q) rank += lab[q] == l;
    const int64_t pos = (int64_t)seg_start[l] + tile_prefix[(int64_t)l * n_tiles + b] + rank;
    perm[pos] = (int)(row0 + r);
}

// Sum over the 64 lanes of a wave of each of B per-lane values (B a power of
// two, at most 64), in a fixed tree order. Each level halves the list: a lane
// keeps one half and adds the partner's copy of it (lanes O apart), so
// B - 1 + log2(64 / B) exchanges give every lane one full sum; `row` says
// which of the B it is. The lanes holding the same row differ only in their
// low 6 - log2(B) bits. Written as a compile-time recursion so that every
// index into q is a constant (q stays in registers).
template <int CNT, int O, int B>
__device__ __forceinline__ void halve_rows(float (&q)[B], int lane, int &row) {
    if constexpr (CNT > 1) {
        constexpr int half = CNT / 2;
        const bool up = (lane & O) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float send = up ? q[i] : q[i + half];
            const float keep = up ? q[i + half] : q[i];
            q[i] = keep + __shfl_xor(send, O);
        }
        if (up) row += half;
        halve_rows<half, O / 2, B>(q, lane, row);
    } else {
#pragma unroll
        for (int o = O; o > 0; o >>= 1) q[0] += __shfl_xor(q[0], o);
    }
}

template <int B>
__device__ __forceinline__ float wave_sum_rows(float (&q)[B], int lane, int &row) {
    row = 0;
    halve_rows<B, 32, B>(q, lane, row);
    return q[0];
}

// Squared norms of one round's rows over this chunk (q, one value per row
// and lane): a fixed-order float32 sum over the wave; value u (u < m) is
// written by one lane to xn[u]. The m values of a round sit side by side.
template <int B>
__device__ __forceinline__ void flush_norms(float (&q)[B], int m, int lane, float *xn) {
    int u;
    const float t = wave_sum_rows<B>(q, lane, u);
    // One writer per row: the lane of its group whose low bits are 0.
    if ((lane & (64 / B - 1)) == 0 && u < m) xn[u] = t;
}

// Rows are fetched in rounds of kBatch: all the round's row loads, then the
// adds in order. kBatch is 16, or 8 when clusters hold 32 rows or fewer on
// average (measured faster there: fewer load slots of a round go unused on
// short clusters, and the kernel needs about 66 registers instead of about
// 100). The order of the adds does not depend on kBatch.
//
// With kNorm (xn != NULL) the same loads also give each row's squared norm
// over this chunk's columns: per lane a float32 fused multiply-add chain over
// its (up to) 4 squares, then a fixed-order float32 sum over the wave (all
// terms are non-negative, so the relative error stays below 9 * 2^-24, about
// 5.4e-7), written to xn[p] for the p-th row of `rows`: the norms follow the
// grouped order, so a wave's writes are contiguous. Float32 keeps the loaded
// values from being held twice (as float and as the float64 the sums take).
// A round's cross-lane sums run after the next round's loads are issued, so
// their exchange latency overlaps the loads.
template <bool kVec, int kBatch, bool kNorm>
__device__ __forceinline__ void sum_rows(const float *__restrict__ X, const int *__restrict__ rows,
                                         int r0, int r1, int64_t d, const int64_t (&col)[4],
                                         double (&s)[4], float *__restrict__ xn) {
    constexpr int B = kVec ? kBatch : kBatch / 2;  // rows per round (the scalar path holds 4x)
    static_assert((B & (B - 1)) == 0 && B <= 64, "rows per round must be a power of two");
    const int lane = threadIdx.x & 63;
    float qp[B];   // the previous round's per-lane squared norms (kNorm)
    int pp = 0;    // its first row
    int mp = 0;    // its row count (0: nothing pending)
    // Row indices come 64 at a time, one per lane (rows[c0 + lane]), the
    // next 64 loaded a chunk ahead; a round takes its own with readlane, so
    // its row loads do not wait for an index load.
    int c0 = r0;
    int idx = r0 + lane < r1 ? rows[r0 + lane] : 0;
    int idx_next = r0 + 64 + lane < r1 ? rows[r0 + 64 + lane] : 0;
    for (int p0 = r0; p0 < r1; p0 += B) {
        if (p0 - c0 == 64) {
            c0 = p0;
            idx = idx_next;
            idx_next = p0 + 64 + lane < r1 ? rows[p0 + 64 + lane] : 0;
        }
        const int m = min(B, r1 - p0);
        int64_t base[B];
#pragma unroll
        for (int u = 0; u < B; ++u)
            base[u] = u < m ? (int64_t)__builtin_amdgcn_readlane(idx, p0 - c0 + u) * d : -1;
        if (kVec) {
            f32x4 v[B];
#pragma unroll
            for (int u = 0; u < B; ++u)
                v[u] = (base[u] >= 0 && col[0] < d)
                           ? *reinterpret_cast<const f32x4 *>(X + base[u] + col[0])
                           : f32x4{0.f, 0.f, 0.f, 0.f};
            if (kNorm && mp > 0) flush_norms<B>(qp, mp, lane, xn + pp);
#pragma unroll
            for (int u = 0; u < B; ++u) {
                if (u < m) {
                    s[0] += (double)v[u].x;
                    s[1] += (double)v[u].y;
                    s[2] += (double)v[u].z;
                    s[3] += (double)v[u].w;
                }
                if (kNorm)
                    qp[u] = fmaf(v[u].w, v[u].w,
                                 fmaf(v[u].z, v[u].z, fmaf(v[u].y, v[u].y, v[u].x * v[u].x)));
            }
        } else {
            float v[B][4];
#pragma unroll
            for (int u = 0; u < B; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[u][e] = (base[u] >= 0 && col[e] < d) ? X[base[u] + col[e]] : 0.f;
            if (kNorm && mp > 0) flush_norms<B>(qp, mp, lane, xn + pp);
#pragma unroll
            for (int u = 0; u < B; ++u) {
                if (u < m)
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[e] += (double)v[u][e];
                if (kNorm)
                    qp[u] = fmaf(v[u][3], v[u][3],
                                 fmaf(v[u][2], v[u][2], fmaf(v[u][1], v[u][1], v[u][0] * v[u][0])));
            }
        }
        pp = p0;
        mp = m;
    }
    if (kNorm && mp > 0) flush_norms<B>(qp, mp, lane, xn + pp);
}

// Writes the new centre elements of this thread and, if kShift, adds their
// squared move (new - old)^2 to `shift` (the old value is read before the new
// one is written, so C_new may be C_old). Without kShift the old centre is
// read only for an empty cluster.
template <bool kShift>
__device__ __forceinline__ void write_mean(const float *C_old, float *C_new, int64_t j, int64_t d,
                                           int count, const int64_t (&col)[4],
                                           const double (&s)[4], double &shift) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (col[e] < d) {
            const int64_t o = j * d + col[e];
            if (kShift || count == 0) {
                const float old = C_old[o];
                const float v = count > 0 ? (float)(s[e] / (double)count) : old;
                C_new[o] = v;
                const double diff = (double)v - (double)old;
                shift += diff * diff;
            } else {
                C_new[o] = (float)(s[e] / (double)count);
            }
        }
    }
}

// One launch for both kinds of cluster, 16 waves per block. Blocks 0 ..
// kBigBlocks-1 come first, so they run beside the others: they take the
// clusters above the split size (listed in big[1 .. big[0]] by the scan) as
// work items (cluster big[1 + i / chunks], chunk i % chunks), blocks taking
// items blockIdx.x, + kBigBlocks, ...; wave p sums part p of the cluster's
// rows (kBigWaves contiguous parts) and wave 0 adds the parts in order and
// writes the mean. Every later block covers kBigWaves consecutive entries
// of `order` (the clusters up to the split size, grouped by load-round
// class; one wave each) x one chunk of kCols columns, and sums each cluster
// alone, in increasing sample order; lane l owns 4 columns.
// If kShift, block b writes the sum of its (new - old)^2 in a fixed order to
// shift_partial[b]. If kNorm, the squared norm over chunk c of the row at
// position p of perm goes to xn_part[c * n + p] (chunks x n float32).
template <bool kVec, bool kShift, int kBatch, bool kNorm>
__global__ __launch_bounds__(kBigWaves * 64) void segment_mean_kernel(
    const float *__restrict__ X, const int *__restrict__ perm, const int *__restrict__ seg_start,
    const int *__restrict__ cnt, const int *__restrict__ big, const int *__restrict__ order,
    const float *C_old, int64_t n, int64_t k, int64_t d, int chunks, float *C_new,
    double *__restrict__ shift_partial, float *__restrict__ xn_part) {
    // C_old and C_new may be the same array: each element is read and written
    // by the same thread only, so they carry no __restrict__.
    __shared__ double part[kBigWaves - 1][kCols];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int lc[4];  // columns within a chunk
#pragma unroll
    for (int e = 0; e < 4; ++e) lc[e] = kVec ? 4 * lane + e : lane + 64 * e;
    double shift = 0.0;
    if (blockIdx.x < kBigBlocks) {
        const int64_t items = (int64_t)big[0] * chunks;
        for (int64_t it = blockIdx.x; it < items; it += kBigBlocks) {
            const int64_t j = big[1 + it / chunks];
            const int64_t c = it % chunks;
            int64_t col[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) col[e] = c * kCols + lc[e];
            const int count = cnt[j];  // > the split size
            const int q = (count + kBigWaves - 1) / kBigWaves;
            const int r0 = min(count, wave * q), r1 = min(count, r0 + q);
            double s[4] = {0.0, 0.0, 0.0, 0.0};
            const int64_t seg = seg_start[j];
            sum_rows<kVec, kBatch, kNorm>(X, perm + seg, r0, r1, d, col, s,
                                          kNorm ? xn_part + c * n + seg : nullptr);
            if (wave > 0)
#pragma unroll
                for (int e = 0; e < 4; ++e) part[wave - 1][lc[e]] = s[e];
            __syncthreads();
            if (wave == 0) {
#pragma unroll 1
                for (int pw = 0; pw < kBigWaves - 1; ++pw)
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[e] += part[pw][lc[e]];
                write_mean<kShift>(C_old, C_new, j, d, count, col, s, shift);
            }
            __syncthreads();  // part is reused by the next item
        }
    } else {
        const unsigned sb = blockIdx.x - kBigBlocks;
        const int64_t i = (int64_t)(sb / (unsigned)chunks) * kBigWaves + wave;
        const int64_t c = sb % (unsigned)chunks;
        int64_t col[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) col[e] = c * kCols + lc[e];
        if (i < k - big[0]) {
            const int64_t j = order[i];
            const int count = cnt[j];  // <= the split size
            {
                double s[4] = {0.0, 0.0, 0.0, 0.0};
                const int64_t seg = seg_start[j];
                sum_rows<kVec, kBatch, kNorm>(X, perm + seg, 0, count, d, col, s,
                                              kNorm ? xn_part + c * n + seg : nullptr);
                write_mean<kShift>(C_old, C_new, j, d, count, col, s, shift);
            }
        }
    }
    if (kShift) {
        for (int off = 32; off > 0; off >>= 1) shift += __shfl_xor(shift, off);
        __syncthreads();  // part may still be read by wave 0 of the last item
        if (lane == 0) part[0][wave] = shift;
        __syncthreads();
        if (threadIdx.x == 0) {
            double t = 0.0;
            for (int w = 0; w < kBigWaves; ++w) t += part[0][w];
            shift_partial[blockIdx.x] = t;
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

static int64_t small_mean_blocks(int64_t k, int64_t d) {
    return cdiv(k, kBigWaves) * cdiv(d, kCols);
}

int64_t update_grid_threads(int64_t n, int64_t k, int64_t d) {
    const int64_t mean = (small_mean_blocks(k, d) + kBigBlocks) * (kBigWaves * 64);
    const int64_t scatter = cdiv(n, kTile) * kTile;  // tile_hist and scatter: 256 per row quarter
    const int64_t scan = cdiv(k, 4) * 256;
    const int64_t m = mean > scatter ? mean : scatter;
    return m > scan ? m : scan;
}

int split_rows(int64_t n, int64_t k, int64_t d) {
    return (n * d >= ((int64_t)1 << 26) && n >= 32 * k) ? kSplitLarge : kSplitSmall;
}

hipError_t launch_count(const int64_t *labels, int64_t n, int64_t k, int64_t d, int64_t *counts,
                        int *num_empty, const UpdateScratch &ws, hipStream_t stream) {
    const int64_t hist_words = k * ws.n_tiles;
    if (hist_words > 0) {
        fill_i32_kernel<<<grid_stride_blocks(hist_words), 256, 0, stream>>>(ws.tile_hist,
                                                                           hist_words);
        if (n > 0)
            tile_hist_kernel<<<(unsigned)(ws.n_tiles * kParts), 256, 0, stream>>>(
                labels, n, k, ws.n_tiles, ws.tile_hist);
        tile_scan_kernel<<<(unsigned)cdiv(k, 4), 256, 0, stream>>>(ws.tile_hist, k, ws.n_tiles,
                                                                   ws.cnt);
    } else {
        // n == 0: every cluster is empty.
        fill_i32_kernel<<<grid_stride_blocks(k), 256, 0, stream>>>(ws.cnt, k);
    }
    if (split_rows(n, k, d) == kSplitLarge)
        cluster_scan_kernel<kSplitLarge><<<1, 1024, 0, stream>>>(ws.cnt, k, ws.seg_start, counts,
                                                                 num_empty, ws.big, ws.order);
    else
        cluster_scan_kernel<kSplitSmall><<<1, 1024, 0, stream>>>(ws.cnt, k, ws.seg_start, counts,
                                                                 num_empty, ws.big, ws.order);
    return hipGetLastError();
}

int64_t mean_blocks(int64_t k, int64_t d) { return small_mean_blocks(k, d) + kBigBlocks; }

int64_t norm_parts(int64_t d) { return cdiv(d, kCols); }

namespace {

// For the row i = perm[p] at every position p < rows:
// min_dist[i] = max(0, ||x_i||^2 + min_dist[i]) with ||x_i||^2 the float64
// sum of its `chunks` partial norms xn_part[c * n + p] (in chunk order),
// rounded once to float32; min_dist holds the assignment's best
// ||c||^2 - 2 x.c on entry. Threads take consecutive positions, so the
// partial norms are read coalesced.
__global__ __launch_bounds__(256) void add_norms_kernel(float *__restrict__ min_dist,
                                                        const float *__restrict__ xn_part,
                                                        const int *__restrict__ perm,
                                                        int64_t rows, int64_t n, int chunks) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < rows; p += stride) {
        // Partials are fetched 16 at a time, all loads before the adds, so a
        // row costs one memory round trip per 16 chunks; the adds stay in
        // chunk order.
        constexpr int G = 16;
        double t = 0.0;
        for (int c0 = 0; c0 < chunks; c0 += G) {
            float v[G];
#pragma unroll
            for (int u = 0; u < G; ++u) v[u] = c0 + u < chunks ? xn_part[(c0 + u) * n + p] : 0.0f;
#pragma unroll
            for (int u = 0; u < G; ++u) t += (double)v[u];
        }
        const int i = perm[p];
        min_dist[i] = fmaxf((float)t + min_dist[i], 0.0f);
    }
}

struct MeanArgs {
    const float *X;
    const int *perm, *seg_start, *cnt, *big, *order;
    const float *C_old;
    int64_t n, k, d;
    int chunks;
    float *C_new;
    double *shift_partial;  // NULL: no centre shift
    float *xn_part;         // NULL: no row norms
};

template <bool kVec, int kBatch>
void launch_mean_vec(const MeanArgs &a, unsigned blocks, unsigned bt, hipStream_t stream) {
    if (a.shift_partial)
        segment_mean_kernel<kVec, true, kBatch, false><<<blocks, bt, 0, stream>>>(
            a.X, a.perm, a.seg_start, a.cnt, a.big, a.order, a.C_old, a.n, a.k, a.d, a.chunks, a.C_new,
            a.shift_partial, nullptr);
    else if (a.xn_part)  // rounds of at most 8 rows: 16 with the pending norms spill
        segment_mean_kernel<kVec, false, (kBatch > 8 ? 8 : kBatch), true><<<blocks, bt, 0, stream>>>(
            a.X, a.perm, a.seg_start, a.cnt, a.big, a.order, a.C_old, a.n, a.k, a.d, a.chunks, a.C_new,
            nullptr, a.xn_part);
    else
        segment_mean_kernel<kVec, false, kBatch, false><<<blocks, bt, 0, stream>>>(
            a.X, a.perm, a.seg_start, a.cnt, a.big, a.order, a.C_old, a.n, a.k, a.d, a.chunks, a.C_new,
            nullptr, nullptr);
}

template <int kBatch>
void launch_mean(const MeanArgs &a, bool vec, unsigned blocks, unsigned bt, hipStream_t stream) {
    if (vec)
        launch_mean_vec<true, kBatch>(a, blocks, bt, stream);
    else
        launch_mean_vec<false, kBatch>(a, blocks, bt, stream);
}

}  // namespace

hipError_t launch_group_and_mean(const float *X, const int64_t *labels, const float *C_old,
                                 int64_t n, int64_t k, int64_t d, float *C_new,
                                 double *shift_partial, float *xn_part, const UpdateScratch &ws,
                                 hipStream_t stream) {
    if (n > 0)
        scatter_kernel<<<(unsigned)(ws.n_tiles * kParts), 256, 0, stream>>>(
            labels, n, k, ws.n_tiles, ws.tile_hist, ws.seg_start, ws.perm);
    const int chunks = (int)cdiv(d, kCols);
    const unsigned blocks = (unsigned)mean_blocks(k, d);
    const unsigned bt = kBigWaves * 64;
    const bool vec = (d % 4 == 0) && ((uintptr_t)X % 16 == 0) && ((uintptr_t)C_old % 16 == 0) &&
                     ((uintptr_t)C_new % 16 == 0);
    const MeanArgs a{X,      ws.perm, ws.seg_start, ws.cnt,      ws.big, ws.order,
                     C_old,  n,       k,            d,           chunks, C_new,
                     shift_partial, xn_part};
    if (n <= 32 * k)  // at most 32 rows per cluster on average
        launch_mean<8>(a, vec, blocks, bt, stream);
    else
        launch_mean<16>(a, vec, blocks, bt, stream);
    return hipGetLastError();
}

hipError_t launch_add_norms(float *min_dist, const float *xn_part, int64_t n, int64_t d,
                            const UpdateScratch &ws, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    add_norms_kernel<<<grid_stride_blocks(n), 256, 0, stream>>>(min_dist, xn_part, ws.perm, n, n,
                                                                (int)norm_parts(d));
    return hipGetLastError();
}

hipError_t launch_update(const float *X, const int64_t *labels, const float *C_old, int64_t n,
                         int64_t k, int64_t d, float *C_new, int64_t *counts, float *xn_part,
                         const UpdateScratch &ws, hipStream_t stream) {
    hipError_t e = launch_count(labels, n, k, d, counts, nullptr, ws, stream);
    if (e != hipSuccess) return e;
    return launch_group_and_mean(X, labels, C_old, n, k, d, C_new, nullptr, xn_part, ws, stream);
}

}  // namespace km
