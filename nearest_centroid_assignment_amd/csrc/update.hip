// update.hip - Lloyd centroid update on gfx950.
//
// The update of "Three shapes that fit an eager Gram assignment", section Full
// Lloyd step, is a one-hot (n, k) membership matrix times X; the Cython kernel
// of "004 - tile sizes ...", section Cython reference, scatters each sample
// into per-thread centre buffers instead. Here the samples are first grouped
// by label with a stable counting sort, then every (cluster, column chunk)
// block adds its cluster's rows in increasing sample order:
//
//   rank_hist_kernel     per tile of 1024 rows: every row's rank among the
//                        tile's rows with the same label (stable), and the
//                        tile's histogram column; in a Lloyd step fused with
//                        the assignment's finalize (keys -> labels)
//   tile_prefix_kernel   per cluster: exclusive prefix over tiles, cluster
//                        size
//   cluster_scan_kernel  one block: exclusive prefix over clusters ->
//                        segment starts, counts, and the lists the mean
//                        kernel schedules by
//   scatter_kernel       perm[segment start + rows of the cluster in earlier
//                        tiles + rank] = row   (stable)
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
constexpr int kTileWaves = kTile / 64;     // one thread per row
constexpr int kRankLdsMax = 16384;         // rank_hist keeps up to this many label counters in LDS
constexpr int kScanRegMax = 16;            // scan: clusters per thread held in registers
constexpr int kCols = 256;                 // columns per segment_mean block (64 lanes x 4)
constexpr int kSplitSmall = 64;            // larger clusters are split in kBigWaves parts ...
constexpr int kSplitLarge = 128;           // ... or larger than this, on big inputs
constexpr int kBigWaves = 16;              // waves (parts) per big-cluster block
constexpr int kBigBlocks = 256;            // segment_mean blocks that take the large clusters

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Rank of each lane's label among the lanes below it with the same label
// (stable), and how many lanes hold that label. Lanes with valid == false
// take no part (rank and count 0). One round per distinct label: the lowest
// pending lane names a label, a ballot finds its lanes.
__device__ __forceinline__ void wave_match(int label, bool valid, int &rank, int &count) {
    const int lane = threadIdx.x & 63;
    const unsigned long long below = (1ull << lane) - 1ull;
    unsigned long long todo = __ballot(valid);
    rank = 0;
    count = 0;
    while (todo != 0ull) {
        const int leader = __builtin_ctzll(todo);
        const int l0 = __builtin_amdgcn_readlane(label, leader);
        const bool eq = valid && label == l0;
        const unsigned long long m = __ballot(eq);
        if (eq) {
            rank = __popcll(m & below);
            count = __popcll(m);
        }
        todo &= ~m;
    }
}

__device__ __forceinline__ int coherent_load(const int *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The label table of rank_hist_kernel: LDS, or global memory read and written
// past the compute unit's cache, so that one wave sees what another stored
// before the barrier between their turns.
template <bool kLds>
__device__ __forceinline__ int table_load(const int *p) {
    return kLds ? *p : coherent_load(p);
}
template <bool kLds>
__device__ __forceinline__ void table_store(int *p, int v) {
    if (kLds)
        *p = v;
    else
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One block of kTile threads per tile of kTile rows, a thread per row.
// rank[i] = number of rows of the tile before row i with the same label;
// tile_hist[b * k + j] = rows of tile b with label j, for every j. Each wave
// first ranks its 64 rows among themselves (wave_match); then the waves take
// turns in row order, behind a barrier each: a wave adds to its rows' ranks
// the counts of their labels over the earlier waves, kept per label in a
// table, and adds its own counts to the table. The table is in LDS when k <=
// kRankLdsMax (kLds), else the tile's own histogram column in global memory.
// Rows with a label outside [0, k) are skipped.
// kFromKeys: the labels come from the assignment's packed keys, turned into
// int64 labels in place first (and min_dist, as finalize_kernel does; the
// index of a key is always < k, and is clamped to be sure).
template <bool kLds, bool kFromKeys>
__global__ __launch_bounds__(kTile) void rank_hist_kernel(const int64_t *__restrict__ labels,
                                                          unsigned long long *__restrict__ keys,
                                                          float *__restrict__ min_dist,
                                                          bool add_norm, int64_t n, int64_t k,
                                                          int *__restrict__ tile_hist,
                                                          unsigned short *__restrict__ rank_out,
                                                          Gate gate) {
    extern __shared__ int lds_table[];
    if (gated(gate)) return;
    const int tid = threadIdx.x, wave = tid >> 6;
    const int64_t b = blockIdx.x;
    const int64_t i = b * kTile + tid;
    int l = -1;
    if (i < n) {
        if (kFromKeys) {
            const unsigned long long key = keys[i];
            if (min_dist) {
                const float partial = key_distance(key);
                min_dist[i] = add_norm ? fmaxf(min_dist[i] + partial, 0.0f) : partial;
            }
            const unsigned long long idx = key & 0xffffffffull;
            l = idx < (unsigned long long)k ? (int)idx : 0;
            keys[i] = (unsigned long long)l;  // the int64 label
        } else {
            const int64_t v = labels[i];
            l = (v >= 0 && v < k) ? (int)v : -1;
        }
    }
    int *table = kLds ? lds_table : tile_hist + b * k;
    for (int64_t j = tid; j < k; j += kTile) table_store<kLds>(table + j, 0);
    int rank, count;
    wave_match(l, l >= 0, rank, count);
    for (int w = 0; w < kTileWaves; ++w) {
        __syncthreads();  // the table holds the counts of waves 0 .. w-1
        if (wave == w && l >= 0) {
            const int before = table_load<kLds>(table + l);
            if (rank == count - 1) table_store<kLds>(table + l, before + count);  // one writer per label
            rank += before;
        }
    }
    __syncthreads();
    if (l >= 0) rank_out[i] = (unsigned short)rank;
    if (kLds)
        for (int64_t j = tid; j < k; j += kTile) tile_hist[b * k + j] = lds_table[j];
}

// Load-round classes of the clusters summed by one wave (at most kSplit
// rows): class ceil(count / 8), 0 .. kSplit / 8.
template <int kSplit>
__device__ __forceinline__ int round_class(int count) {
    return count <= kSplit ? (count + 7) / 8 : -1;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no trip
// through LDS): a Hillis-Steele scan inside each row of 16 lanes (row_shr by
// 1, 2, 4, 8; lanes shifted in from outside the row read 0), then the total of
// row 0 is added to row 1 and that of row 2 to row 3 (row_bcast:15, rows 1
// and 3 only), then that of rows 0-1 to rows 2 and 3 (row_bcast:31). Every
// lane of the wave must be active.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// Exclusive prefixes of Q values over the block's 1024 threads in thread
// order (excl) and their block totals (total): a DPP scan per wave, the wave
// totals through LDS, a prefix over the 16 waves by the first Q threads.
// Three barriers for all Q values; every thread must call it (all lanes
// active).
template <int Q>
__device__ __forceinline__ void block_excl_scan(const int (&x)[Q], int (&excl)[Q], int (&total)[Q]) {
    __shared__ int wsum[16][Q];
    __shared__ int wpre[16][Q];
    __shared__ int btot[Q];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int incl = wave_incl_scan(x[q]);
        excl[q] = incl - x[q];
        if (lane == 63) wsum[wave][q] = incl;
    }
    __syncthreads();
    if (tid < Q) {
        int run = 0;
        for (int w = 0; w < 16; ++w) {
            wpre[w][tid] = run;
            run += wsum[w][tid];
        }
        btot[tid] = run;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        excl[q] += wpre[wave][q];
        total[q] = btot[q];
    }
    __syncthreads();  // the arrays are rewritten by the next call
}

// Class counts travel packed two to an int, 16 bits each: every count is at
// most the number of clusters the scan covers at once (<= 16384 < 2^16), so
// sums of packed ints add the halves independently.
template <int kClasses>
__device__ __forceinline__ void add_class(int (&packed)[(kClasses + 1) / 2], int cl) {
#pragma unroll
    for (int p = 0; p < (kClasses + 1) / 2; ++p)
        packed[p] += (cl >= 0 && (cl >> 1) == p) ? (1 << (16 * (cl & 1))) : 0;
}

__device__ __forceinline__ int unpack_half(int packed, int half) {
    return (packed >> (16 * half)) & 0xffff;
}

// The cluster scan, one block of 1024 threads, for k <= 1024 * R: thread t
// takes clusters t*R .. t*R + R - 1. Writes seg_start (exclusive prefix of the
// sizes), counts (int64 sizes), big[0] = number of clusters above kSplit rows
// and big[1 ..] their indices in increasing order, order = the other clusters
// grouped by load-round class, most rounds first, increasing index within a
// class (ranks from scans, so the order is the same on every run; the mean
// kernel gives 16 consecutive entries of `order` to one block, so a block's
// waves run the same number of load rounds), and the number of empty
// clusters. With R > 1 the sizes come in and the segment starts and the order
// go out through LDS, so that every global access of a wave covers
// consecutive clusters (a thread's own R clusters are R apart from its
// neighbours'); the size table is padded by one word every 32 so that the
// threads' strided LDS accesses fall in distinct banks.
template <int R>
__device__ __forceinline__ int padded(int j) {
    return R > 1 ? j + (j >> 5) : j;
}

template <int R, int kSplit>
__device__ int cluster_scan_regs(const int *cnt, int own, int64_t k, int *seg_start,
                                 int64_t *counts, int *num_empty, int *no_empty, int *big,
                                 int *order) {
    static_assert(R * 1024 < 65536, "packed class counts need k < 2^16");
    constexpr int kClasses = kSplit / 8 + 1;
    constexpr int kPacked = (kClasses + 1) / 2;
    constexpr int Q = 2 + kPacked;  // sizes; above-split | empty << 16; classes, two per int
    constexpr int N = 1024 * R;
    __shared__ int sizes[R > 1 ? N + N / 32 : 1];  // sizes, then segment starts
    __shared__ int placed[R > 1 ? N : 1];          // the order list
    const int tid = threadIdx.x;
    const int64_t j0 = (int64_t)tid * R;
    int v[R];
    if (R == 1) {
        // From cnt, or (cnt == NULL) the thread's own cluster size, -1 past k.
        v[0] = cnt == nullptr ? own : j0 < k ? cnt[j0] : -1;
    } else {
#pragma unroll
        for (int e = 0; e < R; ++e) {
            const int j = e * 1024 + tid;
            const int c = cnt[j < k ? j : k - 1];  // no condition on the load: all R in flight
            if (j < k) {
                sizes[padded<R>(j)] = c;
                counts[j] = c;
            }
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < R; ++e) v[e] = j0 + e < k ? sizes[padded<R>((int)j0 + e)] : -1;
    }
    int x[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) x[q] = 0;
#pragma unroll
    for (int e = 0; e < R; ++e) {
        if (v[e] < 0) continue;
        x[0] += v[e];
        x[1] += (v[e] > kSplit ? 1 : 0) + (v[e] == 0 ? 1 << 16 : 0);
        int (&cls)[kPacked] = *reinterpret_cast<int (*)[kPacked]>(&x[2]);
        add_class<kClasses>(cls, round_class<kSplit>(v[e]));
    }
    int pos[Q], tot[Q];
    block_excl_scan<Q>(x, pos, tot);  // (its barriers also order the LDS reads above)
    // Class c starts after every class with more rounds: fold that start into
    // the thread's packed positions.
    int start = 0;
#pragma unroll
    for (int c = kClasses - 1; c >= 0; --c) {
        pos[2 + c / 2] += start << (16 * (c & 1));
        start += unpack_half(tot[2 + c / 2], c & 1);
    }
    const int n_ordered = start;
    const int first_seg = pos[0];
    int seg = pos[0], bpos = pos[1] & 0xffff;
#pragma unroll
    for (int e = 0; e < R; ++e) {
        if (v[e] < 0) continue;
        const int j = (int)j0 + e;
        if (R == 1) {
            seg_start[j] = seg;
            counts[j] = v[e];
        } else {
            sizes[padded<R>(j)] = seg;  // this thread's own slots only
        }
        seg += v[e];
        if (v[e] > kSplit) big[1 + bpos++] = j;
        const int cl = round_class<kSplit>(v[e]);
        if (cl >= 0) {
            int at = 0;
#pragma unroll
            for (int p = 0; p < kPacked; ++p)
                if ((cl >> 1) == p) {
                    at = unpack_half(pos[2 + p], cl & 1);
                    pos[2 + p] += 1 << (16 * (cl & 1));
                }
            if (R == 1)
                order[at] = j;
            else
                placed[at] = j;
        }
    }
    if (R > 1) {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < R; ++e) {
            const int j = e * 1024 + tid;
            if (j < k) seg_start[j] = sizes[padded<R>(j)];
            if (j < n_ordered) order[j] = placed[j];
        }
    }
    if (tid == 0) {
        big[0] = tot[1] & 0xffff;
        if (num_empty) {
            const int empty = unpack_half(tot[1], 1);
            *num_empty = empty;
            *no_empty = empty == 0;
        }
    }
    return first_seg;
}

// The same for any k, 1024 clusters at a time, a cluster per thread (each
// chunk's sizes loaded in turn; a first pass takes the class totals): used
// when k > 1024 * kScanRegMax. Running totals across chunks are full ints.
template <int kSplit>
__device__ void cluster_scan_chunked(const int *cnt, int64_t k, int *seg_start, int64_t *counts,
                                     int *num_empty, int *no_empty, int *big, int *order) {
    constexpr int kClasses = kSplit / 8 + 1;
    constexpr int kPacked = (kClasses + 1) / 2;
    constexpr int Q = 2 + kPacked;
    const int tid = threadIdx.x;
    int cls_carry[kClasses];
#pragma unroll
    for (int c = 0; c < kClasses; ++c) cls_carry[c] = 0;
    // Pass 1: class totals.
    for (int64_t base = 0; base < k; base += 1024) {
        const int64_t j = base + tid;
        const int v = j < k ? cnt[j] : -1;
        int x[Q], p[Q], t[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) x[q] = 0;
        int (&cls)[kPacked] = *reinterpret_cast<int (*)[kPacked]>(&x[2]);
        add_class<kClasses>(cls, v >= 0 ? round_class<kSplit>(v) : -1);
        block_excl_scan<Q>(x, p, t);
#pragma unroll
        for (int c = 0; c < kClasses; ++c) cls_carry[c] += unpack_half(t[2 + c / 2], c & 1);
    }
    {
        int start = 0;
#pragma unroll
        for (int c = kClasses - 1; c >= 0; --c) {
            const int tc = cls_carry[c];
            cls_carry[c] = start;
            start += tc;
        }
    }
    // Pass 2: placement.
    int seg_carry = 0, big_carry = 0, empty_carry = 0;
    for (int64_t base = 0; base < k; base += 1024) {
        const int64_t j = base + tid;
        const int v = j < k ? cnt[j] : -1;
        const int cl = v >= 0 ? round_class<kSplit>(v) : -1;
        int x[Q], p[Q], t[Q];
        x[0] = v >= 0 ? v : 0;
        x[1] = (v > kSplit ? 1 : 0) + (v == 0 ? 1 << 16 : 0);
#pragma unroll
        for (int q = 2; q < Q; ++q) x[q] = 0;
        int (&cls)[kPacked] = *reinterpret_cast<int (*)[kPacked]>(&x[2]);
        add_class<kClasses>(cls, cl);
        block_excl_scan<Q>(x, p, t);
        if (v >= 0) {
            seg_start[j] = seg_carry + p[0];
            counts[j] = v;
        }
        if (v > kSplit) big[1 + big_carry + (p[1] & 0xffff)] = (int)j;
#pragma unroll
        for (int c = 0; c < kClasses; ++c) {
            if (cl == c) order[cls_carry[c] + unpack_half(p[2 + c / 2], c & 1)] = (int)j;
            cls_carry[c] += unpack_half(t[2 + c / 2], c & 1);
        }
        seg_carry += t[0];
        big_carry += t[1] & 0xffff;
        empty_carry += unpack_half(t[1], 1);
    }
    if (tid == 0) {
        big[0] = big_carry;
        if (num_empty) {
            *num_empty = empty_carry;
            *no_empty = empty_carry == 0;
        }
    }
}

// Per cluster j (a thread each, one wave per block, so that the loads and
// stores spread over k / 64 compute units): the exclusive prefix of its tile
// counts over the tiles, in place, and its size cnt[j]. The loads of a wave
// read 64 consecutive clusters of one tile (the tile's histogram column is
// contiguous); the next U tiles' loads are issued before the current U
// tiles' stores, so a thread waits for memory once per U tiles.
__global__ __launch_bounds__(64) void tile_prefix_kernel(int *__restrict__ tile_hist, int64_t k,
                                                         int64_t n_tiles, int *__restrict__ cnt,
                                                         Gate gate) {
    if (gated(gate)) return;
    const int64_t j = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (j >= k) return;
    int run = 0;
    constexpr int U = 32;  // tile counts in flight per thread
    if (n_tiles <= 2 * U) {
        // Every tile's count in flight at once: one wait for memory.
        int v[2 * U];
#pragma unroll
        for (int u = 0; u < 2 * U; ++u) v[u] = u < n_tiles ? tile_hist[u * k + j] : 0;
#pragma unroll
        for (int u = 0; u < 2 * U; ++u) {
            if (u < n_tiles) tile_hist[u * k + j] = run;
            run += v[u];
        }
    } else {
        int v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = tile_hist[u * k + j];
        for (int64_t b0 = 0; b0 < n_tiles; b0 += U) {
            int nxt[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                nxt[u] = b0 + U + u < n_tiles ? tile_hist[(b0 + U + u) * k + j] : 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (b0 + u < n_tiles) tile_hist[(b0 + u) * k + j] = run;
                run += v[u];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = nxt[u];
        }
    }
    cnt[j] = run;
}

// The cluster scan over cnt, one block (R = 0: any k, in 1024-cluster chunks).
template <int R, int kSplit>
__global__ __launch_bounds__(1024) void cluster_scan_kernel(const int *__restrict__ cnt, int64_t k,
                                                            int *__restrict__ seg_start,
                                                            int64_t *__restrict__ counts,
                                                            int *__restrict__ num_empty,
                                                            int *__restrict__ no_empty,
                                                            int *__restrict__ big,
                                                            int *__restrict__ order, Gate gate) {
    if (gated(gate)) return;
    if (R > 0)
        cluster_scan_regs<(R > 0 ? R : 1), kSplit>(cnt, 0, k, seg_start, counts, num_empty,
                                                   no_empty, big, order);
    else
        cluster_scan_chunked<kSplit>(cnt, k, seg_start, counts, num_empty, no_empty, big, order);
}

// One thread per row: perm[segment start + rows of the cluster in earlier
// tiles + rank within the tile] = row. Stable: inside a cluster, rows keep
// increasing sample order.
__global__ __launch_bounds__(256) void scatter_kernel(const int64_t *__restrict__ labels, int64_t n,
                                                      int64_t k,
                                                      const int *__restrict__ tile_prefix,
                                                      const unsigned short *__restrict__ rank,
                                                      const int *__restrict__ seg_start,
                                                      int *__restrict__ perm, Gate gate) {
    if (gated(gate)) return;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t l = labels[i];
    if (l < 0 || l >= k) return;
    const int64_t b = i / kTile;
    perm[(int64_t)seg_start[l] + tile_prefix[b * k + l] + rank[i]] = (int)i;
}

// For k <= 1024 clusters and at most kPlaceTiles tiles: the tile prefix, the
// cluster scan and the scatter in one launch, a block per tile (the three
// launches they replace cost more in launch gaps than the work they do at
// these sizes). Thread j of every block reads cluster j's counts in all the
// tiles (at most 64 K words in all, from the L2) and takes the rows of j in
// the tiles before its own and in all of them; one block scan of the sizes
// gives the segment starts, and the block places its own tile's rows:
// perm[segment start + rows in earlier tiles + rank] = row. Block 0 also
// writes the per-cluster results of the cluster scan (cnt, counts,
// seg_start, the lists of the mean kernel). The integer sums are the same in
// every block.
constexpr int kPlaceTiles = 64;

template <int kSplit>
__global__ __launch_bounds__(1024) void place_kernel(
    const int64_t *__restrict__ labels, int64_t n, int64_t k, const int *__restrict__ tile_hist,
    const unsigned short *__restrict__ rank, int64_t n_tiles, int *__restrict__ cnt,
    int *__restrict__ seg_start, int64_t *__restrict__ counts, int *__restrict__ num_empty,
    int *__restrict__ no_empty, int *__restrict__ big, int *__restrict__ order,
    int *__restrict__ perm, Gate gate) {
    __shared__ int base[1024];  // per cluster: segment start + rows in earlier tiles
    if (gated(gate)) return;
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int64_t i = b * kTile + tid;
    int64_t lv = -1;
    int r = 0;
    if (i < n) {
        lv = labels[i];
        r = rank[i];  // (meaningless, and unused, for a label outside [0, k))
    }
    int before = 0, total = -1;
    if (tid < k) {
        total = 0;
        if (n_tiles > 0) {
            int v[kPlaceTiles];
            // Past the last tile the index is clamped and the value ignored,
            // so the loads carry no condition and are all in flight at once.
#pragma unroll
            for (int u = 0; u < kPlaceTiles; ++u)
                v[u] = tile_hist[(int64_t)(u < n_tiles ? u : n_tiles - 1) * k + tid];
#pragma unroll
            for (int u = 0; u < kPlaceTiles; ++u) {
                const int c = u < n_tiles ? v[u] : 0;
                before += u < b ? c : 0;
                total += c;
            }
        }
    }
    int seg;
    if (b == 0) {
        seg = cluster_scan_regs<1, kSplit>(nullptr, total, k, seg_start, counts, num_empty,
                                           no_empty, big, order);
        if (tid < k) cnt[tid] = total;
    } else {
        const int x[1] = {total > 0 ? total : 0};
        int p[1], t[1];
        block_excl_scan<1>(x, p, t);
        seg = p[0];
    }
    if (tid < k) base[tid] = seg + before;
    __syncthreads();
    if (lv >= 0 && lv < k) perm[base[lv] + r] = (int)i;
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
// adds in order. X is read once, with non-temporal loads (streamed past the
// caches; measured 10 % faster at 65536 x 1024 x 2048 and 4 % at
// 65536 x 4096 x 16384 than ordinary loads, same bits). kBatch is 8: with
// 16, fewer rows are in flight per wave on short clusters (load slots of a
// round go unused) and the kernel needs about 100 registers instead of about
// 66; measured slower at every workload, also at 65536 x 1024 x 2048 with 64
// rows per cluster. When clusters average at most 8 rows, kBatch is 4: under
// 64 registers, so two 16-wave blocks share a CU, which doubles the rows in
// flight where a cluster fills only one or two rounds (4 % faster at
// 65536 x 16384 x 8192, 4 rows per cluster; the same or slower at 16 rows).
// The order of the adds does not depend on kBatch.
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
                           ? __builtin_nontemporal_load(
                                 reinterpret_cast<const f32x4 *>(X + base[u] + col[0]))
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
                    v[u][e] = (base[u] >= 0 && col[e] < d)
                                  ? __builtin_nontemporal_load(X + base[u] + col[e])
                                  : 0.f;
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
    double *__restrict__ shift_partial, float *__restrict__ xn_part, Gate gate) {
    // C_old and C_new may be the same array: each element is read and written
    // by the same thread only, so they carry no __restrict__.
    __shared__ double part[kBigWaves - 1][kCols];
    if (gated(gate)) return;
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
    const int64_t rank = cdiv(n, kTile) * kTile;  // rank_hist: a thread per row, whole tiles
    const int64_t scatter = cdiv(n, 256) * 256;
    const int64_t scan = cdiv(k, 1024) * 1024;
    int64_t m = mean > rank ? mean : rank;
    m = m > scatter ? m : scatter;
    return m > scan ? m : scan;
}

namespace {
// The counting's last steps and the scatter run as one place_kernel launch.
bool place_fused(int64_t n, int64_t k) { return k <= 1024 && cdiv(n, kTile) <= kPlaceTiles; }
}  // namespace

int split_rows(int64_t n, int64_t k, int64_t d) {
    return (n * d >= ((int64_t)1 << 26) && n >= 32 * k) ? kSplitLarge : kSplitSmall;
}

namespace {

template <bool kFromKeys>
hipError_t launch_rank_hist_impl(const int64_t *labels, unsigned long long *keys,
                                 float *min_dist, bool add_norm, int64_t n, int64_t k,
                                 const UpdateScratch &ws, Gate gate, hipStream_t stream) {
    if (n <= 0) return hipSuccess;  // no tile (the tile prefix then gives every size 0)
    const unsigned blocks = (unsigned)ws.n_tiles;
    if (k <= kRankLdsMax)
        rank_hist_kernel<true, kFromKeys><<<blocks, kTile, (size_t)k * sizeof(int), stream>>>(
            labels, keys, min_dist, add_norm, n, k, ws.tile_hist, ws.rank, gate);
    else
        rank_hist_kernel<false, kFromKeys><<<blocks, kTile, 0, stream>>>(
            labels, keys, min_dist, add_norm, n, k, ws.tile_hist, ws.rank, gate);
    return hipGetLastError();
}

template <int kSplit>
void launch_place(const int64_t *labels, int64_t n, int64_t k, int64_t *counts, int *num_empty,
                  const UpdateScratch &ws, Gate gate, hipStream_t stream) {
    const unsigned blocks = ws.n_tiles > 0 ? (unsigned)ws.n_tiles : 1u;  // block 0 always runs
    place_kernel<kSplit><<<blocks, 1024, 0, stream>>>(labels, n, k, ws.tile_hist, ws.rank,
                                                      ws.n_tiles, ws.cnt, ws.seg_start, counts,
                                                      num_empty, ws.no_empty, ws.big, ws.order,
                                                      ws.perm, gate);
}

template <int kSplit>
void launch_cluster_scan(int64_t k, int64_t *counts, int *num_empty, const UpdateScratch &ws,
                         Gate gate, hipStream_t stream) {
    const int64_t r = cdiv(k, 1024);  // clusters per thread
#define KM_SCAN(R)                                                                        \
    cluster_scan_kernel<R, kSplit><<<1, 1024, 0, stream>>>(ws.cnt, k, ws.seg_start, counts, \
                                                           num_empty, ws.no_empty, ws.big, \
                                                           ws.order, gate)
    if (r <= 1)
        KM_SCAN(1);
    else if (r <= 2)
        KM_SCAN(2);
    else if (r <= 4)
        KM_SCAN(4);
    else if (r <= 8)
        KM_SCAN(8);
    else if (r <= kScanRegMax)
        KM_SCAN(kScanRegMax);
    else
        KM_SCAN(0);
#undef KM_SCAN
}

}  // namespace

hipError_t launch_rank_hist(const int64_t *labels, int64_t n, int64_t k, const UpdateScratch &ws,
                            Gate gate, hipStream_t stream) {
    return launch_rank_hist_impl<false>(labels, nullptr, nullptr, false, n, k, ws, gate, stream);
}

hipError_t launch_finalize_rank_hist(unsigned long long *keys, float *min_dist, bool add_norm,
                                     int64_t n, int64_t k, const UpdateScratch &ws, Gate gate,
                                     hipStream_t stream) {
    return launch_rank_hist_impl<true>(nullptr, keys, min_dist, add_norm, n, k, ws, gate, stream);
}

hipError_t launch_scan(const int64_t *labels, int64_t n, int64_t k, int64_t d, int64_t *counts,
                       int *num_empty, const UpdateScratch &ws, Gate gate, hipStream_t stream) {
    if (place_fused(n, k)) {
        if (split_rows(n, k, d) == kSplitLarge)
            launch_place<kSplitLarge>(labels, n, k, counts, num_empty, ws, gate, stream);
        else
            launch_place<kSplitSmall>(labels, n, k, counts, num_empty, ws, gate, stream);
        return hipGetLastError();
    }
    tile_prefix_kernel<<<(unsigned)cdiv(k, 64), 64, 0, stream>>>(ws.tile_hist, k, ws.n_tiles, ws.cnt,
                                                                  gate);
    if (split_rows(n, k, d) == kSplitLarge)
        launch_cluster_scan<kSplitLarge>(k, counts, num_empty, ws, gate, stream);
    else
        launch_cluster_scan<kSplitSmall>(k, counts, num_empty, ws, gate, stream);
    return hipGetLastError();
}

hipError_t launch_count(const int64_t *labels, int64_t n, int64_t k, int64_t d, int64_t *counts,
                        int *num_empty, const UpdateScratch &ws, Gate gate, hipStream_t stream) {
    hipError_t e = launch_rank_hist(labels, n, k, ws, gate, stream);
    if (e == hipSuccess) e = launch_scan(labels, n, k, d, counts, num_empty, ws, gate, stream);
    return e;
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
template <int G>
__global__ __launch_bounds__(256) void add_norms_kernel(float *__restrict__ min_dist,
                                                        const float *__restrict__ xn_part,
                                                        const int *__restrict__ perm,
                                                        int64_t rows, int64_t n, int chunks) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < rows; p += stride) {
        const int i = perm[p];
        // Partials are fetched G at a time (G >= chunks on the common shapes:
        // one memory round trip per row). The loads carry no condition (past
        // the last chunk the index is clamped and the value then ignored), so
        // all G are in flight together: a branch around each would make the
        // compiler wait for every load before issuing the next. The adds stay
        // in chunk order; the ignored ones add +0.0 to a sum of squares.
        double t = 0.0;
        for (int c0 = 0; c0 < chunks; c0 += G) {
            float v[G];
#pragma unroll
            for (int u = 0; u < G; ++u) {
                const int c = c0 + u < chunks ? c0 + u : chunks - 1;
                v[u] = xn_part[(int64_t)c * n + p];
            }
#pragma unroll
            for (int u = 0; u < G; ++u) t += c0 + u < chunks ? (double)v[u] : 0.0;
        }
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
    Gate gate;
};

template <bool kVec, int kBatch>
void launch_mean_vec(const MeanArgs &a, unsigned blocks, unsigned bt, hipStream_t stream) {
    if (a.shift_partial)
        segment_mean_kernel<kVec, true, kBatch, false><<<blocks, bt, 0, stream>>>(
            a.X, a.perm, a.seg_start, a.cnt, a.big, a.order, a.C_old, a.n, a.k, a.d, a.chunks, a.C_new,
            a.shift_partial, nullptr, a.gate);
    else if (a.xn_part)
        segment_mean_kernel<kVec, false, kBatch, true><<<blocks, bt, 0, stream>>>(
            a.X, a.perm, a.seg_start, a.cnt, a.big, a.order, a.C_old, a.n, a.k, a.d, a.chunks, a.C_new,
            nullptr, a.xn_part, a.gate);
    else
        segment_mean_kernel<kVec, false, kBatch, false><<<blocks, bt, 0, stream>>>(
            a.X, a.perm, a.seg_start, a.cnt, a.big, a.order, a.C_old, a.n, a.k, a.d, a.chunks, a.C_new,
            nullptr, nullptr, a.gate);
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
                                 Gate gate, hipStream_t stream) {
    if (n > 0 && !place_fused(n, k))  // (else the count has placed the rows)
        scatter_kernel<<<(unsigned)cdiv(n, 256), 256, 0, stream>>>(
            labels, n, k, ws.tile_hist, ws.rank, ws.seg_start, ws.perm, gate);
    const int chunks = (int)cdiv(d, kCols);
    const unsigned blocks = (unsigned)mean_blocks(k, d);
    const unsigned bt = kBigWaves * 64;
    const bool vec = (d % 4 == 0) && ((uintptr_t)X % 16 == 0) && ((uintptr_t)C_old % 16 == 0) &&
                     ((uintptr_t)C_new % 16 == 0);
    const MeanArgs a{X,      ws.perm, ws.seg_start, ws.cnt,        ws.big,  ws.order,
                     C_old,  n,       k,            d,             chunks,  C_new,
                     shift_partial, xn_part, gate};
    if (n <= 8 * k)  // clusters of at most 8 rows on average: rounds of 4 (see sum_rows)
        launch_mean<4>(a, vec, blocks, bt, stream);
    else
        launch_mean<8>(a, vec, blocks, bt, stream);
    return hipGetLastError();
}

hipError_t launch_add_norms(float *min_dist, const float *xn_part, int64_t n, int64_t d,
                            const UpdateScratch &ws, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int chunks = (int)norm_parts(d);
    const unsigned blocks = grid_stride_blocks(n);
#define KM_ADD_NORMS(G) \
    add_norms_kernel<G><<<blocks, 256, 0, stream>>>(min_dist, xn_part, ws.perm, n, n, chunks)
    if (chunks <= 4)
        KM_ADD_NORMS(4);
    else if (chunks <= 8)
        KM_ADD_NORMS(8);
    else if (chunks <= 16)
        KM_ADD_NORMS(16);
    else if (chunks <= 32)
        KM_ADD_NORMS(32);
    else
        KM_ADD_NORMS(64);
#undef KM_ADD_NORMS
    return hipGetLastError();
}

hipError_t launch_update(const float *X, const int64_t *labels, const float *C_old, int64_t n,
                         int64_t k, int64_t d, float *C_new, int64_t *counts, float *xn_part,
                         bool counted, const UpdateScratch &ws, hipStream_t stream) {
    hipError_t e = counted ? launch_scan(labels, n, k, d, counts, nullptr, ws, Gate{}, stream)
                           : launch_count(labels, n, k, d, counts, nullptr, ws, Gate{}, stream);
    if (e != hipSuccess) return e;
    return launch_group_and_mean(X, labels, C_old, n, k, d, C_new, nullptr, xn_part, ws, Gate{},
                                 stream);
}

}  // namespace km
