// fit.hip - pieces of the Lloyd driver (kmeans_fit) around the assignment and
// the update: empty-cluster relocation and the per-iteration scalars.
//
// Relocation ("004 - tile sizes ...", section Cython timing: the Lloyd call
// relocates empty clusters; the rule itself is not on the pages). Reading
// implemented here: after the assignment against the old centres, let E be
// the empty clusters in increasing index and m = min(|E|, n). The m samples
// farthest from their assigned old centre (float64 difference-form distance;
// larger first, lower sample index first on equal distances) are moved, the
// r-th becoming the only member of cluster E[r]. The update then runs on the
// new labels; a cluster emptied by a move keeps its old centre.
//
//   reloc_dist_kernel    exact float64 distance of every sample to its centre
//                        (skipped, by every block, when no cluster is empty)
//   reloc_select_kernel  one block: list E, pick the m farthest samples by a
//                        bitwise threshold search on the distances, compact
//                        them in sample order, sort them (bitonic) by distance
//                        descending then index ascending, pair them with E
//   reloc_apply_kernel   relabel the moved samples
//   shift_kernel         one block: centre shift = sum of the update's
//                        per-block partials, in block order; converged flag
//   inertia_kernel       one block: sum of the final squared distances
// Every reduction runs in a fixed order, so results are deterministic.
#include "kernels.h"

namespace km {
namespace {

__global__ __launch_bounds__(256) void reloc_dist_kernel(const float *__restrict__ X,
                                                         const float *__restrict__ C,
                                                         const int64_t *__restrict__ labels,
                                                         int64_t n, int64_t d,
                                                         const int *__restrict__ num_empty,
                                                         double *__restrict__ dist) {
    if (*num_empty == 0) return;  // uniform: nothing to relocate
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= n) return;
    const float *x = X + i * d;
    const float *c = C + labels[i] * d;
    double s = 0.0;
    for (int64_t t = lane; t < d; t += 64) {
        const double diff = (double)x[t] - (double)c[t];
        s += diff * diff;
    }
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) dist[i] = s;
}

// Exclusive prefix of a 0/1 flag over the 1024 threads of the block, in
// thread order; *total receives the block's sum. lds16 holds 16 ints.
__device__ int block_flag_scan(bool flag, int *total, int *lds16) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned long long mask = __ballot(flag);
    const int in_wave = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0) lds16[wave] = __popcll(mask);
    __syncthreads();
    int before = 0, tot = 0;
    for (int w = 0; w < 16; ++w) {
        const int v = lds16[w];
        before += w < wave ? v : 0;
        tot += v;
    }
    __syncthreads();
    *total = tot;
    return before + in_wave;
}

// Sum of a per-thread count over the 1024 threads of the block.
__device__ long long block_count(long long v, long long *lds16) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) lds16[threadIdx.x >> 6] = v;
    __syncthreads();
    long long t = 0;
    for (int w = 0; w < 16; ++w) t += lds16[w];
    __syncthreads();
    return t;
}

// (key_a, idx_a) goes before (key_b, idx_b): larger distance first, then
// lower index.
__device__ __forceinline__ bool before(unsigned long long ka, int ia, unsigned long long kb,
                                       int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

__global__ __launch_bounds__(1024) void reloc_select_kernel(
    const int *__restrict__ cnt, int64_t k, int64_t n, const double *__restrict__ dist,
    const int *__restrict__ num_empty, int *__restrict__ empty, unsigned long long *sort_key,
    int *sort_idx, int64_t sort_cap, int *__restrict__ moves_src, int *__restrict__ moves_dst,
    int *__restrict__ n_moves) {
    __shared__ int lds16[16];
    __shared__ long long lds16ll[16];
    const int tid = threadIdx.x;
    if (*num_empty == 0) {
        if (tid == 0) *n_moves = 0;
        return;
    }
    // E: empty clusters in increasing index.
    int n_empty = 0;
    for (int64_t base = 0; base < k; base += 1024) {
        const int64_t j = base + tid;
        const bool e = j < k && cnt[j] == 0;
        int tot;
        const int pos = block_flag_scan(e, &tot, lds16);
        if (e) empty[n_empty + pos] = (int)j;
        n_empty += tot;
    }
    const int64_t m = n_empty < n ? n_empty : n;

    // Distances are >= 0, so their IEEE bit patterns order like the values.
    // t = the largest 64-bit value with #{i : bits_i >= t} >= m, built bit by
    // bit from the top (the count only falls as t grows).
    unsigned long long t = 0;
    for (int bit = 63; bit >= 0; --bit) {
        const unsigned long long cand = t | (1ull << bit);
        long long c = 0;
        for (int64_t i = tid; i < n; i += 1024)
            c += (unsigned long long)__double_as_longlong(dist[i]) >= cand;
        if (block_count(c, lds16ll) >= m) t = cand;
    }
    long long g = 0;
    for (int64_t i = tid; i < n; i += 1024)
        g += (unsigned long long)__double_as_longlong(dist[i]) > t;
    const long long need_ties = m - block_count(g, lds16ll);

    // The m selected samples, compacted in sample order: all above t, and the
    // need_ties lowest-indexed ones equal to t.
    int sel = 0, ties = 0;
    for (int64_t base = 0; base < n; base += 1024) {
        const int64_t i = base + tid;
        const unsigned long long b =
            i < n ? (unsigned long long)__double_as_longlong(dist[i]) : 0ull;
        const bool eq = i < n && b == t;
        int eq_tot;
        const int eq_pos = block_flag_scan(eq, &eq_tot, lds16);
        const bool take = i < n && (b > t || (eq && ties + eq_pos < need_ties));
        int take_tot;
        const int pos = block_flag_scan(take, &take_tot, lds16);
        if (take) {
            sort_key[sel + pos] = b;
            sort_idx[sel + pos] = (int)i;
        }
        sel += take_tot;
        ties += eq_tot;
    }
    // Pad to a power of two with entries that sort last.
    int64_t p2 = 1;
    while (p2 < m) p2 <<= 1;
    for (int64_t i = m + tid; i < p2 && i < sort_cap; i += 1024) {
        sort_key[i] = 0ull;
        sort_idx[i] = 0x7fffffff;
    }
    __syncthreads();
    // Bitonic sort into "before" order.
    for (int64_t size = 2; size <= p2; size <<= 1) {
        for (int64_t stride = size >> 1; stride > 0; stride >>= 1) {
            for (int64_t i = tid; i < p2; i += 1024) {
                const int64_t j = i ^ stride;
                if (j > i) {
                    const bool ascending = (i & size) == 0;
                    const unsigned long long ki = sort_key[i], kj = sort_key[j];
                    const int ii = sort_idx[i], ij = sort_idx[j];
                    const bool swap = ascending ? before(kj, ij, ki, ii) : before(ki, ii, kj, ij);
                    if (swap) {
                        sort_key[i] = kj;
                        sort_key[j] = ki;
                        sort_idx[i] = ij;
                        sort_idx[j] = ii;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int64_t r = tid; r < m; r += 1024) {
        moves_src[r] = sort_idx[r];
        moves_dst[r] = empty[r];
    }
    if (tid == 0) *n_moves = (int)m;
}

__global__ __launch_bounds__(256) void reloc_apply_kernel(const int *__restrict__ n_moves,
                                                          const int *__restrict__ moves_src,
                                                          const int *__restrict__ moves_dst,
                                                          int64_t *__restrict__ labels) {
    const int m = *n_moves;
    for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < m; r += gridDim.x * blockDim.x)
        labels[moves_src[r]] = moves_dst[r];
}

// Sum of v over the block in a fixed order (each thread a fixed strided set,
// then a fixed tree).
__device__ double block_sum(double v, double *lds16) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) lds16[threadIdx.x >> 6] = v;
    __syncthreads();
    double t = 0.0;
    for (int w = 0; w < 16; ++w) t += lds16[w];
    __syncthreads();
    return t;
}

__global__ __launch_bounds__(1024) void shift_kernel(const double *__restrict__ partial,
                                                     int64_t blocks, double tol,
                                                     double *__restrict__ shift_out,
                                                     int *__restrict__ converged) {
    __shared__ double lds16[16];
    double s = 0.0;
    for (int64_t b = threadIdx.x; b < blocks; b += 1024) s += partial[b];
    const double tot = block_sum(s, lds16);
    if (threadIdx.x == 0) {
        *shift_out = tot;
        *converged = tot <= tol;
    }
}

__global__ __launch_bounds__(1024) void inertia_kernel(const float *__restrict__ min_dist,
                                                       int64_t n, double *__restrict__ out) {
    __shared__ double lds16[16];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 1024) s += (double)min_dist[i];
    const double tot = block_sum(s, lds16);
    if (threadIdx.x == 0) *out = tot;
}

__global__ __launch_bounds__(256) void copy_f32_kernel(float *__restrict__ dst,
                                                       const float *__restrict__ src,
                                                       int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
        dst[i] = src[i];
}

__global__ void store_f64_kernel(double *dst, double v) { *dst = v; }

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

int64_t reloc_sort_cap(int64_t n, int64_t k) {
    const int64_t m = n < k ? n : k;
    int64_t p2 = 1;
    while (p2 < m) p2 <<= 1;
    return p2;
}

hipError_t launch_relocate(const float *X, const float *C_old, int64_t *labels, int64_t n,
                           int64_t k, int64_t d, const RelocScratch &rs, const UpdateScratch &ws,
                           hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    reloc_dist_kernel<<<(unsigned)cdiv(n, 4), 256, 0, stream>>>(X, C_old, labels, n, d,
                                                                 rs.num_empty, rs.dist);
    reloc_select_kernel<<<1, 1024, 0, stream>>>(ws.cnt, k, n, rs.dist, rs.num_empty, rs.empty,
                                                rs.sort_key, rs.sort_idx, reloc_sort_cap(n, k),
                                                rs.moves_src, rs.moves_dst, rs.n_moves);
    int64_t b = cdiv(n < k ? n : k, 256);
    if (b > 1024) b = 1024;
    reloc_apply_kernel<<<(unsigned)b, 256, 0, stream>>>(rs.n_moves, rs.moves_src, rs.moves_dst,
                                                         labels);
    return hipGetLastError();
}

hipError_t launch_shift(const double *partial, int64_t blocks, double tol, double *shift_out,
                        int *converged, hipStream_t stream) {
    shift_kernel<<<1, 1024, 0, stream>>>(partial, blocks, tol, shift_out, converged);
    return hipGetLastError();
}

hipError_t launch_inertia(const float *min_dist, int64_t n, double *out, hipStream_t stream) {
    inertia_kernel<<<1, 1024, 0, stream>>>(min_dist, n, out);
    return hipGetLastError();
}

hipError_t launch_copy_f32(float *dst, const float *src, int64_t count, hipStream_t stream) {
    if (count <= 0 || dst == src) return hipSuccess;
    int64_t b = cdiv(count, 256);
    if (b > 8192) b = 8192;
    copy_f32_kernel<<<(unsigned)b, 256, 0, stream>>>(dst, src, count);
    return hipGetLastError();
}

hipError_t launch_store_f64(double *dst, double v, hipStream_t stream) {
    store_f64_kernel<<<1, 1, 0, stream>>>(dst, v);
    return hipGetLastError();
}

}  // namespace km
