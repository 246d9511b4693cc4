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
//   reloc_select_kernel  one block: list E, find the m-th largest distance by
//                        a radix select (8 bits a pass, from the top), compact
//                        the m farthest samples in sample order, sort them
//                        (bitonic) by distance descending then index
//                        ascending, and relabel the r-th to E[r]
//   shift_kernel         one block: centre shift = sum of the update's
//                        per-block partials, in block order; converged flag
//                        and the count of iterations run
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
                                                         double *__restrict__ dist, Gate gate) {
    if (gated(gate) || *num_empty == 0) return;  // uniform: nothing to relocate
    const int lane = threadIdx.x & 63;
    for (int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); i < n;
         i += (int64_t)gridDim.x * 4) {
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

// (key_a, idx_a) goes before (key_b, idx_b): larger distance first, then
// lower index.
__device__ __forceinline__ bool before(unsigned long long ka, int ia, unsigned long long kb,
                                       int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

__device__ __forceinline__ unsigned long long dist_bits(double v) {
    return (unsigned long long)__double_as_longlong(v);
}

constexpr int kSelWaves = 16;  // reloc_select_kernel: 1024 threads

__global__ __launch_bounds__(1024) void reloc_select_kernel(
    const int *__restrict__ cnt, int64_t k, int64_t n, const double *__restrict__ dist,
    const int *__restrict__ num_empty, int *__restrict__ empty, unsigned long long *sort_key,
    int *sort_idx, int64_t sort_cap, int64_t *__restrict__ labels, Gate gate) {
    __shared__ int lds16[16];
    __shared__ int hist[kSelWaves][256];
    __shared__ int bins[256];
    __shared__ int sel_digit, sel_above;
    __shared__ int wave_gt[kSelWaves], wave_eq[kSelWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (gated(gate) || *num_empty == 0) return;
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
    const int m = n_empty < n ? n_empty : (int)n;

    // Distances are >= 0, so their IEEE bit patterns order like the values.
    // t = the m-th largest bit pattern, one byte a pass from the top: among
    // the samples whose higher bytes equal t's, histogram the next byte (one
    // LDS histogram per wave), and take the largest byte value whose count
    // from the top reaches the rank still wanted. `remaining` ends as the
    // number of samples equal to t that belong to the m farthest.
    unsigned long long t = 0, known = 0;
    int remaining = m;
    for (int shift = 56; shift >= 0; shift -= 8) {
        for (int i = tid; i < kSelWaves * 256; i += 1024) (&hist[0][0])[i] = 0;
        __syncthreads();
        for (int64_t i = tid; i < n; i += 1024) {
            const unsigned long long b = dist_bits(dist[i]);
            if ((b & known) == t) atomicAdd(&hist[wave][(int)(b >> shift) & 255], 1);
        }
        __syncthreads();
        if (tid < 256) {
            int c = 0;
            for (int w = 0; w < kSelWaves; ++w) c += hist[w][tid];
            bins[tid] = c;
        }
        __syncthreads();
        if (wave == 0) {
            // Lane l holds bytes 4l..4l+3; S = count of bytes >= 4l.
            const int h0 = bins[4 * lane], h1 = bins[4 * lane + 1], h2 = bins[4 * lane + 2],
                      h3 = bins[4 * lane + 3];
            const int own = h0 + h1 + h2 + h3;
            int S = own;
            for (int off = 1; off < 64; off <<= 1) {
                const int o = __shfl_down(S, off);
                if (lane + off < 64) S += o;
            }
            // S falls with the lane and lane 0 holds every candidate, so the
            // lanes with S >= remaining are 0..L.
            const unsigned long long ok = __ballot(S >= remaining);
            const int L = 63 - __clzll(ok);
            if (lane == L) {
                int above = S - own;  // candidates with a byte above 4L + 3
                int digit = 4 * L;
                if (above + h3 >= remaining) {
                    digit += 3;
                } else {
                    above += h3;
                    if (above + h2 >= remaining) {
                        digit += 2;
                    } else {
                        above += h2;
                        if (above + h1 >= remaining) {
                            digit += 1;
                        } else {
                            above += h1;
                        }
                    }
                }
                sel_digit = digit;
                sel_above = above;
            }
        }
        __syncthreads();
        t |= (unsigned long long)sel_digit << shift;
        known |= 0xffull << shift;
        remaining -= sel_above;
    }
    const int need_ties = remaining;

    // The m selected samples, compacted in sample order: all above t and the
    // need_ties lowest-indexed ones equal to t. Each wave takes one contiguous
    // range of samples; a first sweep counts, a second writes.
    const int64_t per = (n + kSelWaves * 64 - 1) / (kSelWaves * 64) * 64;
    const int64_t lo = wave * per, hi = lo + per < n ? lo + per : n;
    const unsigned long long below = (1ull << lane) - 1ull;
    int gt = 0, eq = 0;
    for (int64_t base = lo; base < hi; base += 64) {
        const int64_t i = base + lane;
        const unsigned long long b = i < hi ? dist_bits(dist[i]) : 0ull;
        gt += __popcll(__ballot(i < hi && b > t));
        eq += __popcll(__ballot(i < hi && b == t));
    }
    if (lane == 0) {
        wave_gt[wave] = gt;
        wave_eq[wave] = eq;
    }
    __syncthreads();
    int out = 0, eq_seen = 0;
    for (int w = 0; w < wave; ++w) {
        out += wave_gt[w];
        eq_seen += wave_eq[w];
    }
    out += eq_seen < need_ties ? eq_seen : need_ties;
    for (int64_t base = lo; base < hi; base += 64) {
        const int64_t i = base + lane;
        const unsigned long long b = i < hi ? dist_bits(dist[i]) : 0ull;
        const bool is_eq = i < hi && b == t;
        const unsigned long long eq_mask = __ballot(is_eq);
        const bool take =
            i < hi && (b > t || (is_eq && eq_seen + (int)__popcll(eq_mask & below) < need_ties));
        const unsigned long long take_mask = __ballot(take);
        const int pos = out + __popcll(take_mask & below);
        if (take && pos < m) {
            sort_key[pos] = b;
            sort_idx[pos] = (int)i;
        }
        out += __popcll(take_mask);
        eq_seen += __popcll(eq_mask);
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
    // The r-th farthest sample becomes the only member of E[r].
    for (int64_t r = tid; r < m; r += 1024) {
        const int src = sort_idx[r];
        if (src >= 0 && src < n) labels[src] = empty[r];
    }
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

// One iteration's convergence check; once *converged is set it does nothing
// (kmeans_fit enqueues iterations in batches, and the ones after convergence
// are skipped by every kernel).
__global__ __launch_bounds__(1024) void shift_kernel(const double *__restrict__ partial,
                                                     int64_t blocks, double tol,
                                                     double *__restrict__ shift_out,
                                                     int *__restrict__ converged,
                                                     int *__restrict__ iterations) {
    __shared__ double lds16[16];
    if (*converged != 0) return;
    double s = 0.0;
    for (int64_t b = threadIdx.x; b < blocks; b += 1024) s += partial[b];
    const double tot = block_sum(s, lds16);
    if (threadIdx.x == 0) {
        *shift_out = tot;
        *converged = tot <= tol;
        *iterations += 1;
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

__global__ void store_count_kernel(double *dst, const int *count) { *dst = (double)*count; }

__global__ __launch_bounds__(256) void zero_i32_kernel(int *__restrict__ p, int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
        p[i] = 0;
}

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
                           hipStream_t stream, Gate gate) {
    if (n <= 0) return hipSuccess;
    int64_t b = cdiv(n, 4);
    if (b > 65536) b = 65536;
    reloc_dist_kernel<<<(unsigned)b, 256, 0, stream>>>(X, C_old, labels, n, d, rs.num_empty,
                                                       rs.dist, gate);
    reloc_select_kernel<<<1, 1024, 0, stream>>>(ws.cnt, k, n, rs.dist, rs.num_empty, rs.empty,
                                                rs.sort_key, rs.sort_idx, reloc_sort_cap(n, k),
                                                labels, gate);
    return hipGetLastError();
}

hipError_t launch_shift(const double *partial, int64_t blocks, double tol, double *shift_out,
                        int *converged, int *iterations, hipStream_t stream) {
    shift_kernel<<<1, 1024, 0, stream>>>(partial, blocks, tol, shift_out, converged, iterations);
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

hipError_t launch_store_count(double *dst, const int *count, hipStream_t stream) {
    store_count_kernel<<<1, 1, 0, stream>>>(dst, count);
    return hipGetLastError();
}

hipError_t launch_zero_i32(int *p, int64_t count, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    int64_t b = cdiv(count, 256);
    if (b > 1024) b = 1024;
    zero_i32_kernel<<<(unsigned)b, 256, 0, stream>>>(p, count);
    return hipGetLastError();
}

}  // namespace km
