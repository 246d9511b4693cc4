// assign.hip - nearest-centroid assignment on gfx950.
//
// Gram form ("Three shapes that fit an eager Gram assignment", section Gram
// assignment): ||x - c||^2 = ||x||^2 + ||c||^2 - 2 x.c. Inside the product the
// sample norm is dropped because it does not move the argmin ("004 - tile
// sizes ...", section Schedules added); centroid norms are computed once and
// reused by every sample tile.
//
// Kernels:
//   row_sqnorms_kernel  ||c_j||^2 (and ||x_i||^2 when min_dist is wanted)
//   fill_keys_kernel    packed-key identity
//   assign_tile_kernel  float32 MFMA product X_tile . C_tile^T, staged through
//                       LDS, with the distance, the argmin and the merge across
//                       centroid tiles done on the accumulators: the (n, k)
//                       distance matrix never exists in memory
//   finalize_kernel     packed key -> int64 label, full squared distance
#include "kernels.h"

namespace km {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ keys
//
// A (distance, index) pair is packed into one 64-bit key whose unsigned order
// is the lexicographic order (distance first, then index). The unsigned
// minimum over keys therefore keeps the smallest distance and, on an exact
// tie, the lowest index, whatever order the candidates arrive in: the merge
// across lanes, waves, tiles and blocks is order independent.

// Monotone map float -> uint32: a < b  <=>  ordered(a) < ordered(b).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    f = f + 0.0f;  // -0 becomes +0, so equal floats give equal keys
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unordered_bits(uint32_t u) {
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

__device__ __forceinline__ unsigned long long pack_key(float dist, uint32_t idx) {
    return ((unsigned long long)ordered_bits(dist) << 32) | idx;
}

// ------------------------------------------------------------- row norms

// One wave per row; float64 accumulation so the norm is the correctly
// rounded float32 of an almost exact sum (the centroid norm shifts a whole
// column of distances, so its error is not averaged away).
template <bool kVec>
__global__ __launch_bounds__(256) void row_sqnorms_kernel(const float *__restrict__ A,
                                                          int64_t rows, int64_t d,
                                                          float *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float *a = A + row * d;
    double s = 0.0;
    if (kVec) {
        for (int64_t t = 4 * (int64_t)lane; t < d; t += 256) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(a + t);
            s += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
        }
    } else {
        for (int64_t t = lane; t < d; t += 64) s += (double)a[t] * a[t];
    }
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) out[row] = (float)s;
}

__global__ __launch_bounds__(256) void fill_keys_kernel(unsigned long long *__restrict__ keys,
                                                        int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        keys[i] = ~0ull;
}

// ----------------------------------------------------- fused assignment
//
// Tile: kBM centroids x kBN samples, full depth d, 256 threads = 4 waves in a
// 2 x 2 arrangement, each wave owning 64 centroids x 64 samples = 2 x 2 MFMA
// blocks of 32 x 32 (v_mfma_f32_32x32x2_f32).
//
// Operand placement: the MFMA A operand (rows M) holds centroids and the B
// operand (columns N) holds samples. In the 32 x 32 result a lane owns one
// column, i.e. one sample, and 16 centroid rows, so most of the argmin is a
// scan of the lane's own accumulators; one exchange with the lane 32 apart
// (which holds the other rows of the same column) completes it.
//
// K order: a lane reads 4 consecutive features (one 16-byte LDS read) and
// feeds them to 4 successive MFMAs; lanes 0-31 and 32-63 read features 0-3 and
// 4-7 of each group of 8. A and B use the same feature permutation, so the
// product is the same dot product summed in a different order.
constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 32;
constexpr int kLDK = kBK + 4;   // padded LDS row: 16-byte reads of 32 lanes hit distinct banks
constexpr int kGroupM = 8;      // centroid tiles per rasterisation group

template <bool kVec>
__device__ __forceinline__ void load_stage(const float *__restrict__ X,
                                           const float *__restrict__ C, int64_t n, int64_t k,
                                           int64_t d, int64_t m0, int64_t n0, int64_t kbase,
                                           int tid, f32x4 (&r)[8]) {
    const int c4 = (tid & 7) * 4;
    const int64_t col = kbase + c4;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int row = (tid >> 3) + 32 * (q & 3);
        const int64_t g = (q < 4 ? m0 : n0) + row;
        const bool valid = g < (q < 4 ? k : n);
        const float *base = (q < 4 ? C : X) + (valid ? g : 0) * d;
        if (kVec) {
            if (valid && col < d)
                r[q] = *reinterpret_cast<const f32x4 *>(base + col);
            else
                r[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) r[q][e] = (valid && col + e < d) ? base[col + e] : 0.f;
        }
    }
}

__device__ __forceinline__ void store_stage(float (*lds)[kLDK], int tid, const f32x4 (&r)[8]) {
    const int c4 = (tid & 7) * 4;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int row = (tid >> 3) + 32 * (q & 3) + (q < 4 ? 0 : kBM);
        *reinterpret_cast<f32x4 *>(&lds[row][c4]) = r[q];
    }
}

template <bool kVec>
__global__ __launch_bounds__(256, 2) void assign_tile_kernel(
    const float *__restrict__ X, const float *__restrict__ C, const float *__restrict__ cn,
    int64_t n, int64_t k, int64_t d, int tiles_m, int tiles_n,
    unsigned long long *__restrict__ keys) {
    __shared__ float lds[2][kBM + kBN][kLDK];

    // Blocks are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8).
    // Renumber so that each XCD gets one contiguous range of tiles, then walk
    // that range in groups of kGroupM centroid tiles so that the tiles resident
    // on one XCD at a time share centroid and sample rows in its L2.
    const int nb = gridDim.x;
    const int bid = blockIdx.x;
    const int per = nb / 8, rem = nb % 8, xcd = bid % 8, local = bid / 8;
    const int linear = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + local;
    const int group_span = kGroupM * tiles_n;
    const int first_m = (linear / group_span) * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int tm = first_m + (linear % group_span) % gsize;
    const int tn = (linear % group_span) / gsize;
    const int64_t m0 = (int64_t)tm * kBM;
    const int64_t n0 = (int64_t)tn * kBN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;   // which 64 centroids of the tile
    const int wn = wave >> 1;  // which 64 samples of the tile

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int64_t nk = (d + kBK - 1) / kBK;
    f32x4 r[8];
    load_stage<kVec>(X, C, n, k, d, m0, n0, 0, tid, r);
    store_stage(lds[0], tid, r);
    __syncthreads();

    const int a_row = wm * 64 + (lane & 31);
    const int b_row = kBM + wn * 64 + (lane & 31);
    const int kofs = (lane >> 5) * 4;

    for (int64_t it = 0; it < nk; ++it) {
        const int cur = (int)(it & 1);
        if (it + 1 < nk) load_stage<kVec>(X, C, n, k, d, m0, n0, (it + 1) * kBK, tid, r);
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 8) {
            f32x4 a[2], b[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                a[mb] = *reinterpret_cast<const f32x4 *>(&lds[cur][a_row + 32 * mb][kk + kofs]);
#pragma unroll
            for (int nb2 = 0; nb2 < 2; ++nb2)
                b[nb2] = *reinterpret_cast<const f32x4 *>(&lds[cur][b_row + 32 * nb2][kk + kofs]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb2 = 0; nb2 < 2; ++nb2)
                        acc[mb][nb2] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            a[mb][e], b[nb2][e], acc[mb][nb2], 0, 0, 0);
        }
        if (it + 1 < nk) store_stage(lds[cur ^ 1], tid, r);
        __syncthreads();
    }

    // Epilogue. Accumulator element e of a 32 x 32 block sits at row
    // 8 * (e / 4) + 4 * (lane / 32) + e % 4 and column lane % 32.
    float cnv[2][16];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t m = m0 + wm * 64 + mb * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            cnv[mb][e] = m < k ? cn[m] : __builtin_inff();
        }
#pragma unroll
    for (int nb2 = 0; nb2 < 2; ++nb2) {
        // Rows are visited in increasing centroid index and only a strictly
        // smaller distance replaces the winner: lowest index on ties.
        float best = __builtin_inff();
        uint32_t bidx = 0xffffffffu;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t m = m0 + wm * 64 + mb * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const float v = cnv[mb][e] - 2.0f * acc[mb][nb2][e];
                if (m < k && v < best) {
                    best = v;
                    bidx = (uint32_t)m;
                }
            }
        unsigned long long key = pack_key(best, bidx);
        const unsigned long long other = __shfl_xor(key, 32);
        key = other < key ? other : key;
        const int64_t s = n0 + wn * 64 + nb2 * 32 + (lane & 31);
        if (lane < 32 && s < n) atomicMin(keys + s, key);
    }
}

__global__ __launch_bounds__(256) void finalize_kernel(unsigned long long *__restrict__ keys,
                                                       float *__restrict__ min_dist, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const unsigned long long key = keys[i];
        if (min_dist) {
            const float partial = unordered_bits((uint32_t)(key >> 32));
            min_dist[i] = fmaxf(min_dist[i] + partial, 0.0f);
        }
        keys[i] = key & 0xffffffffull;  // the int64 label
    }
}

inline bool vec_ok(const void *p, int64_t d) {
    return (d % 4 == 0) && ((uintptr_t)p % 16 == 0);
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline unsigned grid_stride_blocks(int64_t n) {
    int64_t b = cdiv(n, 256);
    if (b > 4096) b = 4096;
    if (b < 1) b = 1;
    return (unsigned)b;
}

}  // namespace

int64_t assign_grid_blocks(int64_t n, int64_t k) { return cdiv(n, kBN) * cdiv(k, kBM); }

hipError_t launch_row_sqnorms(const float *A, int64_t rows, int64_t d, float *out,
                              hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)cdiv(rows, 4);
    if (vec_ok(A, d))
        row_sqnorms_kernel<true><<<blocks, 256, 0, stream>>>(A, rows, d, out);
    else
        row_sqnorms_kernel<false><<<blocks, 256, 0, stream>>>(A, rows, d, out);
    return hipGetLastError();
}

hipError_t launch_fill_keys(unsigned long long *keys, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    fill_keys_kernel<<<grid_stride_blocks(n), 256, 0, stream>>>(keys, n);
    return hipGetLastError();
}

hipError_t launch_assign_tiles(const float *X, const float *C, const float *cn, int64_t n,
                               int64_t k, int64_t d, unsigned long long *keys,
                               hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int tiles_m = (int)cdiv(k, kBM);
    const int tiles_n = (int)cdiv(n, kBN);
    const unsigned blocks = (unsigned)((int64_t)tiles_m * tiles_n);
    if (vec_ok(X, d) && vec_ok(C, d))
        assign_tile_kernel<true><<<blocks, 256, 0, stream>>>(X, C, cn, n, k, d, tiles_m,
                                                             tiles_n, keys);
    else
        assign_tile_kernel<false><<<blocks, 256, 0, stream>>>(X, C, cn, n, k, d, tiles_m,
                                                              tiles_n, keys);
    return hipGetLastError();
}

hipError_t launch_finalize(unsigned long long *keys, float *min_dist, int64_t n,
                           hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    finalize_kernel<<<grid_stride_blocks(n), 256, 0, stream>>>(keys, min_dist, n);
    return hipGetLastError();
}

}  // namespace km
