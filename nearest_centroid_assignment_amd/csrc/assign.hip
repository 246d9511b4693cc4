// assign.hip - nearest-centroid assignment on gfx950.
//
// Gram form ("Three shapes that fit an eager Gram assignment", section Gram
// assignment): ||x - c||^2 = ||x||^2 + ||c||^2 - 2 x.c. Inside the product the
// sample norm is dropped because it does not move the argmin ("004 - tile
// sizes ...", section Schedules added); centroid norms are computed once and
// reused by every sample tile.
//
// Kernels:
//   row_sqnorms_kernel  ||c_j||^2 (and ||x_i||^2 for min_dist outside a Lloyd step)
//   fill_keys_kernel    packed-key identity
//   assign_dma_kernel   float32 MFMA product X_tile . C_tile^T in 256 x 256
//                       tiles (d a multiple of 4; edge tiles cut short where
//                       n or k is not a multiple of 256), the operands moved
//                       from global memory straight into LDS by buffer loads,
//                       with the distance, the argmin and the merge across
//                       centroid tiles done on the accumulators: the (n, k)
//                       distance matrix never exists in memory
//   assign_smallk_kernel  the same for small k: C resident in LDS, X read
//                       once, straight into 16 x 16 x 4 MFMAs, one key store
//                       per sample
//   assign_tile_kernel  the same for any shape, operands staged through
//                       registers into LDS, several tile sizes
//   finalize_kernel     packed key -> int64 label, full squared distance
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>

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
// column of distances, so its error is not averaged away). The rows are
// read once, with non-temporal loads, eight 16-byte loads of a lane issued
// before their adds (one load per trip left each trip waiting on memory:
// 49-65 us for 4096 rows of 16384 floats); the adds keep their order and
// each term its expression, so the sums are the same bits either way.
template <bool kVec>
__global__ __launch_bounds__(256) void row_sqnorms_kernel(const float *__restrict__ A,
                                                          int64_t rows, int64_t d,
                                                          float *__restrict__ out, Gate gate) {
    if (gated(gate)) return;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float *a = A + row * d;
    double s = 0.0;
    if (kVec) {
        constexpr int U = 8;  // loads in flight per lane
        int64_t t = 4 * (int64_t)lane;
        for (; t + (U - 1) * 256 < d; t += U * 256) {
            f32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a + t + u * 256));
#pragma unroll
            for (int u = 0; u < U; ++u)
                s += (double)v[u].x * v[u].x + (double)v[u].y * v[u].y +
                     (double)v[u].z * v[u].z + (double)v[u].w * v[u].w;
        }
        for (; t < d; t += 256) {
            const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a + t));
            s += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
        }
    } else {
        for (int64_t t = lane; t < d; t += 64) s += (double)a[t] * a[t];
    }
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) out[row] = (float)s;
}

__global__ __launch_bounds__(256) void fill_keys_kernel(unsigned long long *__restrict__ keys,
                                                        int64_t n, Gate gate) {
    if (gated(gate)) return;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        keys[i] = ~0ull;
}

// ----------------------------------------------------- fused assignment
//
// Tile: BM centroids x BN samples, full depth d. The block has WM x WN waves;
// each wave owns MB x NB blocks of 32 x 32 results computed with
// v_mfma_f32_32x32x2_f32 (BM = WM * MB * 32, BN = WN * NB * 32).
//
// Operand placement: the MFMA A operand (rows M) holds centroids and the B
// operand (columns N) holds samples. In a 32 x 32 result a lane owns one
// column, i.e. one sample, and 16 centroid rows, so most of the argmin is a
// scan of the lane's own accumulators; one exchange with the lane 32 apart
// (which holds the other rows of the same column) completes it.
//
// K order: a lane reads 4 consecutive features (one 16-byte LDS read) and
// feeds them to 4 successive MFMAs; lanes 0-31 and 32-63 read features 0-3 and
// 4-7 of each group of 8. A and B use the same feature permutation, so the
// product is the same dot product summed in a different order.
//
// Pipeline: features advance in stages of BK through two LDS buffers. At the
// start of stage s each thread reads the stage's first fragments, writes its
// registers (stage s + 1, loaded one stage earlier) into the free LDS buffer
// and issues the global loads of stage s + 2; the LDS writes and the loads
// then overlap the MFMAs of stage s. Inside a stage the fragments of the next
// group of 8 features are read from LDS while the current group's MFMAs run;
// the last group's MFMAs are deferred past the stage's barrier. One barrier
// per stage.
constexpr int kGroupM = 8;  // centroid tiles per rasterisation group

template <int WM_, int WN_, int MB_, int NB_, int BK_>
struct TileCfg {
    static constexpr int WM = WM_, WN = WN_, MB = MB_, NB = NB_;
    static constexpr int BM = WM * MB * 32;  // centroids per tile
    static constexpr int BN = WN * NB * 32;  // samples per tile
    static constexpr int BK = BK_;           // features per stage
    // Padded LDS row: the 16-byte reads of 16 consecutive rows hit distinct banks.
    static constexpr int LDK = BK + 4;
    static constexpr int kThreads = WM * WN * 64;
    static constexpr int kChunks = BK / 4;               // 16-byte chunks per row and stage
    static constexpr int kRows = BM + BN;                // LDS rows per stage
    static constexpr int kRowStep = kThreads / kChunks;  // rows covered by one pass of loads
    static constexpr int Q = kRows / kRowStep;           // 16-byte loads per thread per stage
    // The one-block-per-CU tiles (8 waves, up to 256 registers a lane) load
    // the epilogue's centroid norms before the last stages, so their latency
    // passes under MFMAs; the smaller tiles, bound to 168 or 128 registers,
    // load them after the last stage.
    static constexpr bool kEarlyNorms = BM * BN >= 128 * 256;
    static_assert(BK % 8 == 0 && kThreads % kChunks == 0, "bad stage depth");
    static_assert(kRows % kRowStep == 0, "tile rows must be a multiple of threads / chunks");
};

// Loading mode: kFull = every tile is full (n % BN == 0, k % BM == 0,
// d % BK == 0) and 16-byte aligned, no bounds checks; kVec = 16-byte loads
// with row / column checks; otherwise scalar loads with checks.
enum LoadMode { kScalar = 0, kVec = 1, kFull = 2 };

template <class Cfg, int Mode>
__device__ __forceinline__ void load_stage(const float *__restrict__ X,
                                           const float *__restrict__ C, int64_t n, int64_t k,
                                           int64_t d, int64_t m0, int64_t n0, int64_t kbase,
                                           int tid, f32x4 (&r)[Cfg::Q]) {
    const int c4 = (tid % Cfg::kChunks) * 4;
    const int64_t col = kbase + c4;
#pragma unroll
    for (int q = 0; q < Cfg::Q; ++q) {
        const int row = tid / Cfg::kChunks + Cfg::kRowStep * q;
        const bool is_c = row < Cfg::BM;
        const int64_t g = is_c ? m0 + row : n0 + (row - Cfg::BM);
        if (Mode == kFull) {
            r[q] = *reinterpret_cast<const f32x4 *>((is_c ? C : X) + g * d + col);
        } else {
            const bool valid = g < (is_c ? k : n);
            const float *base = (is_c ? C : X) + (valid ? g : 0) * d;
            if (Mode == kVec) {
                if (valid && col < d)
                    r[q] = *reinterpret_cast<const f32x4 *>(base + col);
                else
                    r[q] = f32x4{0.f, 0.f, 0.f, 0.f};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    r[q][e] = (valid && col + e < d) ? base[col + e] : 0.f;
            }
        }
    }
}

template <class Cfg>
__device__ __forceinline__ void store_stage(float (*lds)[Cfg::LDK], int tid,
                                            const f32x4 (&r)[Cfg::Q]) {
    const int c4 = (tid % Cfg::kChunks) * 4;
#pragma unroll
    for (int q = 0; q < Cfg::Q; ++q) {
        const int row = tid / Cfg::kChunks + Cfg::kRowStep * q;
        *reinterpret_cast<f32x4 *>(&lds[row][c4]) = r[q];
    }
}

// One stage of MFMAs: for each group of 8 features, every (mb, nb) block
// takes 4 MFMAs. The LDS->register fragments of the next group are read while
// the MFMAs of the current group run.
// Fragments of the first group of 8 features of a stage.
template <class Cfg>
__device__ __forceinline__ void first_frags(float (*lds)[Cfg::LDK], int lane, int wm, int wn,
                                            f32x4 (&a0)[Cfg::MB], f32x4 (&b0)[Cfg::NB]) {
    const int a_row = wm * Cfg::MB * 32 + (lane & 31);
    const int b_row = Cfg::BM + wn * Cfg::NB * 32 + (lane & 31);
    const int kofs = (lane >> 5) * 4;
#pragma unroll
    for (int mb = 0; mb < Cfg::MB; ++mb)
        a0[mb] = *reinterpret_cast<const f32x4 *>(&lds[a_row + 32 * mb][kofs]);
#pragma unroll
    for (int nb = 0; nb < Cfg::NB; ++nb)
        b0[nb] = *reinterpret_cast<const f32x4 *>(&lds[b_row + 32 * nb][kofs]);
}

// The MFMAs of one group of 8 features for every (mb, nb) block.
template <class Cfg>
__device__ __forceinline__ void mma_group(const f32x4 (&a)[Cfg::MB], const f32x4 (&b)[Cfg::NB],
                                          f32x16 (&acc)[Cfg::MB][Cfg::NB]) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int mb = 0; mb < Cfg::MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < Cfg::NB; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[mb][e], b[nb][e],
                                                                  acc[mb][nb], 0, 0, 0);
}

// Every group of a stage but the last: the fragments of the next group are
// read while the current group's MFMAs run. The last group's fragments are
// returned in aL / bL; its MFMAs run after the stage's barrier (mma_group),
// once the next stage's first reads have been issued.
template <class Cfg>
__device__ __forceinline__ void mma_head(float (*lds)[Cfg::LDK], int lane, int wm, int wn,
                                         const f32x4 (&a0)[Cfg::MB], const f32x4 (&b0)[Cfg::NB],
                                         f32x16 (&acc)[Cfg::MB][Cfg::NB], f32x4 (&aL)[Cfg::MB],
                                         f32x4 (&bL)[Cfg::NB]) {
    constexpr int G = Cfg::BK / 8;
    const int a_row = wm * Cfg::MB * 32 + (lane & 31);
    const int b_row = Cfg::BM + wn * Cfg::NB * 32 + (lane & 31);
    const int kofs = (lane >> 5) * 4;
    f32x4 a[2][Cfg::MB], b[2][Cfg::NB];
#pragma unroll
    for (int mb = 0; mb < Cfg::MB; ++mb) a[0][mb] = a0[mb];
#pragma unroll
    for (int nb = 0; nb < Cfg::NB; ++nb) b[0][nb] = b0[nb];
#pragma unroll
    for (int g = 0; g + 1 < G; ++g) {
        const int cur = g & 1;
#pragma unroll
        for (int mb = 0; mb < Cfg::MB; ++mb)
            a[cur ^ 1][mb] =
                *reinterpret_cast<const f32x4 *>(&lds[a_row + 32 * mb][8 * (g + 1) + kofs]);
#pragma unroll
        for (int nb = 0; nb < Cfg::NB; ++nb)
            b[cur ^ 1][nb] =
                *reinterpret_cast<const f32x4 *>(&lds[b_row + 32 * nb][8 * (g + 1) + kofs]);
        mma_group<Cfg>(a[cur], b[cur], acc);
    }
#pragma unroll
    for (int mb = 0; mb < Cfg::MB; ++mb) aL[mb] = a[(G - 1) & 1][mb];
#pragma unroll
    for (int nb = 0; nb < Cfg::NB; ++nb) bL[nb] = b[(G - 1) & 1][nb];
}

template <class Cfg, int Mode, int MinWaves, bool kPersistent>
__global__ __launch_bounds__(Cfg::kThreads, MinWaves) void assign_tile_kernel(
    const float *__restrict__ X, const float *__restrict__ C, const float *__restrict__ cn,
    int64_t n, int64_t k, int64_t d, int tiles_m, int tiles_n,
    unsigned long long *__restrict__ keys, const int *__restrict__ stop) {
    __shared__ float lds[2][Cfg::kRows][Cfg::LDK];
    if (stop != nullptr && *stop != 0) return;  // kmeans_fit: converged

    // Blocks are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8).
    // The tiles are renumbered so that each XCD gets one contiguous range of
    // them, walked in groups of kGroupM centroid tiles, so that the tiles
    // resident on one XCD at a time share centroid and sample rows in its L2.
    // Without kPersistent the grid has one block per tile and the loop below
    // runs once. With it (full tiles of the one-block-per-CU shapes) the grid
    // has at most one block per CU and each block takes every x_blocks-th
    // tile of its XCD's range: the same tiles run side by side on an XCD as
    // with one block per tile, and the per-block start-up and tear-down is
    // paid once per CU instead of once per tile. Tile counts fit an int: the
    // library rejects shapes whose launch grid would exceed 2^32 - 1
    // work-items, far fewer than 2^31 tiles.
    const int T = tiles_m * tiles_n;
    const int per = T / 8, rem = T % 8, xcd = blockIdx.x % 8;
    const int x_start = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
    const int x_count = per + (xcd < rem ? 1 : 0);
    const int x_blocks = ((int)gridDim.x - xcd + 7) / 8;  // blocks on this XCD
    const int group_span = kGroupM * tiles_n;
    for (int local = blockIdx.x / 8; !kPersistent || local < x_count; local += x_blocks) {
    const int linear = x_start + local;
    const int first_m = (linear / group_span) * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int tm = first_m + (linear % group_span) % gsize;
    const int tn = (linear % group_span) / gsize;
    const int64_t m0 = (int64_t)tm * Cfg::BM;
    const int64_t n0 = (int64_t)tn * Cfg::BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % Cfg::WM;  // which centroid rows of the tile
    const int wn = wave / Cfg::WM;  // which sample columns of the tile

    f32x16 acc[Cfg::MB][Cfg::NB];
#pragma unroll
    for (int i = 0; i < Cfg::MB; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::NB; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    constexpr int kBK = Cfg::BK;
    const int64_t nk = (d + kBK - 1) / kBK;
    // Two register sets carry the global loads: rA the odd stages, rB the
    // even ones (from stage 2 on), so each load has two stages to arrive.
    f32x4 rA[Cfg::Q], rB[Cfg::Q];
    load_stage<Cfg, Mode>(X, C, n, k, d, m0, n0, 0, tid, rA);
    store_stage<Cfg>(lds[0], tid, rA);
    if (nk > 1) load_stage<Cfg, Mode>(X, C, n, k, d, m0, n0, kBK, tid, rA);
    if (nk > 2) load_stage<Cfg, Mode>(X, C, n, k, d, m0, n0, 2 * kBK, tid, rB);
    __syncthreads();
    // Each stage's last group of MFMAs is deferred past the barrier into the
    // next stage, where it keeps the matrix cores busy while the next stage's
    // first fragments are read. Those reads are issued before the stage's LDS
    // writes, so the first MFMAs do not wait behind the writes. The main loop
    // takes two stages at a time (stage it even: lds[0] holds it, rA holds
    // it + 1, rB holds it + 2) and runs while both of its loads exist, so it
    // has no branch between those reads and the MFMAs (a branch there makes
    // the compiler wait for every LDS operation, writes included); the last
    // one to four stages follow. Before the first stage the pending group is
    // zeros: those MFMAs add exact zeros to the zero accumulators, and every
    // accumulator still sees its features in order.
    f32x4 aL[Cfg::MB], bL[Cfg::NB];
#pragma unroll
    for (int mb = 0; mb < Cfg::MB; ++mb) aL[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < Cfg::NB; ++nb) bL[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    int64_t it = 0;
    for (; it + 4 < nk; it += 2) {
        {
            f32x4 a0[Cfg::MB], b0[Cfg::NB];
            first_frags<Cfg>(lds[0], lane, wm, wn, a0, b0);
            mma_group<Cfg>(aL, bL, acc);
            store_stage<Cfg>(lds[1], tid, rA);
            load_stage<Cfg, Mode>(X, C, n, k, d, m0, n0, (it + 3) * kBK, tid, rA);
            // Keep the global loads here, ahead of the MFMAs: left alone, the
            // scheduler sinks them below the MFMAs to reuse registers.
            __builtin_amdgcn_sched_barrier(0);
            mma_head<Cfg>(lds[0], lane, wm, wn, a0, b0, acc, aL, bL);
            __syncthreads();
        }
        {
            f32x4 a0[Cfg::MB], b0[Cfg::NB];
            first_frags<Cfg>(lds[1], lane, wm, wn, a0, b0);
            mma_group<Cfg>(aL, bL, acc);
            store_stage<Cfg>(lds[0], tid, rB);
            load_stage<Cfg, Mode>(X, C, n, k, d, m0, n0, (it + 4) * kBK, tid, rB);
            __builtin_amdgcn_sched_barrier(0);
            mma_head<Cfg>(lds[1], lane, wm, wn, a0, b0, acc, aL, bL);
            __syncthreads();
        }
    }
    // Centroid norms of this wave's rows for the epilogue. Accumulator
    // element e of a 32 x 32 block sits at row 8 * (e / 4) + 4 * (lane / 32)
    // + e % 4 and column lane % 32.
    float cnv[Cfg::MB][16];
    if constexpr (Cfg::kEarlyNorms) {
#pragma unroll
        for (int mb = 0; mb < Cfg::MB; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t m =
                    m0 + (wm * Cfg::MB + mb) * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                cnv[mb][e] = m < k ? cn[m] : __builtin_inff();
            }
    }
    // The last 1 to 4 stages: it, it + 1, it + 2, it + 3 (it is even).
    {
        f32x4 a0[Cfg::MB], b0[Cfg::NB];
        first_frags<Cfg>(lds[0], lane, wm, wn, a0, b0);
        mma_group<Cfg>(aL, bL, acc);
        if (it + 1 < nk) store_stage<Cfg>(lds[1], tid, rA);
        if (it + 3 < nk) load_stage<Cfg, Mode>(X, C, n, k, d, m0, n0, (it + 3) * kBK, tid, rA);
        mma_head<Cfg>(lds[0], lane, wm, wn, a0, b0, acc, aL, bL);
        if (it + 1 < nk) __syncthreads();
    }
    if (it + 1 < nk) {
        f32x4 a0[Cfg::MB], b0[Cfg::NB];
        first_frags<Cfg>(lds[1], lane, wm, wn, a0, b0);
        mma_group<Cfg>(aL, bL, acc);
        if (it + 2 < nk) store_stage<Cfg>(lds[0], tid, rB);
        mma_head<Cfg>(lds[1], lane, wm, wn, a0, b0, acc, aL, bL);
        if (it + 2 < nk) __syncthreads();
    }
    if (it + 2 < nk) {
        f32x4 a0[Cfg::MB], b0[Cfg::NB];
        first_frags<Cfg>(lds[0], lane, wm, wn, a0, b0);
        mma_group<Cfg>(aL, bL, acc);
        if (it + 3 < nk) store_stage<Cfg>(lds[1], tid, rA);
        mma_head<Cfg>(lds[0], lane, wm, wn, a0, b0, acc, aL, bL);
        if (it + 3 < nk) __syncthreads();
    }
    if (it + 3 < nk) {
        f32x4 a0[Cfg::MB], b0[Cfg::NB];
        first_frags<Cfg>(lds[1], lane, wm, wn, a0, b0);
        mma_group<Cfg>(aL, bL, acc);
        mma_head<Cfg>(lds[1], lane, wm, wn, a0, b0, acc, aL, bL);
    }
    mma_group<Cfg>(aL, bL, acc);

    // Epilogue.
    if constexpr (!Cfg::kEarlyNorms) {
#pragma unroll
        for (int mb = 0; mb < Cfg::MB; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t m =
                    m0 + (wm * Cfg::MB + mb) * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                cnv[mb][e] = m < k ? cn[m] : __builtin_inff();
            }
    }
#pragma unroll
    for (int nb = 0; nb < Cfg::NB; ++nb) {
        // Rows are visited in increasing centroid index and only a strictly
        // smaller distance replaces the winner: lowest index on ties. The
        // winner starts as the lane's first (lowest) valid centroid at +inf,
        // so a lane whose candidates are all +inf or NaN (a norm that
        // overflows float32) still names a centroid in [0, k): +inf ties go
        // to the lowest index like any other tie, and NaN never wins.
        const int64_t m_first = m0 + wm * Cfg::MB * 32 + 4 * (lane >> 5);
        float best = __builtin_inff();
        uint32_t bidx = m_first < k ? (uint32_t)m_first : 0xffffffffu;
#pragma unroll
        for (int mb = 0; mb < Cfg::MB; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t m =
                    m0 + (wm * Cfg::MB + mb) * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const float v = cnv[mb][e] - 2.0f * acc[mb][nb][e];
                if (m < k && v < best) {
                    best = v;
                    bidx = (uint32_t)m;
                }
            }
        unsigned long long key = pack_key(best, bidx);
        const unsigned long long other = __shfl_xor(key, 32);
        key = other < key ? other : key;
        const int64_t s = n0 + (wn * Cfg::NB + nb) * 32 + (lane & 31);
        if (lane < 32 && s < n) atomicMin(keys + s, key);
    }
    if (!kPersistent) break;
    __syncthreads();  // the next tile's LDS writes follow these reads
    }
}

// ------------------------------------------------ DMA-staged 256 x 256 tiles
//
// 16-byte aligned rows of d % 4 == 0 floats, any n and k (the ragged
// instances read only the rows below n and k and skip the rest, and the
// any-d one also zeroes a partial last stage past d). 8 waves in 2 x 4; each wave owns 128 centroids x 64 samples (4 x 2
// blocks of 32 x 32), so a fragment read from LDS feeds more MFMAs than in
// the 128 x 256 tile (6 reads per 32 MFMAs instead of 4 per 16), a stage
// holds twice the MFMAs per barrier, and the 128 accumulators per lane fit
// because the operands never pass through registers: buffer loads with the
// LDS bit move them from global memory straight into LDS (16 bytes per lane;
// lane i of an instruction writes the 16 bytes at its LDS base + 16 i), one
// stage ahead. The buffer form, not global_load_lds, because the compiler
// treats a pending global (FLAT) LDS load as both a memory and an LDS access
// and then waits for every outstanding LDS read (lgkmcnt(0)) before using
// any fragment; with buffer loads it waits only for the reads it needs.
// LDS rows are 32 floats, unpadded (two 64 KiB stage buffers); the 16-byte
// chunks of a row are XOR-swizzled so that the fragment reads of
// consecutive rows hit distinct banks.
namespace dma {
constexpr int BM = 256, BN = 256, BK = 32, ROWS = BM + BN;
constexpr int WM = 2, WN = 4, MB = 4, NB = 2, NT = WM * WN * 64;
constexpr int SLOTS = ROWS * (BK / 4);           // 16-byte slots per stage
constexpr int PER_WAVE = SLOTS / NT;             // DMA instructions per wave and stage
static_assert(PER_WAVE * NT == SLOTS, "slots must split evenly over the threads");
// Chunk swizzle: rows 2r and 2r + 1 share one, consecutive pairs differ, so
// the 16-byte fragment reads of 16 consecutive rows cover all 64 banks once
// (measured: no bank conflicts; the row % 8 swizzle conflicts, which shows
// the 64 banks).
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
}  // namespace dma

// One stage of this wave's DMA: instruction j moves 64 slots (8 rows x 8
// chunks) into buf + (wave * PER_WAVE + j) * 64 slots. voff[p] is the lane's
// byte offset inside the wave's source block for instructions of parity p
// (the swizzled chunk alternates with j). The offset of the instruction's
// rows (j * row_bytes8) goes with the uniform part, except in ragged tiles:
// there it joins the lane's offset, which the buffer's range check covers
// (the uniform offset may not be checked), so that every row past the
// buffer's last record reads as zero instead of touching memory.
template <bool kRagged>
__device__ __forceinline__ void dma_stage(__amdgpu_buffer_rsrc_t rsrc, const int (&voff)[2],
                                          int row_bytes8, int kbytes, float *buf, int wave) {
#pragma unroll
    for (int j = 0; j < dma::PER_WAVE; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void *)(buf + (wave * dma::PER_WAVE + j) * 64 * 4),
            16, kRagged ? voff[j & 1] + j * row_bytes8 : voff[j & 1],
            kRagged ? kbytes : j * row_bytes8 + kbytes, 0, 0);
}

// Zeros the 16-byte chunks from `valid` on of every row of a stage buffer
// (thread t: row t), so that a stage that ends inside the rows contributes
// nothing past the last feature, whatever its DMA left there.
__device__ __forceinline__ void dma_zero_tail(float *buf, int valid, int tid) {
    static_assert(dma::NT == dma::ROWS, "one thread per stage row");
    for (int c = valid; c < dma::BK / 4; ++c)
        *reinterpret_cast<f32x4 *>(buf + tid * dma::BK + ((c ^ dma::swz(tid)) << 2)) =
            f32x4{0.f, 0.f, 0.f, 0.f};
}

// Fragments of group g (features 8g .. 8g + 7) for this lane: A rows
// a_base + 32 mb, B rows b_base + 32 nb, chunk 2g + lane / 32 swizzled.
__device__ __forceinline__ void dma_frags(const float *buf, int a_base, int b_base, int lane, int g,
                                          f32x4 (&a)[dma::MB], f32x4 (&b)[dma::NB]) {
    const int h = lane >> 5;
#pragma unroll
    for (int mb = 0; mb < dma::MB; ++mb) {
        const int row = a_base + 32 * mb;
        a[mb] = *reinterpret_cast<const f32x4 *>(buf + row * dma::BK +
                                                 (((2 * g + h) ^ dma::swz(row)) << 2));
    }
#pragma unroll
    for (int nb = 0; nb < dma::NB; ++nb) {
        const int row = b_base + 32 * nb;
        b[nb] = *reinterpret_cast<const f32x4 *>(buf + row * dma::BK +
                                                 (((2 * g + h) ^ dma::swz(row)) << 2));
    }
}

__device__ __forceinline__ void dma_mma(const f32x4 (&a)[dma::MB], const f32x4 (&b)[dma::NB],
                                        f32x16 (&acc)[dma::MB][dma::NB]) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int mb = 0; mb < dma::MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < dma::NB; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[mb][e], b[nb][e],
                                                                  acc[mb][nb], 0, 0, 0);
}

// One stage read from buf while this wave's share of the next stage moves
// into dst: the deferred group of the previous stage, then groups 0 .. 2 of
// this one with the next group's fragments read ahead; the fragments of
// group 3 are left in aL / bL for the next stage. The eight DMA instructions
// are spread over the deferred group's MFMAs, one per four: issued back to
// back, all 64 of a CU queue at the texture unit right after the barrier and
// hold up the MFMAs behind them.
template <bool kRagged>
__device__ __forceinline__ void dma_compute(const float *buf, float *dst, __amdgpu_buffer_rsrc_t rsrc,
                                            const int (&voff)[2], int row_bytes8, int kbytes, int wave,
                                            int a_base, int b_base, int lane,
                                            f32x4 (&aL)[dma::MB], f32x4 (&bL)[dma::NB],
                                            f32x16 (&acc)[dma::MB][dma::NB]) {
    f32x4 a[2][dma::MB], b[2][dma::NB];
    dma_frags(buf, a_base, b_base, lane, 0, a[0], b[0]);
    dma_stage<kRagged>(rsrc, voff, row_bytes8, kbytes, dst, wave);
    dma_mma(aL, bL, acc);
#pragma unroll
    for (int g = 0; g < 3; ++g) {
        dma_frags(buf, a_base, b_base, lane, g + 1, a[(g + 1) & 1], b[(g + 1) & 1]);
        dma_mma(a[g & 1], b[g & 1], acc);
    }
    // Order: group 0's fragment reads, the deferred MFMAs with a DMA
    // instruction after every fourth, then the fragment reads of group g + 1
    // ahead of the MFMAs of group g.
    __builtin_amdgcn_sched_group_barrier(0x100, dma::MB + dma::NB, 0);
#pragma unroll
    for (int j = 0; j < dma::PER_WAVE; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * dma::MB * dma::NB / dma::PER_WAVE, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
#pragma unroll
    for (int g = 0; g < 3; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x100, dma::MB + dma::NB, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * dma::MB * dma::NB, 0);
    }
#pragma unroll
    for (int mb = 0; mb < dma::MB; ++mb) aL[mb] = a[1][mb];
#pragma unroll
    for (int nb = 0; nb < dma::NB; ++nb) bL[nb] = b[1][nb];
}

// The kernel's instances: whole tiles and pairs of stages; edge tiles cut
// short, still pairs of stages; anything else (edge tiles, any number of
// stages, a partial last one).
enum DmaMode { kDmaFull = 0, kDmaRagged = 1, kDmaAnyD = 2 };

template <int kMode>
__global__ __launch_bounds__(dma::NT, 2) void assign_dma_kernel(
    const float *__restrict__ X, const float *__restrict__ C, const float *__restrict__ cn,
    int64_t n, int64_t k, int64_t d, int tiles_m, int tiles_n,
    unsigned long long *__restrict__ keys, const int *__restrict__ stop) {
    __shared__ __align__(16) float buf0[dma::ROWS * dma::BK];
    __shared__ __align__(16) float buf1[dma::ROWS * dma::BK];
    if (stop != nullptr && *stop != 0) return;  // kmeans_fit: converged
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % dma::WM, wn = wave / dma::WM;
    const int a_base = wm * dma::MB * 32 + (lane & 31);
    const int b_base = dma::BM + wn * dma::NB * 32 + (lane & 31);
    constexpr bool kRagged = kMode != kDmaFull;
    constexpr bool kAnyD = kMode == kDmaAnyD;
    const int64_t nk = kAnyD ? (d + dma::BK - 1) / dma::BK : d / dma::BK;  // stages (even unless kAnyD)
    // 16-byte chunks of features in the last stage (8: a whole stage).
    const int tail_chunks = (int)(d - (nk - 1) * dma::BK) / 4;
    // Tile counts fit an int: the library rejects shapes whose launch grid
    // would exceed 2^32 - 1 work-items, far fewer than 2^31 tiles.
    const int T = tiles_m * tiles_n;
    const int per = T / 8, rem = T % 8, xcd = blockIdx.x % 8;
    const int x_start = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
    const int x_count = per + (xcd < rem ? 1 : 0);
    const int x_blocks = ((int)gridDim.x - xcd + 7) / 8;
    const int group_span = kGroupM * tiles_n;
    for (int local = blockIdx.x / 8; local < x_count; local += x_blocks) {
        const int linear = x_start + local;
        const int first_m = (linear / group_span) * kGroupM;
        const int gsize = min(tiles_m - first_m, kGroupM);
        // (the division by gsize runs on the vector unit: the tile indices
        // go back to scalar registers, where the descriptors need them)
        const int64_t m0 =
            (int64_t)__builtin_amdgcn_readfirstlane(first_m + (linear % group_span) % gsize) * dma::BM;
        const int64_t n0 = (int64_t)__builtin_amdgcn_readfirstlane((linear % group_span) / gsize) * dma::BN;
        // This wave's DMA source: waves 0-3 copy centroid rows, 4-7 sample
        // rows, 64 rows each. Slot s of the wave's block is row s / 8 of it,
        // stored chunk s % 8, which holds logical chunk (s % 8) ^ swz(row);
        // with the (row / 2) % 8 swizzle that is (lane % 8) ^ (lane / 16),
        // flipped by 4 on odd instructions.
        // In ragged tiles the buffer holds only the block's rows below k (or
        // n), none for a block wholly past them (its base then stays at row 0
        // of the matrix): the rows beyond read as zeros, or leave stale LDS,
        // and reach only accumulators of centroids and samples that the
        // epilogue skips.
        const int half = wave / (dma::PER_WAVE / 2);  // 0: centroids, 1: samples
        const int64_t b0 = (half == 0 ? m0 : n0) + (wave % 4) * 64;
        int blk_rows = 64;
        if (kRagged) {
            // (clamped in 64 bits, which only the vector unit compares; the
            // result goes back to a scalar register, where the descriptor
            // must live)
            const int64_t left = (half == 0 ? k : n) - b0;
            blk_rows = __builtin_amdgcn_readfirstlane((int)(left < 0 ? 0 : left < 64 ? left : 64));
        }
        const float *blk = (half == 0 ? C : X) + (blk_rows > 0 ? b0 : 0) * d;
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void *)blk, 0, (int)(blk_rows * d * 4), 0x00020000);
        const int c0 = (lane & 7) ^ (lane >> 4);
        const int voff[2] = {(int)((lane >> 3) * d * 4 + c0 * 16),
                             (int)((lane >> 3) * d * 4 + (c0 ^ 4) * 16)};
        const int row_bytes8 = (int)(8 * d * 4);
        // The last stage of a ragged tile may end inside the rows: there the
        // lanes whose chunk lies past d take an offset of 2^31, beyond any
        // buffer's records, so they touch no memory (also where the uniform
        // offset is left out of the range check: the row's end can be the
        // matrix's). Their LDS slots are zeroed once the stage has landed.
        int voff_t[2] = {voff[0], voff[1]};
        if (kAnyD) {
#pragma unroll
            for (int p = 0; p < 2; ++p)
                if ((c0 ^ (4 * p)) >= tail_chunks) voff_t[p] = (int)0x80000000u;
        }
        f32x16 acc[dma::MB][dma::NB];
#pragma unroll
        for (int i = 0; i < dma::MB; ++i)
#pragma unroll
            for (int j = 0; j < dma::NB; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
        f32x4 aL[dma::MB], bL[dma::NB];
#pragma unroll
        for (int mb = 0; mb < dma::MB; ++mb) aL[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nb = 0; nb < dma::NB; ++nb) bL[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

        if constexpr (!kAnyD) {
            dma_stage<kRagged>(rsrc, voff, row_bytes8, 0, buf0, wave);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            // Two stages per iteration: stage s from buf0 while s + 1 lands in
            // buf1, then stage s + 1 from buf1 while s + 2 lands in buf0 (on
            // the last iteration that load repeats stage s + 1 into buf0,
            // which no one reads any more; it completes before the tile's
            // final barrier).
            for (int64_t s = 0; s < nk; s += 2) {
                dma_compute<kRagged>(buf0, buf1, rsrc, voff, row_bytes8, (int)((s + 1) * dma::BK * 4),
                                     wave, a_base, b_base, lane, aL, bL, acc);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                const int64_t s2 = s + 2 < nk ? s + 2 : s + 1;
                dma_compute<kRagged>(buf1, buf0, rsrc, voff, row_bytes8, (int)(s2 * dma::BK * 4), wave,
                                     a_base, b_base, lane, aL, bL, acc);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            }
        } else {
            // One stage per iteration (any number of them), the buffers
            // alternating: stage s from one while stage s + 1 lands in the
            // other (the last iteration repeats stage s, which no one reads).
            // A partial last stage loads with the tail offsets and is zeroed
            // past d before anyone reads it. (Two stages per iteration with
            // the odd and partial cases around them ran 1-5 % slower: the
            // extra branches pushed the kernel past its registers.)
            const bool partial = tail_chunks < dma::BK / 4;
            dma_stage<true>(rsrc, partial && nk == 1 ? voff_t : voff, row_bytes8, 0, buf0, wave);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (partial && nk == 1) {
                dma_zero_tail(buf0, tail_chunks, tid);
                __syncthreads();
            }
            for (int64_t s = 0; s < nk; ++s) {
                float *cur = (s & 1) ? buf1 : buf0;
                float *nxt = (s & 1) ? buf0 : buf1;
                const int64_t sn = s + 1 < nk ? s + 1 : s;
                const bool tail_next = partial && sn == nk - 1;
                dma_compute<true>(cur, nxt, rsrc, tail_next ? voff_t : voff, row_bytes8,
                                  (int)(sn * dma::BK * 4), wave, a_base, b_base, lane, aL, bL, acc);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (tail_next && s + 1 < nk) {
                    dma_zero_tail(nxt, tail_chunks, tid);
                    __syncthreads();
                }
            }
        }
        dma_mma(aL, bL, acc);

        // Epilogue, as in assign_tile_kernel, one block of 32 centroid rows at
        // a time (16 norms live instead of 64); rows are still visited in
        // increasing index for each sample, strict less-than keeps the lowest.
        // The winner starts as the lane's first centroid at +inf (as in
        // assign_tile_kernel: all-+inf or NaN candidates still give a valid
        // index, the lowest one).
        float best[dma::NB];
        uint32_t bidx[dma::NB];
        if constexpr (!kRagged) {
#pragma unroll
            for (int nb = 0; nb < dma::NB; ++nb) {
                best[nb] = __builtin_inff();
                bidx[nb] = (uint32_t)(m0 + wm * dma::MB * 32 + 4 * (lane >> 5));
            }
#pragma unroll
            for (int mb = 0; mb < dma::MB; ++mb) {
                float cnv[16];
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    cnv[e] = cn[m0 + (wm * dma::MB + mb) * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)];
#pragma unroll
                for (int nb = 0; nb < dma::NB; ++nb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int64_t m = m0 + (wm * dma::MB + mb) * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                        const float v = cnv[e] - 2.0f * acc[mb][nb][e];
                        if (v < best[nb]) {
                            best[nb] = v;
                            bidx[nb] = (uint32_t)m;
                        }
                    }
            }
        } else {
            // Ragged tiles skip the centroids from k on: their norm is taken
            // as NaN (read at a clamped index, so every load stays
            // unconditional), which never wins a strict less-than. A lane with
            // no centroid below k starts from an index that every real
            // candidate beats. Rows are counted from the tile's first one,
            // starting from an offset the compiler cannot see through, so it
            // forms the 64 per-element rows here rather than hoisting them out
            // of the tile loop (where they spill).
            int r0 = wm * dma::MB * 32 + 4 * (lane >> 5);
            asm volatile("" : "+v"(r0));
            const int lim = __builtin_amdgcn_readfirstlane(
                (int)(k - m0 < dma::BM ? k - m0 : dma::BM));  // rows of this tile below k
#pragma unroll
            for (int nb = 0; nb < dma::NB; ++nb) {
                best[nb] = __builtin_inff();
                bidx[nb] = r0 < lim ? (uint32_t)(m0 + r0) : 0xffffffffu;
            }
#pragma unroll
            for (int mb = 0; mb < dma::MB; ++mb) {
                float cnv[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int r = r0 + mb * 32 + 8 * (e >> 2) + (e & 3);
                    const float c = cn[m0 + (r < lim ? r : lim - 1)];
                    cnv[e] = r < lim ? c : __builtin_nanf("");
                }
#pragma unroll
                for (int nb = 0; nb < dma::NB; ++nb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int r = r0 + mb * 32 + 8 * (e >> 2) + (e & 3);
                        const float v = cnv[e] - 2.0f * acc[mb][nb][e];
                        if (v < best[nb]) {
                            best[nb] = v;
                            bidx[nb] = (uint32_t)(m0 + r);
                        }
                    }
            }
        }
#pragma unroll
        for (int nb = 0; nb < dma::NB; ++nb) {
            unsigned long long key = pack_key(best[nb], bidx[nb]);
            const unsigned long long other = __shfl_xor(key, 32);
            key = other < key ? other : key;
            const int64_t smp = n0 + (wn * dma::NB + nb) * 32 + (lane & 31);
            if (lane < 32 && (!kRagged || smp < n)) atomicMin(keys + smp, key);
        }
        __syncthreads();  // the next tile's first DMA follows this tile's reads
    }
}

// ------------------------------------------------ small k: C resident in LDS
//
// k <= 128 (up to eight 16-row blocks): the whole of C sits in LDS for the life of a block (rows rounded
// up to 16, features to 64, zero-padded), and each wave streams groups of 16
// samples of X from global memory straight into the B operand of
// v_mfma_f32_16x16x4f32, so the kernel reads X once, at HBM speed, where a
// 128- or 256-row centroid tile would repeat mostly-padding MFMAs for every
// sample tile. Operand layout (probed on the chip): lane l holds A[l % 16]
// [l / 16] and B[l / 16][l % 16], and value i of lane l receives D[4 (l / 16)
// + i][l % 16]. With A = 16 centroid rows and B = 16 samples, lane (g = l /
// 16, r = l % 16) feeds feature 16 q + 4 g + e of step (q, e) for both, so
// one 16-byte load of row r gives four steps, and ends with sample r against
// rows 4 g .. 4 g + 3 of each 16-row block. Every sample's key is stored once
// (one pass covers all centroids): no atomics, no identity fill.
namespace sk {
constexpr int kWaves = 8;          // waves per block
constexpr int kLdsFloats = 16384;  // C's LDS budget: 64 KiB (two blocks per CU)
constexpr int kChunk = 64;         // features per load: four 16-byte loads per lane
}  // namespace sk

// Floats per LDS row of C: d rounded up to 64 plus 4, so that the 16-byte
// reads of 16 consecutive rows (one per lane) fall on distinct banks.
__host__ __device__ inline int64_t sk_ld(int64_t d) { return (d + sk::kChunk - 1) / sk::kChunk * sk::kChunk + 4; }

template <int KB, int NCB>
__global__ __launch_bounds__(sk::kWaves * 64) void assign_smallk_kernel(
    const float *__restrict__ X, const float *__restrict__ C, const float *__restrict__ cn,
    int64_t n, int64_t k, int64_t d, unsigned long long *__restrict__ keys,
    const int *__restrict__ stop) {
    extern __shared__ __align__(16) float cs[];  // 16 KB rows of sk_ld(d) floats
    if (stop != nullptr && *stop != 0) return;  // kmeans_fit: converged
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r = lane & 15;
    const int64_t ld = sk_ld(d), q4 = (ld - 4) / 4;  // 16-byte chunks per padded row
    // C into LDS: rows from k on and features from d on are zeros.
    for (int64_t e = tid; e < 16 * KB * q4; e += sk::kWaves * 64) {
        const int64_t row = e / q4, c = 4 * (e % q4);
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (row < k && c < d) v = *reinterpret_cast<const f32x4 *>(C + row * d + c);
        *reinterpret_cast<f32x4 *>(cs + row * ld + c) = v;
    }
    // Norms of this lane's rows 16 kb + 4 g + i; NaN from k on, which never
    // wins a strict less-than.
    float cnv[KB][4];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t j = 16 * kb + 4 * g + i;
            const float t = cn[j < k ? j : k - 1];
            cnv[kb][i] = j < k ? t : __builtin_nanf("");
        }
    __syncthreads();  // the last barrier: waves run on their own from here

    // C's rows as 16-byte units (ld is a multiple of 4), so that the A
    // operands are read 16 bytes at a time.
    const f32x4 *cs4 = reinterpret_cast<const f32x4 *>(cs);
    const int64_t ld4 = ld / 4;
    const int64_t groups = (n + 15) / 16;
    const int64_t stride = (int64_t)gridDim.x * sk::kWaves;
    const int64_t nc = (d + sk::kChunk - 1) / sk::kChunk;  // 64-feature chunks
    // Each group's loads are issued together, NCB chunks (up to 256
    // features) at a time, and used in the same iteration: the latency is
    // covered by the other waves of the CU (up to 32), not by a prefetch
    // carried from one iteration to the next (the compiler then waits for
    // the prefetched loads at the top of each iteration).
    for (int64_t grp = (int64_t)blockIdx.x * sk::kWaves + wave; grp < groups; grp += stride) {
        const int64_t s = grp * 16 + r;
        const float *row = X + (s < n ? s : n - 1) * d;
        f32x4 acc[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int64_t c0 = 0; c0 < nc; c0 += NCB) {
            // Chunk c: features 64 c + 16 q + 4 g; past d zeros, read at a
            // clamped address so that every load is unconditional. Ordinary
            // loads, not non-temporal ones: an instruction reads half of
            // each row's 128-byte line (4 lanes x 16 bytes) and the next one
            // the other half, which then comes from the cache (measured:
            // 45.8 against 54.4 us at 1M x 16 x 64).
            f32x4 x[NCB][4];
#pragma unroll
            for (int b = 0; b < NCB; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t f = (c0 + b) * sk::kChunk + 16 * q + 4 * g;
                    const f32x4 t = *reinterpret_cast<const f32x4 *>(row + (f < d ? f : 0));
                    x[b][q] = f < d ? t : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            // All of the batch's loads first (left alone, the scheduler
            // moves each next to its products and the loads run one by one).
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < NCB; ++b) {
                // (chunks past the last one read column 0 of C: their x is 0)
                const int64_t cc = c0 + b < nc ? c0 + b : 0;
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const f32x4 a = cs4[(16 * kb + r) * ld4 + cc * (sk::kChunk / 4) + 4 * q + g];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], x[b][q][e], acc[kb], 0, 0, 0);
                    }
            }
        }
        // Rows in increasing index per lane, strict less-than: the lowest
        // index on ties, then the packed-key minimum over the four lane
        // groups (which also prefers the lower index).
        float best = __builtin_inff();
        uint32_t bidx = 4 * g < k ? (uint32_t)(4 * g) : 0xffffffffu;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = cnv[kb][i] - 2.0f * acc[kb][i];
                if (v < best) {
                    best = v;
                    bidx = (uint32_t)(16 * kb + 4 * g + i);
                }
            }
        unsigned long long key = pack_key(best, bidx);
        unsigned long long other = __shfl_xor(key, 16);
        key = other < key ? other : key;
        other = __shfl_xor(key, 32);
        key = other < key ? other : key;
        if (g == 0 && s < n) keys[s] = key;
    }
}

// Tile shapes (centroids x samples; the launcher picks one by problem shape).
using Tile128x256 = TileCfg<2, 4, 2, 2, 32>;  // 512 threads, 108 KiB LDS, 1 block per CU
using Tile256x128 = TileCfg<4, 2, 2, 2, 32>;  // 512 threads, 108 KiB LDS, 1 block per CU
using Tile128x128 = TileCfg<2, 2, 2, 2, 16>;  // 256 threads, 40 KiB LDS, 3 blocks per CU
using Tile64x64 = TileCfg<2, 2, 1, 1, 32>;    // 256 threads, 36 KiB LDS, small problems

// The epilogues always name a centroid in [0, k) (see there); the clamp keeps
// every later index into C, the counts and the grouping in bounds even if a
// key were never lowered.
__global__ __launch_bounds__(256) void finalize_kernel(unsigned long long *__restrict__ keys,
                                                       float *__restrict__ min_dist,
                                                       bool add_norm, int64_t n, int64_t k) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const unsigned long long key = keys[i];
        if (min_dist) {
            const float partial = unordered_bits((uint32_t)(key >> 32));
            min_dist[i] = add_norm ? fmaxf(min_dist[i] + partial, 0.0f) : partial;
        }
        const unsigned long long idx = key & 0xffffffffull;
        keys[i] = idx < (unsigned long long)k ? idx : 0ull;  // the int64 label
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


hipError_t launch_row_sqnorms(const float *A, int64_t rows, int64_t d, float *out,
                              hipStream_t stream, Gate gate) {
    if (rows <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)cdiv(rows, 4);
    if (vec_ok(A, d))
        row_sqnorms_kernel<true><<<blocks, 256, 0, stream>>>(A, rows, d, out, gate);
    else
        row_sqnorms_kernel<false><<<blocks, 256, 0, stream>>>(A, rows, d, out, gate);
    return hipGetLastError();
}

hipError_t launch_fill_keys(unsigned long long *keys, int64_t n, hipStream_t stream, Gate gate) {
    if (n <= 0) return hipSuccess;
    fill_keys_kernel<<<grid_stride_blocks(n), 256, 0, stream>>>(keys, n, gate);
    return hipGetLastError();
}

namespace {

// Compute units of the current device, 0 if the query fails. Cached per
// device in atomics: threads that fill an entry at the same time store the
// same value.
int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

template <class Cfg, int MinWaves>
hipError_t launch_tiles_cfg(const float *X, const float *C, const float *cn, int64_t n, int64_t k,
                            int64_t d, unsigned long long *keys, const int *stop,
                            hipStream_t stream) {
    const int tiles_m = (int)cdiv(k, Cfg::BM);
    const int tiles_n = (int)cdiv(n, Cfg::BN);
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    const unsigned blocks = (unsigned)tiles;
    const bool vec = vec_ok(X, d) && vec_ok(C, d);
    const bool full = vec && n % Cfg::BN == 0 && k % Cfg::BM == 0 && d % Cfg::BK == 0;
    if constexpr (Cfg::kThreads == 512) {
        // Full tiles of the one-block-per-CU shapes: one persistent block per
        // CU (no second block fits), each walking its share of the tiles. The
        // walk covers every tile once when the grid has at least one block per
        // XCD (8) or one block per tile, hence the 8-CU minimum.
        const int cus = device_cus();
        if (full && cus >= 8) {
            const unsigned pblocks = (unsigned)(tiles < cus ? tiles : cus);
            assign_tile_kernel<Cfg, kFull, MinWaves, true><<<pblocks, Cfg::kThreads, 0, stream>>>(
                X, C, cn, n, k, d, tiles_m, tiles_n, keys, stop);
            return hipGetLastError();
        }
    }
    if (full)
        assign_tile_kernel<Cfg, kFull, MinWaves, false><<<blocks, Cfg::kThreads, 0, stream>>>(
            X, C, cn, n, k, d, tiles_m, tiles_n, keys, stop);
    else if (vec)
        assign_tile_kernel<Cfg, kVec, MinWaves, false><<<blocks, Cfg::kThreads, 0, stream>>>(
            X, C, cn, n, k, d, tiles_m, tiles_n, keys, stop);
    else
        assign_tile_kernel<Cfg, kScalar, MinWaves, false><<<blocks, Cfg::kThreads, 0, stream>>>(
            X, C, cn, n, k, d, tiles_m, tiles_n, keys, stop);
    return hipGetLastError();
}

template <class Cfg>
int64_t tile_blocks(int64_t n, int64_t k) {
    return cdiv(n, Cfg::BN) * cdiv(k, Cfg::BM);
}

}  // namespace

// Whether the DMA-staged kernel takes a shape: rows of whole 16-byte chunks
// (32-bit buffer offsets need 64 * d * 4 < 2^31); any n and k. Its full-tile
// instance takes whole 256 x 256 tiles and pairs of 32-feature stages, the
// ragged one everything else (edge tiles cut short where n or k is not a
// multiple of 256, any number of stages, the last one partial).
static bool dma_shape(int64_t d) { return d % 4 == 0 && d < (1 << 22); }

static bool dma_full(int64_t n, int64_t k, int64_t d) {
    return n % dma::BN == 0 && k % dma::BM == 0 && d % (2 * dma::BK) == 0;
}

// Rounds of one tile per CU that `tiles` one-block-per-CU tiles take when
// each XCD (an eighth of the CUs) runs an eighth of them.
static int64_t tile_rounds(int64_t tiles, int64_t cus) {
    const int64_t per_xcd = cus >= 8 ? cus / 8 : 1;
    return cdiv(cdiv(tiles, 8), per_xcd);
}

// 16-row blocks of C for the small-k kernel, 0 where it does not take the
// shape: k above 128, or above 64 with fewer than 2^17 samples (there the
// tiles keep more CUs busy: 4096 x 100 x 128 was 19 % slower on this kernel,
// 2^18 x 128 x 128 the same, 2^20 samples with k = 72 to 128 17-50 %
// faster), rows not whole 16-byte chunks, or C past its LDS budget.
static int smallk_blocks(int64_t n, int64_t k, int64_t d) {
    if (k > 128 || (k > 64 && n < (1 << 17)) || d % 4 != 0 || d >= (1 << 22)) return 0;
    const int kb = (int)((k + 15) / 16);
    return 16 * kb * sk_ld(d) <= sk::kLdsFloats ? kb : 0;
}

static const char *regular_tile_name(int64_t n, int64_t k, int64_t d);

static const char *assign_tile_name(int64_t n, int64_t k, int64_t d) {
    // KMEANS_ASSIGN_TILE=smallk | 256x256 | 128x256 | 256x128 | 128x128 |
    // 64x64 forces a tile (tuning); smallk and 256x256 fall back where they
    // do not apply (smallk to the rule below, 256x256 to 128x256).
    const char *forced = getenv("KMEANS_ASSIGN_TILE");
    if (forced && (!strcmp(forced, "256x128") || !strcmp(forced, "128x128") ||
                   !strcmp(forced, "64x64") || !strcmp(forced, "128x256") ||
                   !strcmp(forced, "256x256") || !strcmp(forced, "smallk")))
        return forced;
    // Small k: C resident in LDS and X streamed once.
    if (smallk_blocks(n, k, d) > 0) return "smallk";
    return regular_tile_name(n, k, d);
}

static const char *regular_tile_name(int64_t n, int64_t k, int64_t d) {
    // The DMA-staged 256 x 256 tile where there are enough tiles to give each
    // CU one and either every tile is full or, with edge tiles cut short, it
    // still beats 128 x 256: a round of 256 x 256 tiles costs 1.8 rounds of
    // 128 x 256 ones (measured at d = 1024 ... 4096: 1.79-1.82), so it loses
    // where its coarser edge or last round wastes more (k = 300: 512 rows
    // computed against 384). Else the largest register-staged tile (fewest
    // operand bytes per flop) when it gives at least two blocks per CU;
    // otherwise 128 x 128 with short stages (3 blocks per CU), unless that
    // leaves CUs idle, then 64 x 64.
    const int64_t big = cdiv(n, dma::BN) * cdiv(k, dma::BM);
    const int64_t mid = tile_blocks<Tile128x256>(n, k);
    if (dma_shape(d) && big >= 256) {
        if (dma_full(n, k, d)) return "256x256";
        const int cus = device_cus();
        const int64_t c = cus > 0 ? cus : 256;
        if (mid >= 512 && 9 * tile_rounds(big, c) < 5 * tile_rounds(mid, c)) return "256x256";
    }
    if (mid >= 512) return "128x256";
    if (tile_blocks<Tile128x128>(n, k) >= 256) return "128x128";
    return "64x64";
}

int64_t assign_grid_threads(int64_t n, int64_t k, int64_t d) {
    if (n <= 0) return 0;
    const char *tile = assign_tile_name(n, k, d);
    // The small-k grid is at most two blocks per CU, but unaligned rows fall
    // back to the rule's tile: bound both by the latter.
    if (!strcmp(tile, "smallk")) tile = regular_tile_name(n, k, d);
    if (!strcmp(tile, "256x128")) return tile_blocks<Tile256x128>(n, k) * Tile256x128::kThreads;
    if (!strcmp(tile, "128x128")) return tile_blocks<Tile128x128>(n, k) * Tile128x128::kThreads;
    // 256x256 launches at most one block per CU, but falls back to the
    // 128 x 256 grid for unaligned rows: bound both by the latter.
    if (!strcmp(tile, "128x256") || !strcmp(tile, "256x256"))
        return tile_blocks<Tile128x256>(n, k) * Tile128x256::kThreads;
    return tile_blocks<Tile64x64>(n, k) * Tile64x64::kThreads;
}

template <int KB>
static void launch_smallk_kb(int ncb, unsigned nb, unsigned nt, size_t lds, hipStream_t stream,
                             const float *X, const float *C, const float *cn, int64_t n, int64_t k,
                             int64_t d, unsigned long long *keys, const int *stop) {
    switch (ncb) {
    case 1: assign_smallk_kernel<KB, 1><<<nb, nt, lds, stream>>>(X, C, cn, n, k, d, keys, stop); break;
    case 2: assign_smallk_kernel<KB, 2><<<nb, nt, lds, stream>>>(X, C, cn, n, k, d, keys, stop); break;
    case 3: assign_smallk_kernel<KB, 3><<<nb, nt, lds, stream>>>(X, C, cn, n, k, d, keys, stop); break;
    default: assign_smallk_kernel<KB, 4><<<nb, nt, lds, stream>>>(X, C, cn, n, k, d, keys, stop); break;
    }
}

// Blocks of the (KB, NCB) instance a CU holds at once by its registers and
// waves (the runtime's occupancy query without LDS; 0 if it fails). Cached
// per device and instance in atomics: racing threads store the same value.
template <int KB, int NCB>
static int smallk_occupancy() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, assign_smallk_kernel<KB, NCB>,
                                                         sk::kWaves * 64, 0) != hipSuccess)
            return 0;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

template <int KB>
static int smallk_blocks_per_cu_kb(int ncb) {
    switch (ncb) {
    case 1: return smallk_occupancy<KB, 1>();
    case 2: return smallk_occupancy<KB, 2>();
    case 3: return smallk_occupancy<KB, 3>();
    default: return smallk_occupancy<KB, 4>();
    }
}

static int smallk_blocks_per_cu(int kb, int ncb) {
    switch (kb) {
    case 1: return smallk_blocks_per_cu_kb<1>(ncb);
    case 2: return smallk_blocks_per_cu_kb<2>(ncb);
    case 3: return smallk_blocks_per_cu_kb<3>(ncb);
    case 4: return smallk_blocks_per_cu_kb<4>(ncb);
    case 5: return smallk_blocks_per_cu_kb<5>(ncb);
    case 6: return smallk_blocks_per_cu_kb<6>(ncb);
    case 7: return smallk_blocks_per_cu_kb<7>(ncb);
    default: return smallk_blocks_per_cu_kb<8>(ncb);
    }
}

static void launch_smallk(int kb, int ncb, unsigned nb, unsigned nt, size_t lds, hipStream_t stream,
                          const float *X, const float *C, const float *cn, int64_t n, int64_t k,
                          int64_t d, unsigned long long *keys, const int *stop) {
    switch (kb) {
    case 1: launch_smallk_kb<1>(ncb, nb, nt, lds, stream, X, C, cn, n, k, d, keys, stop); break;
    case 2: launch_smallk_kb<2>(ncb, nb, nt, lds, stream, X, C, cn, n, k, d, keys, stop); break;
    case 3: launch_smallk_kb<3>(ncb, nb, nt, lds, stream, X, C, cn, n, k, d, keys, stop); break;
    case 4: launch_smallk_kb<4>(ncb, nb, nt, lds, stream, X, C, cn, n, k, d, keys, stop); break;
    case 5: launch_smallk_kb<5>(ncb, nb, nt, lds, stream, X, C, cn, n, k, d, keys, stop); break;
    case 6: launch_smallk_kb<6>(ncb, nb, nt, lds, stream, X, C, cn, n, k, d, keys, stop); break;
    case 7: launch_smallk_kb<7>(ncb, nb, nt, lds, stream, X, C, cn, n, k, d, keys, stop); break;
    default: launch_smallk_kb<8>(ncb, nb, nt, lds, stream, X, C, cn, n, k, d, keys, stop); break;
    }
}

// Whether the small-k kernel runs for these arguments (it stores every key).
static bool takes_smallk(const float *X, const float *C, int64_t n, int64_t k, int64_t d) {
    return n > 0 && !strcmp(assign_tile_name(n, k, d), "smallk") && smallk_blocks(n, k, d) > 0 &&
           vec_ok(X, d) && vec_ok(C, d);
}

bool assign_stores_keys(const float *X, const float *C, int64_t n, int64_t k, int64_t d) {
    return takes_smallk(X, C, n, k, d);
}

hipError_t launch_assign_tiles(const float *X, const float *C, const float *cn, int64_t n,
                               int64_t k, int64_t d, unsigned long long *keys,
                               hipStream_t stream, const int *stop) {
    if (n <= 0) return hipSuccess;
    const char *tile = assign_tile_name(n, k, d);
    if (!strcmp(tile, "smallk")) {
        if (takes_smallk(X, C, n, k, d)) {
            // Persistent waves over the 16-sample groups: as many blocks as
            // the CUs hold at once, fewer where there are fewer groups.
            const int kb = smallk_blocks(n, k, d);
            const int ncb = (int)std::min<int64_t>(cdiv(d, sk::kChunk), 4);
            const int cus = device_cus();
            const size_t lds = (size_t)16 * kb * sk_ld(d) * sizeof(float);
            // As many blocks as the CUs hold at once (by LDS, 160 KiB per CU,
            // and by registers), so that no block waits for another to end.
            int64_t per_cu = (int64_t)((160 << 10) / lds);
            const int by_regs = smallk_blocks_per_cu(kb, ncb);
            if (by_regs > 0 && per_cu > by_regs) per_cu = by_regs;
            if (per_cu < 1) per_cu = 1;
            int64_t blocks = cdiv(cdiv(n, 16), sk::kWaves);
            const int64_t cap = per_cu * (int64_t)(cus > 0 ? cus : 256);
            if (blocks > cap) blocks = cap;
            const unsigned nb = (unsigned)blocks, nt = sk::kWaves * 64;
            launch_smallk(kb, ncb, nb, nt, lds, stream, X, C, cn, n, k, d, keys, stop);
            return hipGetLastError();
        }
        tile = regular_tile_name(n, k, d);
    }
    if (!strcmp(tile, "256x256")) {
        // One persistent block per CU (128 KiB of LDS: one fits), each walking
        // its XCD's tiles; the walk needs at least 8 blocks or one per tile.
        const int cus = device_cus();
        if (dma_shape(d) && vec_ok(X, d) && vec_ok(C, d) && cus >= 8) {
            const int tm = (int)cdiv(k, dma::BM), tn = (int)cdiv(n, dma::BN);
            const int64_t tiles = (int64_t)tm * tn;
            const unsigned blocks = (unsigned)(tiles < cus ? tiles : cus);
            if (dma_full(n, k, d))
                assign_dma_kernel<kDmaFull><<<blocks, dma::NT, 0, stream>>>(X, C, cn, n, k, d, tm,
                                                                            tn, keys, stop);
            else if (d % (2 * dma::BK) == 0)
                assign_dma_kernel<kDmaRagged><<<blocks, dma::NT, 0, stream>>>(X, C, cn, n, k, d, tm,
                                                                              tn, keys, stop);
            else
                assign_dma_kernel<kDmaAnyD><<<blocks, dma::NT, 0, stream>>>(X, C, cn, n, k, d, tm,
                                                                            tn, keys, stop);
            return hipGetLastError();
        }
        return launch_tiles_cfg<Tile128x256, 2>(X, C, cn, n, k, d, keys, stop, stream);
    }
    if (!strcmp(tile, "256x128"))
        return launch_tiles_cfg<Tile256x128, 2>(X, C, cn, n, k, d, keys, stop, stream);
    if (!strcmp(tile, "128x128"))
        return launch_tiles_cfg<Tile128x128, 3>(X, C, cn, n, k, d, keys, stop, stream);
    if (!strcmp(tile, "128x256"))
        return launch_tiles_cfg<Tile128x256, 2>(X, C, cn, n, k, d, keys, stop, stream);
    return launch_tiles_cfg<Tile64x64, 4>(X, C, cn, n, k, d, keys, stop, stream);
}

hipError_t launch_finalize(unsigned long long *keys, float *min_dist, bool add_norm, int64_t n,
                           int64_t k, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    finalize_kernel<<<grid_stride_blocks(n), 256, 0, stream>>>(keys, min_dist, add_norm, n, k);
    return hipGetLastError();
}

}  // namespace km
