// kmeanspp.hip - greedy k-means++ seeding on gfx950 ("004 - tile sizes ...",
// section k-means++: 2 + log(k) candidate trials per centre; the pages'
// faster version computes the sample norms once and gathers the candidate
// rows instead of pulling indices to the host).
//
// Definition followed (the same as the float64 CPU oracle): the first centre
// is given. D(i) is the squared distance of sample i to its nearest chosen
// centre and pot = sum_i D(i). For centre c, trial t draws u = rand[(c-1) *
// trials + t] and takes the first sample whose running sum of D reaches
// u * pot (the last sample if none does); the candidate whose potential
// sum_i min(D(i), |x_i - x_cand|^2) is smallest (lowest trial on ties) is
// kept, and D becomes those minima.
//
// Distances are float64 in Gram form, |x|^2 + |c|^2 - 2 x.c clamped at 0,
// with the sample norms computed once per call as the pages' faster version
// does. A float32 x float32 product is exact in float64, so the only
// roundings are those of the float64 sums; the norms use the same per-lane
// order and reduction tree as the dot products, so a sample's distance to
// itself is exactly 0.
//
// Per call, pp_norm_kernel computes |x_i|^2 once. Per centre, two launches
// and nothing on the host:
//   pp_select_kernel  one 1024-thread block: potentials of the previous trials from the
//                     per-block partials (fixed-order block reduction), the
//                     winner, its row copied out as a centre, then the next
//                     candidates: a scan over the block sums of D finds the
//                     block each draw falls in, one wave per draw walks its
//                     rows
//   pp_dist_kernel    every sample against all candidates: candidate rows
//                     staged in LDS 256 or 512 features at a time (double
//                     buffered, the next stage's loads in flight during the
//                     current one), a wave on 1, 2 or 4 samples at once,
//                     float64 dot products; min with D; per-block partials
// Buffers of D and partials alternate between centres (A <-> B).
#include "kernels.h"

namespace km {
namespace {

constexpr int kPPMaxTrials = 16;
constexpr int kPPChunk = 256;       // features per lane-slice of a stage: 4 per lane
constexpr int kPPRowsPerBlock = 64; // samples per block of pp_dist_kernel

struct PPState {
    double pot;  // potential of the chosen candidate
    int best;    // its trial index
};

// X[i, f .. f+3] with zeros for i >= n or features >= d. kVec: X is 16-byte
// aligned and d % 4 == 0, so the four values are one 16-byte load.
template <bool kVec>
__device__ __forceinline__ float4 load_row4(const float *__restrict__ X, int64_t n, int64_t d,
                                            int64_t i, int64_t f) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i >= n) return v;
    const float *p = X + i * d + f;
    if (kVec) {
        if (f < d) v = *(const float4 *)p;
    } else {
        if (f < d) v.x = p[0];
        if (f + 1 < d) v.y = p[1];
        if (f + 2 < d) v.z = p[2];
        if (f + 3 < d) v.w = p[3];
    }
    return v;
}

// Sums over the 64 lanes of a wave of M values per lane, M = 2^m <= 64: at
// each halving step a lane keeps one half of its values and adds the
// partner's copy of that half, sending the other half (M - 1 shuffles
// instead of M * 6). On return v[0] of lane l holds the total of value
// l >> (6 - m). The order of the additions is fixed.
template <int M>
__device__ __forceinline__ void wave_sum_transpose(double (&v)[M], int lane) {
    static_assert(M >= 1 && M <= 64 && (M & (M - 1)) == 0, "M must be a power of two");
    constexpr int kSteps = M == 1 ? 0 : M == 2 ? 1 : M == 4 ? 2 : M == 8 ? 3 : M == 16 ? 4 : M == 32 ? 5 : 6;
#pragma unroll
    for (int step = 0; step < kSteps; ++step) {
        const int half = M >> (step + 1), bit = 5 - step;
        const bool hi = (lane >> bit) & 1;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            // Opaque copies: without them the compiler turns the two selects
            // below into a lane-dependent index into v, which it can only
            // lower as a compare chain over the whole array.
            double lo = v[i], up = v[i + half];
            asm volatile("" : "+v"(lo), "+v"(up));
            const double send = hi ? lo : up;
            const double keep = hi ? up : lo;
            v[i] = keep + __shfl_xor(send, 1 << bit);
        }
    }
#pragma unroll
    for (int bit = 5 - kSteps; bit >= 0; --bit) v[0] += __shfl_xor(v[0], 1 << bit);
}

constexpr int pow2_at_least(int x) { return x <= 1 ? 1 : 2 * pow2_at_least((x + 1) / 2); }

constexpr int kPPWaves = 8;  // waves per block of pp_dist_kernel (512 threads)

// Samples [b * 64, b * 64 + 64) against the T candidate rows cand[0..T).
// prev_buf + best * n holds D of the previous centre set (prev_buf NULL: the
// first centre, D = +inf).
//
// 8 waves; a wave works on R samples at once, so every candidate value read
// from LDS and widened to float64 serves R samples (R = 1, 2 or 4). Wave w's
// samples are b*64 + w + 8 m for m = p*R + r (pass p, slot r), 8/R passes.
// The work is a sequence of stages (pass, chunk of 256 V features); lane l
// loads features 256 v + 4 l .. +3 (v < V) of its R samples and of the
// candidates it stages. Everything a stage reads sits in LDS: the wave's own
// sample values in xs (each wave overwrites only its own slice, after its
// own reads, so one buffer suffices) and the candidates in cs, double
// buffered and stored [t][4 v + q][lane] so that the reads of one (t, v, q)
// are 64 consecutive words. The registers only carry the next stage's loads,
// issued before the current stage is computed; one barrier per stage. At
// most 128 registers (4 waves per SIMD) let two blocks share a CU, so one
// computes while the other waits.
// |x_i|^2 in float64, one wave per sample, 4 samples per 256-thread block.
// Lane l adds x_f^2 for f = 256 s' + 4 l + q in the order of slices s' and
// then q, and the lanes are combined by the butterfly of wave_sum_transpose:
// the same order as the dot products of pp_dist_kernel, so |x_i|^2 equals
// x_i . x_i there bit for bit.
__global__ __launch_bounds__(256) void pp_norm_kernel(const float *__restrict__ X, int64_t n,
                                                     int64_t d, double *__restrict__ xnorm) {
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= n) return;  // whole wave
    const float *x = X + i * d;
    double acc[1] = {0.0};
    for (int64_t f0 = 4 * lane; f0 < d; f0 += kPPChunk) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const double v = f0 + q < d ? (double)x[f0 + q] : 0.0;
            acc[0] = __builtin_fma(v, v, acc[0]);
        }
    }
    wave_sum_transpose<1>(acc, lane);
    if (lane == 0) xnorm[i] = acc[0];
}

// LDS of one pp_dist_kernel block: xs, cs and wave_part below.
constexpr int pp_dist_lds_bytes(int T, int R, int V) {
    return kPPWaves * R * V * 64 * 16 + 2 * T * 4 * V * 64 * 4 + kPPWaves * R * T * 8;
}

template <int T, int R, int V, bool kVec>
__global__ __launch_bounds__(kPPWaves * 64, 4) void pp_dist_kernel(
    const float *__restrict__ X, const double *__restrict__ xnorm, int64_t n, int64_t d,
    const long long *__restrict__ cand, const PPState *__restrict__ st,
    const double *__restrict__ prev_buf, double *__restrict__ out_buf,
    double *__restrict__ out_parts, int64_t nb) {
    constexpr int kChunk = kPPChunk * V;
    constexpr int kPasses = kPPRowsPerBlock / (kPPWaves * R);
    constexpr int kCandPerWave = (T + kPPWaves - 1) / kPPWaves;
    constexpr int kM = pow2_at_least(R * T);          // values per lane to reduce
    constexpr int kGroup = 64 / kM;                   // lanes holding one total
    __shared__ float4 xs[kPPWaves][R][V][64];
    __shared__ float cs[2][T][4 * V][64];
    __shared__ double wave_part[kPPWaves][R][T];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t b = blockIdx.x;
    const double *closest = prev_buf ? prev_buf + (int64_t)st->best * n : nullptr;
    const int64_t chunks = (d + kChunk - 1) / kChunk;
    const int64_t stages = kPasses * chunks;
    // Wave w stages candidates w, w + 8 (those below T).
    int64_t my_cand[kCandPerWave];
#pragma unroll
    for (int j = 0; j < kCandPerWave; ++j) {
        const int t = wave + kPPWaves * j;
        my_cand[j] = t < T ? (int64_t)cand[t] : 0;
    }
    __shared__ double cand_norm[T];
    if (tid < T) cand_norm[tid] = xnorm[cand[tid]];

    auto row = [&](int64_t p, int r) {
        return b * kPPRowsPerBlock + (p * R + r) * kPPWaves + wave;
    };
    auto load_stage = [&](int64_t s, float4 (&xr)[R][V], float4 (&cv)[kCandPerWave][V]) {
        const int64_t p = s / chunks, f = (s % chunks) * kChunk + 4 * lane;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int v = 0; v < V; ++v)
                xr[r][v] = load_row4<kVec>(X, n, d, row(p, r), f + kPPChunk * v);
#pragma unroll
        for (int j = 0; j < kCandPerWave; ++j)
            if (wave + kPPWaves * j < T)
#pragma unroll
                for (int v = 0; v < V; ++v)
                    cv[j][v] = load_row4<kVec>(X, n, d, my_cand[j], f + kPPChunk * v);
    };
    auto store_stage = [&](int buf, const float4 (&xr)[R][V], const float4 (&cv)[kCandPerWave][V]) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int v = 0; v < V; ++v) xs[wave][r][v][lane] = xr[r][v];
#pragma unroll
        for (int j = 0; j < kCandPerWave; ++j) {
            const int t = wave + kPPWaves * j;
            if (t < T) {
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    cs[buf][t][4 * v + 0][lane] = cv[j][v].x;
                    cs[buf][t][4 * v + 1][lane] = cv[j][v].y;
                    cs[buf][t][4 * v + 2][lane] = cv[j][v].z;
                    cs[buf][t][4 * v + 3][lane] = cv[j][v].w;
                }
            }
        }
    };

    float4 xn[R][V], cv[kCandPerWave][V];
    load_stage(0, xn, cv);
    store_stage(0, xn, cv);
    __syncthreads();

    // acc[r * T + t]: this lane's part of x . c_t for slot r; the entries
    // from R * T up to kM stay 0 and only pad the reduction.
    double acc[kM];
#pragma unroll
    for (int j = 0; j < kM; ++j) acc[j] = 0.0;
    // This lane's running sum of the final D over its passes, for the value
    // (r, t) it receives from the reduction.
    const int my_idx = lane / kGroup;
    double my_part = 0.0;

    for (int64_t s = 0; s < stages; ++s) {
        const int cur = (int)(s & 1);
        if (s + 1 < stages) load_stage(s + 1, xn, cv);
        // Features beyond d were loaded as 0 for samples and candidates alike,
        // so they add 0. Per lane the features come in the order 256 s' + 4
        // lane + q over slices s' and then q, as in pp_norm_kernel. (Not
        // unrolled over v: the compiler would hoist the
        // LDS reads of every slice and run out of registers.)
#pragma unroll 1
        for (int v = 0; v < V; ++v) {
            float4 xf[R];
#pragma unroll
            for (int r = 0; r < R; ++r) xf[r] = xs[wave][r][v][lane];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                double xd[R];
#pragma unroll
                for (int r = 0; r < R; ++r)
                    xd[r] = (double)(q == 0 ? xf[r].x : q == 1 ? xf[r].y : q == 2 ? xf[r].z : xf[r].w);
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const double c = (double)cs[cur][t][4 * v + q][lane];
#pragma unroll
                    for (int r = 0; r < R; ++r) acc[r * T + t] = __builtin_fma(xd[r], c, acc[r * T + t]);
                }
            }
        }
        if (s % chunks == chunks - 1) {
            // The R samples of this pass are complete.
            wave_sum_transpose<kM>(acc, lane);
            const int64_t i = row(s / chunks, my_idx / T);
            if (lane % kGroup == 0 && my_idx < R * T && i < n) {
                const int t = my_idx % T;
                const double cur_d = closest ? closest[i] : __builtin_inf();
                const double dist = __builtin_fma(-2.0, acc[0], xnorm[i] + cand_norm[t]);
                const double pos = dist > 0.0 ? dist : 0.0;
                const double nd = pos < cur_d ? pos : cur_d;
                out_buf[(int64_t)t * n + i] = nd;
                my_part += nd;
            }
#pragma unroll
            for (int j = 0; j < kM; ++j) acc[j] = 0.0;
        }
        if (s + 1 < stages) store_stage(cur ^ 1, xn, cv);
        __syncthreads();
    }
    if (lane % kGroup == 0 && my_idx < R * T) wave_part[wave][my_idx / T][my_idx % T] = my_part;
    __syncthreads();
    if (tid < T) {
        double sum = 0.0;
        for (int w = 0; w < kPPWaves; ++w)
            for (int r = 0; r < R; ++r) sum += wave_part[w][r][tid];
        out_parts[(int64_t)tid * nb + b] = sum;
    }
}

// Launch of pp_dist_kernel for a run-time trial count. A wave takes R
// samples at once with R * T <= 16, so that the float64 accumulators fit in
// 32 registers and two blocks fit on a CU without spilling.
template <int T>
void launch_dist_t(bool vec, unsigned nb, hipStream_t stream, const float *X,
                   const double *xnorm, int64_t n, int64_t d, const long long *cand,
                   const PPState *st, const double *prev, double *out, double *parts) {
    constexpr int R = T <= 4 ? 4 : T <= 8 ? 2 : 1;
    // Two 256-feature slices per stage where the LDS of two blocks still fits
    // in a CU's 160 KiB, else one.
    constexpr int V = 2 * pp_dist_lds_bytes(T, R, 2) <= 160 * 1024 ? 2 : 1;
    if (vec)
        pp_dist_kernel<T, R, V, true><<<nb, kPPWaves * 64, 0, stream>>>(X, xnorm, n, d, cand, st,
                                                                        prev, out, parts, nb);
    else
        pp_dist_kernel<T, R, V, false><<<nb, kPPWaves * 64, 0, stream>>>(X, xnorm, n, d, cand, st,
                                                                         prev, out, parts, nb);
}

void launch_dist(int trials, bool vec, unsigned nb, hipStream_t stream, const float *X,
                 const double *xnorm, int64_t n, int64_t d, const long long *cand,
                 const PPState *st, const double *prev, double *out, double *parts) {
    switch (trials) {
#define KM_PP_CASE(T) \
    case T: launch_dist_t<T>(vec, nb, stream, X, xnorm, n, d, cand, st, prev, out, parts); break;
        KM_PP_CASE(1) KM_PP_CASE(2) KM_PP_CASE(3) KM_PP_CASE(4)
        KM_PP_CASE(5) KM_PP_CASE(6) KM_PP_CASE(7) KM_PP_CASE(8)
        KM_PP_CASE(9) KM_PP_CASE(10) KM_PP_CASE(11) KM_PP_CASE(12)
        KM_PP_CASE(13) KM_PP_CASE(14) KM_PP_CASE(15) KM_PP_CASE(16)
#undef KM_PP_CASE
        default: break;  // trials is validated to 1 .. kPPMaxTrials by the caller
    }
}

constexpr int kSelWaves = 16;  // pp_select_kernel: one 1024-thread block

// Winner of the previous trials, recorded as centre c_rec; then, if rand_row
// is not NULL, the next candidates. One block of 1024 threads; every sum has
// a fixed order.
__global__ __launch_bounds__(kSelWaves * 64) void pp_select_kernel(
    const float *__restrict__ X, int64_t n, int64_t d, const double *__restrict__ prev_buf,
    const double *__restrict__ prev_parts, int64_t nb, int trials_prev,
    const long long *__restrict__ cand_prev, PPState *st, int64_t c_rec,
    long long *__restrict__ chosen, float *__restrict__ centres,
    const double *__restrict__ rand_row, int trials_next, long long *__restrict__ cand_next) {
    constexpr int kThreads = kSelWaves * 64;
    __shared__ double wsum[kPPMaxTrials][kSelWaves];
    __shared__ double pots[kPPMaxTrials];
    __shared__ double scan_tot[kSelWaves];
    __shared__ double chunk_excl[kThreads];
    __shared__ int wave_first[kPPMaxTrials][kSelWaves];
    __shared__ int found_block[kPPMaxTrials];
    __shared__ double found_before[kPPMaxTrials];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // Potentials: thread j adds the partials b = j, j + 1024, ... in order;
    // the threads are combined by a butterfly within each wave, then the
    // waves in order. All trials' loads are issued together.
    {
        double s[kPPMaxTrials];
#pragma unroll
        for (int t = 0; t < kPPMaxTrials; ++t) s[t] = 0.0;
        for (int64_t b = tid; b < nb; b += kThreads) {
            double v[kPPMaxTrials];
#pragma unroll
            for (int t = 0; t < kPPMaxTrials; ++t)
                v[t] = t < trials_prev ? prev_parts[(int64_t)t * nb + b] : 0.0;
#pragma unroll
            for (int t = 0; t < kPPMaxTrials; ++t) s[t] += v[t];
        }
#pragma unroll
        for (int t = 0; t < kPPMaxTrials; ++t) {
            if (t < trials_prev) {
                double v = s[t];
                for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
                if (lane == 0) wsum[t][wave] = v;
            }
        }
        __syncthreads();
        if (tid < trials_prev) {
            double tot = 0.0;
            for (int w = 0; w < kSelWaves; ++w) tot += wsum[tid][w];
            pots[tid] = tot;
        }
        __syncthreads();
    }
    int best = 0;
    for (int t = 1; t < trials_prev; ++t)
        if (pots[t] < pots[best]) best = t;
    const double pot = pots[best];
    const long long row = cand_prev[best];
    if (tid == 0) {
        st->best = best;
        st->pot = pot;
        chosen[c_rec] = row;
    }
    for (int64_t f = tid; f < d; f += kThreads) centres[c_rec * d + f] = X[row * d + f];
    if (!rand_row) return;

    // Candidate draws: the first sample whose running sum of D reaches
    // u * pot. The running sum is evaluated as (sum of the whole blocks before
    // the sample's block, scanned in block order) + (the sample sums inside
    // its block, in sample order).
    const double *D = prev_buf + (int64_t)best * n;
    const double *parts = prev_parts + (int64_t)best * nb;
    if (tid < kPPMaxTrials) {
        found_block[tid] = -1;
        found_before[tid] = 0.0;
    }
    double carry = 0.0;
    for (int64_t b0 = 0; b0 < nb; b0 += kThreads) {
        const int64_t b = b0 + tid;
        const double v = b < nb ? parts[b] : 0.0;
        double incl = v;
        for (int off = 1; off < 64; off <<= 1) {
            const double up = __shfl_up(incl, off);
            if (lane >= off) incl += up;
        }
        double excl = __shfl_up(incl, 1);
        if (lane == 0) excl = 0.0;
        if (lane == 63) scan_tot[wave] = incl;
        __syncthreads();  // also publishes found_block from the previous chunk
        double before_wave = 0.0, chunk_tot = 0.0;
        for (int w = 0; w < kSelWaves; ++w) {
            before_wave += w < wave ? scan_tot[w] : 0.0;
            chunk_tot += scan_tot[w];
        }
        const double run_incl = carry + (before_wave + incl);
        chunk_excl[tid] = carry + (before_wave + excl);
        // For each trial still open: this wave's lowest block whose inclusive
        // running sum reaches the trial's target.
        for (int t = 0; t < trials_next; ++t) {
            const bool hit = found_block[t] < 0 && b < nb && run_incl >= rand_row[t] * pot;
            const unsigned long long m = __ballot(hit);
            if (lane == 0) wave_first[t][wave] = m ? (int)(b0 + wave * 64 + __ffsll((long long)m) - 1) : -1;
        }
        __syncthreads();
        bool all_found = true;
        if (tid < trials_next && found_block[tid] < 0) {
            for (int w = 0; w < kSelWaves; ++w)
                if (wave_first[tid][w] >= 0) {
                    found_block[tid] = wave_first[tid][w];
                    found_before[tid] = chunk_excl[wave_first[tid][w] - b0];
                    break;
                }
        }
        carry += chunk_tot;
        __syncthreads();  // found_block, found_before published; scan_tot, chunk_excl reusable
        for (int t = 0; t < trials_next; ++t) all_found = all_found && found_block[t] >= 0;
        if (all_found) break;  // uniform: every thread reads the same LDS values
    }
    // One wave per trial: walk the rows from the block found (64 rows = one
    // wave), continuing into later blocks if the target lies beyond it.
    for (int t = wave; t < trials_next; t += kSelWaves) {
        const double target = rand_row[t] * pot;
        int64_t idx = n - 1;
        if (found_block[t] >= 0) {
            double base = found_before[t];
            for (int64_t r0 = (int64_t)found_block[t] * kPPRowsPerBlock; r0 < n; r0 += 64) {
                const int64_t i = r0 + lane;
                double incl = i < n ? D[i] : 0.0;
                for (int off = 1; off < 64; off <<= 1) {
                    const double up = __shfl_up(incl, off);
                    if (lane >= off) incl += up;
                }
                const double acc = base + incl;
                const unsigned long long m = __ballot(i < n && acc >= target);
                if (m) {
                    idx = r0 + __ffsll((long long)m) - 1;
                    break;
                }
                base += __shfl(incl, 63);
            }
        }
        if (lane == 0) cand_next[t] = idx;
    }
}

__global__ void pp_init_kernel(long long *cand, long long first) { cand[0] = first; }

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

int64_t pp_blocks(int64_t n) { return cdiv(n, kPPRowsPerBlock); }
int pp_max_trials() { return kPPMaxTrials; }
int pp_block_threads() { return kPPWaves * 64; }
size_t pp_state_bytes() { return sizeof(PPState); }

hipError_t launch_kmeanspp(const float *X, int64_t n, int64_t d, int64_t k, int64_t first,
                           int trials, const double *rand, float *centres, int64_t *chosen,
                           const PPScratch &ws, hipStream_t stream) {
    const int64_t nb = pp_blocks(n);
    PPState *st = (PPState *)ws.state;
    double *buf[2] = {ws.buf_a, ws.buf_b};
    double *parts[2] = {ws.parts_a, ws.parts_b};
    long long *cand[2] = {(long long *)ws.cand_a, (long long *)ws.cand_b};
    pp_init_kernel<<<1, 1, 0, stream>>>(cand[0], first);
    // D of the first centre alone (one "trial": the given sample).
    const bool vec = d % 4 == 0 && reinterpret_cast<uintptr_t>(X) % 16 == 0;
    pp_norm_kernel<<<(unsigned)cdiv(n, 4), 256, 0, stream>>>(X, n, d, ws.xnorm);
    launch_dist(1, vec, (unsigned)nb, stream, X, ws.xnorm, n, d, cand[0], st, nullptr, buf[0],
                parts[0]);
    int cur = 0, trials_prev = 1;
    for (int64_t c = 1; c <= k; ++c) {
        const bool more = c < k;
        pp_select_kernel<<<1, kSelWaves * 64, 0, stream>>>(
            X, n, d, buf[cur], parts[cur], nb, trials_prev, cand[cur], st, c - 1,
            (long long *)chosen, centres, more ? rand + (c - 1) * trials : nullptr, trials,
            cand[cur ^ 1]);
        if (!more) break;
        launch_dist(trials, vec, (unsigned)nb, stream, X, ws.xnorm, n, d, cand[cur ^ 1], st,
                    buf[cur], buf[cur ^ 1], parts[cur ^ 1]);
        cur ^= 1;
        trials_prev = trials;
    }
    return hipGetLastError();
}

}  // namespace km
