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
// kept, and D becomes those minima. Distances are float64 in difference form.
//
// Per centre, two launches and nothing on the host:
//   pp_select_kernel  one block: potentials of the previous trials from the
//                     per-block partials (fixed-order block reduction), the
//                     winner, its row copied out as a centre, then the next
//                     candidates: a scan over the block sums of D finds the
//                     block each draw falls in, one wave per draw walks its
//                     rows
//   pp_dist_kernel    every sample against all candidates: candidate rows
//                     staged in LDS 1024 features at a time (double buffered,
//                     the next stage's loads in flight during the current
//                     one), one wave per sample, float64 sums; min with D;
//                     per-block partials
// Buffers of D and partials alternate between centres (A <-> B).
#include "kernels.h"

namespace km {
namespace {

constexpr int kPPMaxTrials = 16;
constexpr int kPPChunk = 1024;      // features per LDS stage
constexpr int kPPRowsPerBlock = 64; // samples per block of pp_dist_kernel

struct PPState {
    double pot;  // potential of the chosen candidate
    int best;    // its trial index
};

// Samples [b * kPPRowsPerBlock, ...) against the `trials` candidate rows.
// closest_prev = D of the previous centre set (NULL: +inf, the first centre).
//
// 16 waves; wave w handles samples b*64 + w, +16, +32, +48 (4 row groups).
// The work is a sequence of stages (row group g, feature chunk c); at every
// stage each lane holds 16 features of its wave's sample in registers and the
// block holds the candidates' values of chunk c in LDS. The loads of stage
// s + 1 (sample values into registers, candidate values into registers, then
// into the other LDS buffer) are issued before stage s is computed, so memory
// latency overlaps the float64 arithmetic. One barrier per stage.
__global__ __launch_bounds__(1024) void pp_dist_kernel(
    const float *__restrict__ X, int64_t n, int64_t d, int trials,
    const long long *__restrict__ cand, const PPState *__restrict__ st,
    const double *__restrict__ prev_buf, double *__restrict__ out_buf,
    double *__restrict__ out_parts, int64_t nb) {
    __shared__ float cs[2][kPPMaxTrials * kPPChunk];  // 2 x 64 KiB
    __shared__ double wave_part[16][kPPMaxTrials];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t b = blockIdx.x;
    const double *closest = prev_buf ? prev_buf + (int64_t)st->best * n : nullptr;
    const int64_t chunks = (d + kPPChunk - 1) / kPPChunk;
    const int64_t stages = 4 * chunks;
    constexpr int kPerLane = kPPChunk / 64;  // 16 features per lane and stage

    if (lane < kPPMaxTrials) wave_part[wave][lane] = 0.0;

    // Stage s: row group s / chunks, chunk s % chunks.
    auto load_x = [&](int64_t s, float (&xr)[kPerLane]) {
        const int64_t i = b * kPPRowsPerBlock + (s / chunks) * 16 + wave;
        const int64_t c0 = (s % chunks) * kPPChunk;
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int64_t f = c0 + lane + 64 * j;
            xr[j] = (i < n && f < d) ? X[i * d + f] : 0.f;
        }
    };
    auto load_c = [&](int64_t s, float (&cv)[kPPMaxTrials]) {
        const int64_t f = (s % chunks) * kPPChunk + tid;
#pragma unroll
        for (int t = 0; t < kPPMaxTrials; ++t)
            cv[t] = (t < trials && f < d) ? X[(int64_t)cand[t] * d + f] : 0.f;
    };
    auto store_c = [&](int buf, const float (&cv)[kPPMaxTrials]) {
#pragma unroll
        for (int t = 0; t < kPPMaxTrials; ++t)
            if (t < trials) cs[buf][t * kPPChunk + tid] = cv[t];
    };

    float xr[kPerLane], xn[kPerLane], cv[kPPMaxTrials];
    load_x(0, xr);
    load_c(0, cv);
    store_c(0, cv);
    __syncthreads();

    double acc[kPPMaxTrials];
#pragma unroll
    for (int t = 0; t < kPPMaxTrials; ++t) acc[t] = 0.0;
    for (int64_t s = 0; s < stages; ++s) {
        const int cur = (int)(s & 1);
        if (s + 1 < stages) {
            load_x(s + 1, xn);
            load_c(s + 1, cv);
        }
        // Features of this stage beyond d were loaded as 0 for the sample and
        // every candidate, so they add 0.
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const double xv = (double)xr[j];
            const int f = lane + 64 * j;
#pragma unroll
            for (int t = 0; t < kPPMaxTrials; ++t) {
                if (t < trials) {
                    const double diff = xv - (double)cs[cur][t * kPPChunk + f];
                    acc[t] += diff * diff;
                }
            }
        }
        if (s % chunks == chunks - 1) {
            // The wave's sample of this row group is complete.
            const int64_t i = b * kPPRowsPerBlock + (s / chunks) * 16 + wave;
            if (i < n) {
                const double cur_d = closest ? closest[i] : __builtin_inf();
#pragma unroll
                for (int t = 0; t < kPPMaxTrials; ++t) {
                    if (t < trials) {
                        double v = acc[t];
                        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
                        const double nd = v < cur_d ? v : cur_d;
                        if (lane == 0) {
                            out_buf[(int64_t)t * n + i] = nd;
                            wave_part[wave][t] += nd;  // this wave's rows, in order
                        }
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < kPPMaxTrials; ++t) acc[t] = 0.0;
        }
        if (s + 1 < stages) {
            store_c(cur ^ 1, cv);
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) xr[j] = xn[j];
        }
        __syncthreads();
    }
    if (tid < trials) {
        double sum = 0.0;
        for (int w = 0; w < 16; ++w) sum += wave_part[w][tid];
        out_parts[(int64_t)tid * nb + b] = sum;
    }
}

// Sum over the 256 threads of the block in a fixed order.
__device__ double block_sum256(double v, double *lds4) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) lds4[threadIdx.x >> 6] = v;
    __syncthreads();
    const double t = ((lds4[0] + lds4[1]) + lds4[2]) + lds4[3];
    __syncthreads();
    return t;
}

// Winner of the previous trials, recorded as centre c_rec; then, if rand_row
// is not NULL, the next candidates. One block of 256 threads.
__global__ __launch_bounds__(256) void pp_select_kernel(
    const float *__restrict__ X, int64_t n, int64_t d, const double *__restrict__ prev_buf,
    const double *__restrict__ prev_parts, int64_t nb, int trials_prev,
    const long long *__restrict__ cand_prev, PPState *st, int64_t c_rec,
    long long *__restrict__ chosen, float *__restrict__ centres,
    const double *__restrict__ rand_row, int trials_next, long long *__restrict__ cand_next) {
    __shared__ double lds4[4];
    __shared__ double pots[kPPMaxTrials];
    __shared__ double scan_tot[4];
    __shared__ int found_block[kPPMaxTrials];
    __shared__ double found_before[kPPMaxTrials];
    __shared__ int wave_first[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // Potentials: thread j adds the partials b = j, j + 256, ... in order,
    // then a fixed tree over the threads.
    for (int t = 0; t < trials_prev; ++t) {
        double s = 0.0;
        for (int64_t b = tid; b < nb; b += 256) s += prev_parts[(int64_t)t * nb + b];
        const double tot = block_sum256(s, lds4);
        if (tid == 0) pots[t] = tot;
    }
    __syncthreads();
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
    for (int64_t f = tid; f < d; f += 256) centres[c_rec * d + f] = X[row * d + f];
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
    __syncthreads();
    double carry = 0.0;
    for (int64_t b0 = 0; b0 < nb; b0 += 256) {
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
        __syncthreads();
        double before_wave = 0.0;
        for (int w = 0; w < wave; ++w) before_wave += scan_tot[w];
        const double chunk_tot = ((scan_tot[0] + scan_tot[1]) + scan_tot[2]) + scan_tot[3];
        const double run_incl = carry + (before_wave + incl);
        const double run_excl = carry + (before_wave + excl);
        // For each trial still open: the lowest block of this chunk whose
        // inclusive running sum reaches its target.
        for (int t = 0; t < trials_next; ++t) {
            const bool open = found_block[t] < 0;  // uniform
            const bool hit = open && b < nb && run_incl >= rand_row[t] * pot;
            const unsigned long long m = __ballot(hit);
            if (lane == 0) wave_first[wave] = m ? (int)(b0 + wave * 64 + __ffsll((long long)m) - 1) : -1;
            __syncthreads();
            if (tid == 0 && open) {
                for (int w = 0; w < 4; ++w)
                    if (wave_first[w] >= 0) {
                        found_block[t] = wave_first[w];
                        break;
                    }
            }
            __syncthreads();
            if (open && b == found_block[t]) found_before[t] = run_excl;
            __syncthreads();
        }
        carry += chunk_tot;
        __syncthreads();  // scan_tot is rewritten by the next chunk
    }
    // One wave per trial: walk the rows from the block found (64 rows = one
    // wave), continuing into later blocks if the target lies beyond it.
    for (int t = wave; t < trials_next; t += 4) {
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
    pp_dist_kernel<<<(unsigned)nb, 1024, 0, stream>>>(X, n, d, 1, cand[0], st, nullptr, buf[0],
                                                      parts[0], nb);
    int cur = 0, trials_prev = 1;
    for (int64_t c = 1; c <= k; ++c) {
        const bool more = c < k;
        pp_select_kernel<<<1, 256, 0, stream>>>(
            X, n, d, buf[cur], parts[cur], nb, trials_prev, cand[cur], st, c - 1,
            (long long *)chosen, centres, more ? rand + (c - 1) * trials : nullptr, trials,
            cand[cur ^ 1]);
        if (!more) break;
        pp_dist_kernel<<<(unsigned)nb, 1024, 0, stream>>>(X, n, d, trials, cand[cur ^ 1], st,
                                                          buf[cur], buf[cur ^ 1],
                                                          parts[cur ^ 1], nb);
        cur ^= 1;
        trials_prev = trials;
    }
    return hipGetLastError();
}

}  // namespace km
