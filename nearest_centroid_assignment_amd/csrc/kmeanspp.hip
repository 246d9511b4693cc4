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
// roundings are those of the float64 sums; a sample's distance to itself is
// set to exactly 0.
//
// Per call, pp_norm_kernel computes |x_i|^2 once and pp_gather_kernel copies
// the chosen rows out as the centres at the end. Per centre, two launches and
// nothing on the host:
//   pp_select_kernel  one 1024-thread block: potentials of the previous
//                     trials from the per-block partials (fixed-order
//                     reduction), the winner recorded as a centre index,
//                     then the next candidates: a scan over the block sums of
//                     D finds the block each draw falls in, one wave per draw
//                     walks its rows
//   pp_dist_kernel    every sample against all candidates on the float64
//                     matrix cores (16 samples x 16 candidate slots per wave),
//                     samples staged through per-wave LDS slices, candidates
//                     through shared LDS, the next stage's loads in flight
//                     during the current one; min with D; per-block partials
// Buffers of D and partials alternate between centres (A <-> B).
#include "kernels.h"

namespace km {
namespace {

constexpr int kPPMaxTrials = 16;
constexpr int kPPRowsPerBlock = 64; // samples per block of pp_dist_kernel

struct PPState {
    double pot;  // potential of the chosen candidate
    int best;    // its trial index
};

// X[i, f .. f+3] with zeros for i >= n or features >= d. kVec: X is 16-byte
// aligned and d % 4 == 0, so the four values are one 16-byte load. kNT: a
// non-temporal load (the samples stream through once per centre; the
// candidate rows, read by every block, keep ordinary loads): 3 % less time
// per centre at 65536 x 8192, same bits.
template <bool kVec, bool kNT = false>
__device__ __forceinline__ float4 load_row4(const float *__restrict__ X, int64_t n, int64_t d,
                                            int64_t i, int64_t f) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i >= n) return v;
    const float *p = X + i * d + f;
    if (kVec) {
        if (f < d) {
            if (kNT) {
                typedef float f4v __attribute__((ext_vector_type(4)));
                const f4v t = __builtin_nontemporal_load((const f4v *)p);
                v = make_float4(t.x, t.y, t.z, t.w);
            } else {
                v = *(const float4 *)p;
            }
        }
    } else {
        if (f < d) v.x = p[0];
        if (f + 1 < d) v.y = p[1];
        if (f + 2 < d) v.z = p[2];
        if (f + 3 < d) v.w = p[3];
    }
    return v;
}

// |x_i|^2 in float64 (exact float32 squares, float64 sums in a fixed order),
// one wave per sample, 4 samples per 256-thread block.
__global__ __launch_bounds__(256) void pp_norm_kernel(const float *__restrict__ X, int64_t n,
                                                     int64_t d, double *__restrict__ xnorm) {
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= n) return;  // whole wave
    const float *x = X + i * d;
    double acc = 0.0;
    for (int64_t f = lane; f < d; f += 64) {
        const double v = (double)x[f];
        acc = __builtin_fma(v, v, acc);
    }
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) xnorm[i] = acc;
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float f4_at(const float4 &v, int e) {
    return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

// Every sample against up to 16 candidates with float64 matrix cores
// (v_mfma_f64_16x16x4_f64: D(16 x 16) += A(16 x 4) B(4 x 16)). A block holds
// 64 samples, 16 per wave; a wave's tile is its 16 samples x the 16 candidate
// slots (slots >= trials are zero), so one 16 x 16 float64 accumulator (4
// values per lane) carries whole dot products and no cross-lane sum is
// needed. Features go in stages of kMfF; inside a stage, k-group g (lanes
// 16g .. 16g+15) takes the contiguous features g * kMfRun .. +kMfRun, one per
// MFMA step (the same order for samples and candidates). Samples are loaded
// coalesced (whole 512-byte row pieces per half-wave) one stage ahead into
// registers and turned round through the wave's own LDS slice, which needs no
// barrier because a wave's LDS operations run in order; candidates are staged
// in shared, double-buffered LDS. Registers carry no accumulators but the 4
// per lane, which leaves room for the next stage's samples in flight: with
// three blocks per CU, 96 KiB of samples per CU.
// Output layout (probed on the chip): lane l, value i is sample (l / 16) +
// 4 i of the wave's 16, candidate slot l % 16.
//
// With at most 12 trials (kQuad, kSlots = 8 or 12; 8 at the pages' k = 1024)
// a quarter to a half of those 16 slots would multiply zeros, so the product
// runs on v_mfma_f64_4x4x4_4b_f64 instead: four independent 4 x 4 x 4 blocks
// per instruction, a quarter of the 16 x 16 x 4 work. Its layout (probed on the
// chip): lane 16k + 4b + i holds A[b][i][k], lane 16k + 4b + j holds
// B[b][k][j], and lane 16i + 4b + j receives D[b][i][j]. The four blocks take
// the same 4 samples and 4 candidates over four different feature
// sub-ranges: a stage's 128 features are split into 16 runs of 8, lane
// 16k + 4b + i taking run sigma(b, k) for both operands, and block b's
// partial products are summed over the blocks at the end. Per feature step a
// wave issues 4 H instructions: sample group g = 0 .. 3 (samples 4g + i) x
// candidate group h < H = kSlots / 4 (candidates 4h + j). Every lane thus
// reads from LDS only the operands it uses: its 8 features of 4 samples and
// H candidates per stage (had the blocks taken four sample groups against
// the same candidates, each lane would read the candidates four times over:
// measured 4 % slower per seeding at 65536 x 8192, k = 1024, same centres).
// After the sum, lane l keeps sample 4 ((l / 4) % 4) + l / 16 against
// candidates 4h + l % 4. At 9 to 11 trials the 12-slot instance takes
// 367-373 us per centre at 65536 x 8192 against 391-397 for the 16 x 16
// product, with the same chosen centres.
constexpr int kMfF = 128;           // features per stage
constexpr int kMfRun = kMfF / 4;    // contiguous features per lane per stage
constexpr int kMfLdk = kMfF + 4;    // padded LDS row of a candidate

template <bool kVec, int kSlots, bool kQuad>
__global__ __launch_bounds__(256, 3) void pp_dist_kernel(
    const float *__restrict__ X, const double *__restrict__ xnorm, int64_t n, int64_t d,
    int trials, const long long *__restrict__ cand, const PPState *__restrict__ st,
    const double *__restrict__ prev_buf, double *__restrict__ out_buf,
    double *__restrict__ out_parts, int64_t nb) {
    __shared__ __attribute__((aligned(16))) float cs[2][16][kMfLdk];
    __shared__ __attribute__((aligned(16))) float xw[4][16][kMfLdk];  // per wave
    __shared__ double wpart[4][16];
    __shared__ double cand_norm[16];
    __shared__ long long cand_row[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t b = blockIdx.x;
    const double *closest = prev_buf ? prev_buf + (int64_t)st->best * n : nullptr;
    const int grp = lane >> 4;  // k-group of this lane's MFMA operands
    const int64_t row0 = b * kPPRowsPerBlock + wave * 16;
    const int64_t chunks = (d + kMfF - 1) / kMfF;
    if (tid < 16) {
        cand_row[tid] = tid < trials ? cand[tid] : -1;
        cand_norm[tid] = tid < trials ? xnorm[cand[tid]] : 0.0;
    }
    // Candidate staging: thread tid moves 8 features (two 16-byte pieces) of
    // candidate slot tid / 16 per stage.
    const int c_slot = tid >> 4, c_off = (tid & 15) * 8;
    const long long c_row = c_slot < trials ? cand[c_slot] : -1;

    // Sample staging, coalesced: piece e = lane + 64 q (q < 8) of the wave's
    // 16 rows x kMfF features is row e / 32, features 4 (e % 32) .. +3.
    auto load_x = [&](int64_t c, float4 (&xv)[8]) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int e = lane + 64 * q;
            xv[q] = load_row4<kVec, true>(X, n, d, row0 + (e >> 5), c * kMfF + 4 * (e & 31));
        }
    };
    auto store_x = [&](const float4 (&xv)[8]) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int e = lane + 64 * q;
            *reinterpret_cast<float4 *>(&xw[wave][e >> 5][4 * (e & 31)]) = xv[q];
        }
    };
    auto load_c = [&](int64_t c, float4 (&cv)[2]) {
        const int64_t f = c * kMfF + c_off;
#pragma unroll
        for (int q = 0; q < 2; ++q)
            cv[q] = c_row >= 0 ? load_row4<kVec>(X, n, d, c_row, f + 4 * q)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    auto store_c = [&](int buf, const float4 (&cv)[2]) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
            *reinterpret_cast<float4 *>(&cs[buf][c_slot][c_off + 4 * q]) = cv[q];
    };

    float4 xn[8], cv[2];
    // Block b walks the feature stages from stage 5b mod chunks (wrapping
    // round), so the blocks in flight read different column strips of X at
    // any moment rather than all the same one: 1 % faster at 65536 x 8192.
    // The float64 sums then run in that rotated stage order, the same on
    // every call.
    const int64_t rot = (b * 5) % chunks;
    load_x(rot, xn);
    load_c(rot, cv);
    store_x(xn);
    store_c(0, cv);
    __syncthreads();

    f64x4 acc = {0.0, 0.0, 0.0, 0.0};  // !kQuad (16 slots)
    // kQuad: with l = 16 i + 4 b + j (the output layout), block b's partial
    // product of sample 4 g + i against candidate 4 h + j.
    constexpr int H = kQuad ? kSlots / 4 : 1;
    double acc8[4][H];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int h = 0; h < H; ++h) acc8[g][h] = 0.0;
    // Its operands (l = 16 k + 4 b + i): the 8 features 8 sigma(b, k) .. + 7
    // of the stage, sigma(b, k) = 2 b + k % 2 + 8 (k / 2), a permutation of
    // 0 .. 15 that puts the 16-byte reads of 16 consecutive lanes on
    // distinct banks (rows 132 floats apart: a row shifts the banks by 4).
    const int sig8 = 8 * (2 * ((lane >> 2) & 3) + (grp & 1) + 8 * (grp >> 1));
    for (int64_t c = 0; c < chunks; ++c) {
        const int cur = (int)(c & 1);
        // This lane's operands of the stage: samples from its own wave's
        // slice (the wave's LDS operations run in order, so the slice can be
        // rewritten below without a barrier), candidates (kQuad) from the
        // shared buffer the last barrier published.
        float4 xa[kMfRun / 4];
        float4 xa8[4][2], cb8[H][2];
        if constexpr (!kQuad) {
            const float *arow = &xw[wave][lane & 15][grp * kMfRun];
#pragma unroll
            for (int q = 0; q < kMfRun / 4; ++q) xa[q] = *reinterpret_cast<const float4 *>(arow + 4 * q);
        } else {
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    xa8[g][hh] = *reinterpret_cast<const float4 *>(&xw[wave][4 * g + (lane & 3)][sig8 + 4 * hh]);
#pragma unroll
            for (int h = 0; h < H; ++h)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    cb8[h][hh] = *reinterpret_cast<const float4 *>(&cs[cur][4 * h + (lane & 3)][sig8 + 4 * hh]);
        }
        if (c + 1 < chunks) {
            const int64_t next = (c + 1 + rot) % chunks;
            load_x(next, xn);
            load_c(next, cv);
        }
        // Features beyond d were loaded as 0 for samples and candidates alike.
        if constexpr (!kQuad) {
            const float *brow = &cs[cur][lane & 15][grp * kMfRun];
#pragma unroll
            for (int q = 0; q < kMfRun / 4; ++q) {
                const float4 bv = *reinterpret_cast<const float4 *>(brow + 4 * q);
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xa[q].x, (double)bv.x, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xa[q].y, (double)bv.y, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xa[q].z, (double)bv.z, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xa[q].w, (double)bv.w, acc, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int st = 0; st < 8; ++st) {
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int h = 0; h < H; ++h)
                        acc8[g][h] = __builtin_amdgcn_mfma_f64_4x4x4f64(
                            (double)f4_at(xa8[g][st >> 2], st & 3), (double)f4_at(cb8[h][st >> 2], st & 3),
                            acc8[g][h], 0, 0, 0);
            }
        }
        if (c + 1 < chunks) {
            store_x(xn);
            store_c(cur ^ 1, cv);
        }
        __syncthreads();
    }

    // D for this lane's samples against its candidate slots; the sample that
    // is the candidate itself gets exactly 0.
    auto dist_of = [&](int64_t gi, int t, double dot) {
        const double dist =
            gi == cand_row[t] ? 0.0 : __builtin_fma(-2.0, dot, xnorm[gi] + cand_norm[t]);
        const double pos = dist > 0.0 ? dist : 0.0;
        const double cur_d = closest ? closest[gi] : __builtin_inf();
        const double nd = pos < cur_d ? pos : cur_d;
        out_buf[(int64_t)t * n + gi] = nd;
        return nd;
    };
    if constexpr (!kQuad) {
        // Lane l: samples l / 16 + 4 i against slot l % 16.
        const int t = lane & 15;
        double part = 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t gi = row0 + grp + 4 * i;
            if (t < trials && gi < n) part += dist_of(gi, t, acc[i]);
        }
        // The four lanes of candidate t (t, t + 16, t + 32, t + 48), then
        // the waves in order.
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        if (lane < 16) wpart[wave][lane] = part;
    } else {
        // Lane l: sample 4 ((l / 4) % 4) + l / 16 against slots 4h + l % 4;
        // the 16 lanes of a slot differ in bits 2 .. 5.
        const int gsel = (lane >> 2) & 3;
        const int64_t gi = row0 + 4 * gsel + grp;
        double part[H];
#pragma unroll
        for (int h = 0; h < H; ++h) {
            // Sum over the blocks (lanes differing in bits 2 and 3): every lane
            // adds (b0 + b1) + (b2 + b3), so all four hold the same bits.
            double red[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                double v = acc8[g][h];
                v += __shfl_xor(v, 4);
                v += __shfl_xor(v, 8);
                red[g] = v;
            }
            const double dot = gsel == 0 ? red[0] : gsel == 1 ? red[1] : gsel == 2 ? red[2] : red[3];
            const int t = 4 * h + (lane & 3);
            part[h] = (t < trials && gi < n) ? dist_of(gi, t, dot) : 0.0;
#pragma unroll
            for (int o = 4; o < 64; o <<= 1) part[h] += __shfl_xor(part[h], o);
        }
        if (lane < 4) {
#pragma unroll
            for (int h = 0; h < H; ++h) wpart[wave][4 * h + lane] = part[h];
        }
    }
    __syncthreads();
    if (tid < trials)
        out_parts[(int64_t)tid * nb + b] = ((wpart[0][tid] + wpart[1][tid]) + wpart[2][tid]) + wpart[3][tid];
}

template <int kSlots, bool kQuad>
void launch_dist_slots(bool vec, int trials, unsigned nb, hipStream_t stream, const float *X,
                       const double *xnorm, int64_t n, int64_t d, const long long *cand,
                       const PPState *st, const double *prev, double *out, double *parts) {
    if (vec)
        pp_dist_kernel<true, kSlots, kQuad><<<nb, 256, 0, stream>>>(X, xnorm, n, d, trials, cand, st,
                                                             prev, out, parts, nb);
    else
        pp_dist_kernel<false, kSlots, kQuad><<<nb, 256, 0, stream>>>(X, xnorm, n, d, trials, cand, st,
                                                              prev, out, parts, nb);
}

void launch_dist(int trials, bool vec, unsigned nb, hipStream_t stream, const float *X,
                 const double *xnorm, int64_t n, int64_t d, const long long *cand,
                 const PPState *st, const double *prev, double *out, double *parts) {
    // Up to 12 trials: 4 x 4 blocks, 2 or 3 candidate groups. 13 to 16: the
    // 16 x 16 product (16 candidate slots on the 4 x 4 blocks take more
    // registers than three blocks per CU allow, and spill: 50 % slower).
    if (trials <= 8)
        launch_dist_slots<8, true>(vec, trials, nb, stream, X, xnorm, n, d, cand, st, prev, out, parts);
    else if (trials <= 12)
        launch_dist_slots<12, true>(vec, trials, nb, stream, X, xnorm, n, d, cand, st, prev, out, parts);
    else
        launch_dist_slots<16, false>(vec, trials, nb, stream, X, xnorm, n, d, cand, st, prev, out,
                                     parts);
}

constexpr int kSelWaves = 16;  // pp_select_kernel: one 1024-thread block

// Winner of the previous trials, recorded as centre c_rec; then, if rand_row
// is not NULL, the next candidates. One block of 1024 threads; every sum has
// a fixed order.
__global__ __launch_bounds__(kSelWaves * 64) void pp_select_kernel(
    int64_t n, const double *__restrict__ prev_buf, const double *__restrict__ prev_parts,
    int64_t nb, int trials_prev,
    const long long *__restrict__ cand_prev, PPState *st, int64_t c_rec,
    long long *__restrict__ chosen, const double *__restrict__ rand_row, int trials_next,
    long long *__restrict__ cand_next) {
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

namespace {

// centres[c] = X[chosen[c]] for every centre, a block per centre; each
// thread's loads go out before its stores (the row copies leave the
// per-centre chain of launches, where each would be one more memory round
// trip per centre).
__global__ __launch_bounds__(256) void pp_gather_kernel(const float *__restrict__ X, int64_t d,
                                                        const int64_t *__restrict__ chosen,
                                                        float *__restrict__ centres) {
    constexpr int kU = 8;
    const int64_t c = blockIdx.x;
    const float *src = X + chosen[c] * d;
    float *dst = centres + c * d;
    for (int64_t f0 = 0; f0 < d; f0 += 256 * kU) {
        float v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t f = f0 + u * 256 + threadIdx.x;
            v[u] = src[f < d ? f : d - 1];  // clamped, so the loads carry no condition
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t f = f0 + u * 256 + threadIdx.x;
            if (f < d) dst[f] = v[u];
        }
    }
}

}  // namespace

int64_t pp_blocks(int64_t n) { return cdiv(n, kPPRowsPerBlock); }
int pp_max_trials() { return kPPMaxTrials; }
int pp_block_threads() { return 256; }
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
            n, buf[cur], parts[cur], nb, trials_prev, cand[cur], st, c - 1,
            (long long *)chosen, more ? rand + (c - 1) * trials : nullptr, trials, cand[cur ^ 1]);
        if (!more) break;
        launch_dist(trials, vec, (unsigned)nb, stream, X, ws.xnorm, n, d, cand[cur ^ 1], st,
                    buf[cur], buf[cur ^ 1], parts[cur ^ 1]);
        cur ^= 1;
        trials_prev = trials;
    }
    pp_gather_kernel<<<(unsigned)k, 256, 0, stream>>>(X, d, chosen, centres);
    return hipGetLastError();
}

}  // namespace km
