/*
 * oracle.c - float64 brute-force CPU oracle for nearest-centroid assignment and
 * the Lloyd centroid update.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code, header or constant
 * with the GPU path and must never be used to produce a product result.
 *
 * What it computes is the plain definition, written out:
 *
 *  - Assignment. The naive formula of the fusion probe ("Fusion probe",
 *    section PyTorch, the naive argmin variant; "Three shapes that fit an eager
 *    Gram assignment", section Shapes): for every sample i and centroid j the
 *    squared distance D_ij = sum_t (x_it - c_jt)^2, taken directly in the
 *    difference form (not the Gram form), every operand widened to double. The
 *    label is the smallest j reaching min_j D_ij: centroids are scanned in
 *    increasing j and only a strictly smaller distance replaces the winner,
 *    the strict-less-than-then-where rule of the running argmin ("Three shapes
 *    ...", section Running argmin, one centroid). The second-smallest value
 *    over the other centroids is returned too, so that a caller can tell how
 *    close a row is to a tie.
 *
 *  - Update. The Lloyd update of "Three shapes ...", section Full Lloyd step,
 *    and of the Cython iteration on "004 - tile sizes ...", section Cython
 *    reference: count_j = number of samples labelled j; sum_j = the sum of those
 *    samples, accumulated in double in increasing sample order; the new centre
 *    is sum_j / count_j (double divide, then rounded to float). A cluster with
 *    no sample keeps its old centre (reading taken where the pages are silent;
 *    the pages' Cython kernel relocates such clusters instead).
 *
 * Threads only split the outer loop (rows for the assignment, feature columns
 * for the update), so every result is independent of the thread count.
 */
#include <math.h>
#include <stdint.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of threads the OpenMP runtime will use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * oracle_assign: X (n, d) and C (k, d) are row-major float32 on the host.
 * Outputs, per sample i:
 *   labels[i]  smallest j with D_ij minimal           (int64)
 *   best[i]    D_i,labels[i]                          (double)
 *   second[i]  min over j != labels[i] of D_ij, +inf when k == 1 (double)
 * best/second may be NULL.
 */
void oracle_assign(const float *X, const float *C, int64_t n, int64_t k, int64_t d,
                   int64_t *labels, double *best, double *second) {
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < n; ++i) {
        const float *x = X + i * d;
        double b1 = INFINITY, b2 = INFINITY;
        int64_t arg = 0;
        for (int64_t j = 0; j < k; ++j) {
            const float *c = C + j * d;
            double s = 0.0;
#pragma omp simd reduction(+ : s)
            for (int64_t t = 0; t < d; ++t) {
                double diff = (double)x[t] - (double)c[t];
                s += diff * diff;
            }
            if (s < b1) {
                b2 = b1;
                b1 = s;
                arg = j;
            } else if (s < b2) {
                b2 = s;
            }
        }
        labels[i] = arg;
        if (best) best[i] = b1;
        if (second) second[i] = b2;
    }
}

/*
 * oracle_update: given labels in [0, k), writes
 *   counts[j]   number of samples with label j        (int64)
 *   sums[j, t]  sum over those samples of x_it, in increasing i (double, k*d)
 *   C_new[j, t] (float)(sums[j, t] / counts[j]), or C_old[j, t] when counts[j] == 0
 * sums is a caller-owned k*d double buffer (the sums are part of what is checked).
 * Returns 0, or -1 when a label lies outside [0, k).
 */
int oracle_update(const float *X, const int64_t *labels, const float *C_old,
                  int64_t n, int64_t k, int64_t d,
                  float *C_new, int64_t *counts, double *sums) {
    for (int64_t i = 0; i < n; ++i)
        if (labels[i] < 0 || labels[i] >= k) return -1;
    for (int64_t j = 0; j < k; ++j) counts[j] = 0;
    for (int64_t i = 0; i < n; ++i) counts[labels[i]] += 1;

    for (int64_t e = 0; e < k * d; ++e) sums[e] = 0.0;

    /* Each thread owns a contiguous range of feature columns and adds the rows
     * in increasing i, so every sums[j, t] is accumulated in sample order. */
#pragma omp parallel
    {
        int64_t nt = 1, me = 0;
#ifdef _OPENMP
        nt = omp_get_num_threads();
        me = omp_get_thread_num();
#endif
        int64_t t0 = d * me / nt, t1 = d * (me + 1) / nt;
        for (int64_t i = 0; i < n; ++i) {
            const float *x = X + i * d;
            double *s = sums + labels[i] * d;
            for (int64_t t = t0; t < t1; ++t) s[t] += (double)x[t];
        }
        for (int64_t j = 0; j < k; ++j) {
            for (int64_t t = t0; t < t1; ++t) {
                if (counts[j] > 0)
                    C_new[j * d + t] = (float)(sums[j * d + t] / (double)counts[j]);
                else
                    C_new[j * d + t] = C_old[j * d + t];
            }
        }
    }
    return 0;
}

/* Squared distance between rows a and b of X in float64, difference form. */
static double row_dist(const float *X, int64_t d, int64_t a, int64_t b) {
    const float *x = X + a * d, *y = X + b * d;
    double s = 0.0;
#pragma omp simd reduction(+ : s)
    for (int64_t t = 0; t < d; ++t) {
        double diff = (double)x[t] - (double)y[t];
        s += diff * diff;
    }
    return s;
}

/*
 * oracle_kmeanspp: greedy k-means++ seeding ("004 - tile sizes ...", section
 * k-means++: 2 + log(k) trials per centre, sample norms computed once in the
 * pages' version; here the plain difference form is used).
 *
 *   chosen[0] = first. D(i) = squared distance of sample i to its nearest
 *   chosen centre; pot = sum_i D(i). For every further centre c, each trial t
 *   draws u = rand[(c-1)*trials + t] in [0, 1) and takes the first sample i
 *   whose running sum D(0) + ... + D(i) reaches u * pot (the last sample if
 *   none does). For each candidate, the potential sum_i min(D(i), dist(i,
 *   candidate)) is computed; the candidate of smallest potential (lowest t on
 *   ties) becomes centre c, and D and pot are updated to it.
 *
 * Scratch: closest (n doubles), cand_d (trials * n doubles), cand (trials),
 * pots (trials). All sums are sequential in sample order.
 */
void oracle_kmeanspp(const float *X, int64_t n, int64_t d, int64_t k, int64_t first,
                     int64_t trials, const double *rand, int64_t *chosen, double *closest,
                     double *cand_d, int64_t *cand, double *pots) {
    chosen[0] = first;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) closest[i] = row_dist(X, d, i, first);
    double pot = 0.0;
    for (int64_t i = 0; i < n; ++i) pot += closest[i];

    for (int64_t c = 1; c < k; ++c) {
        for (int64_t t = 0; t < trials; ++t) {
            const double target = rand[(c - 1) * trials + t] * pot;
            double acc = 0.0;
            int64_t idx = n - 1;
            for (int64_t i = 0; i < n; ++i) {
                acc += closest[i];
                if (acc >= target) {
                    idx = i;
                    break;
                }
            }
            cand[t] = idx;
        }
        for (int64_t t = 0; t < trials; ++t) {
            double *dt = cand_d + t * n;
#pragma omp parallel for schedule(static)
            for (int64_t i = 0; i < n; ++i) {
                const double di = row_dist(X, d, i, cand[t]);
                dt[i] = di < closest[i] ? di : closest[i];
            }
            double p = 0.0;
            for (int64_t i = 0; i < n; ++i) p += dt[i];
            pots[t] = p;
        }
        int64_t best = 0;
        for (int64_t t = 1; t < trials; ++t)
            if (pots[t] < pots[best]) best = t;
        chosen[c] = cand[best];
        pot = pots[best];
        const double *db = cand_d + best * n;
        for (int64_t i = 0; i < n; ++i) closest[i] = db[i];
    }
}
