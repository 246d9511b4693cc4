/*
 * kmeans_mi355x.h - C ABI of the MI355X (gfx950) nearest-centroid assignment
 * and Lloyd centroid update.
 *
 * Operations (pages: "Three shapes that fit an eager Gram assignment",
 * "Fusion probe", "004 - tile sizes, a Cython Lloyd step, and k-means++"):
 *
 *   assign  labels[i] = argmin_j ||x_i - c_j||^2, computed in Gram form as the
 *           argmin of ||c_j||^2 - 2 x_i.c_j (the Gram identity of "Three
 *           shapes ...", section Gram assignment, with ||x||^2 dropped inside
 *           the tile as in "004 ...", section Schedules added). Exact ties go
 *           to the lowest index. min_dist[i] = max(0, ||x_i||^2 + that
 *           minimum) is the full squared distance, the running winning
 *           distance of "Three shapes ...", section Running argmin.
 *   update  counts[j] = #{i : labels[i] = j}; C_new[j] = mean of those x_i;
 *           a cluster with no sample keeps C_old[j] ("Three shapes ...",
 *           section Full Lloyd step; "004 ...", section Lloyd step).
 *   lloyd   assign against C_old, then update with those labels: one Lloyd
 *           iteration ("004 ...", sections Lloyd step and Cython reference).
 *
 * Common conventions
 *   - Every array pointer is a DEVICE pointer owned by the caller. Matrices are
 *     row-major and dense: X is (n, d) float32, C / C_old / C_new are (k, d)
 *     float32, labels is (n,) int64, counts is (k,) int64, min_dist is (n,)
 *     float32. The library never allocates, frees or keeps device memory.
 *   - workspace is a caller-owned device buffer of at least
 *     kmeans_workspace_bytes(n, k, d, op) bytes, any alignment. Its contents
 *     on entry do not matter; it is clobbered. Two calls that may run at the
 *     same time need two workspaces.
 *   - stream is a hipStream_t (NULL = the default stream). Every call except
 *     kmeans_fit (see there) only enqueues kernels on it and returns: no host
 *     synchronisation, no memset, no copy. Results are ready when the stream
 *     has reached that point. Such a call can also be captured into a HIP
 *     graph and replayed; a replay reads the buffers' contents at replay
 *     time. A fault inside a kernel surfaces at the caller's next
 *     synchronisation, not as a return value.
 *   - Shapes: 0 <= n < 2^31, 1 <= k < 2^31, 1 <= d < 2^31. With n = 0 nothing
 *     is read from X, labels or min_dist (they may be NULL). k > n is allowed.
 *     A shape whose launch grid would exceed 2^32 - 1 work-items in one
 *     dimension (for the assignment roughly n * k > 2^38 with the tile chosen
 *     for large problems) returns KM_ERR_SHAPE.
 *   - Inputs must be finite; NaN or Inf inputs give unspecified labels.
 *   - Outputs must not overlap any input, any other output or the workspace,
 *     with one exception: C_new may equal C_old exactly (in-place update).
 *   - Arguments are validated on the host before any HIP call; an invalid
 *     call returns a negative km_status and enqueues nothing.
 *   - Arithmetic: float32 MFMA products with float32 accumulation for the
 *     assignment; per-cluster sums accumulated in float64 (in increasing
 *     sample order for a cluster of at most 64 samples, or 128 when
 *     n * d >= 2^26 and n >= 32 k; as sixteen contiguous parts of its
 *     samples, added in order, for a larger one),
 *     divided in float64 and rounded once to float32. Every reduction has a fixed
 *     order: the same inputs give the same bits.
 */
#ifndef KMEANS_MI355X_H
#define KMEANS_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
typedef enum {
    KM_OK = 0,
    KM_ERR_NULL = -1,      /* a required pointer is NULL                          */
    KM_ERR_SHAPE = -2,     /* n, k or d outside the documented range              */
    KM_ERR_ALIGN = -3,     /* a pointer is not aligned to its element size        */
    KM_ERR_WORKSPACE = -4, /* workspace_bytes < kmeans_workspace_bytes(...)       */
    KM_ERR_ALIAS = -5,     /* an output overlaps an input, output or workspace    */
    KM_ERR_HIP = -6,       /* a kernel launch was rejected by the HIP runtime     */
    KM_ERR_OP = -7,        /* unknown op code or flag                             */
    KM_ERR_SCRATCH = -8    /* kmeans_lloyd_step_noalloc: the shape needs more than
                              KM_NOALLOC_SCRATCH_BYTES of scratch                 */
} km_status;

/* Op codes for kmeans_workspace_bytes. */
enum { KM_OP_ASSIGN = 0, KM_OP_UPDATE = 1, KM_OP_LLOYD = 2, KM_OP_FIT = 3, KM_OP_KMEANSPP = 4 };

/* Flags for kmeans_fit. */
enum { KM_FIT_RELOCATE_EMPTY = 1 };

/*
 * Workspace bytes needed by one call of the given op at shape (n, k, d).
 * The size is O(k + n + k * ceil(n / 1024)) 4-byte words, plus about
 * k * d / 4096 + 256 doubles for kmeans_fit (per-block partial sums of the
 * centre shift), n doubles, n floats and 12 bytes per entry of a sort buffer
 * of the next power of two >= min(n, k) entries (relocation and min_dist
 * scratch), and, when ceil(d / 256) <= k / 16,
 * n * ceil(d / 256) floats for kmeans_lloyd_step (partial squared norms of
 * the rows: at most 1/256 of the size of X and 1/16 of an (n, k) matrix):
 * far below the (n, k) distance matrix and the (n, d) sample matrix.
 * Returns 0 when the shape or op is invalid or the shape's launch grid does
 * not fit (a valid shape never needs 0 bytes).
 */
size_t kmeans_workspace_bytes(int64_t n, int64_t k, int64_t d, int op);

/*
 * Nearest-centroid assignment ("Three shapes ...", section Gram assignment).
 *   X         (n, d) float32 samples, read only.
 *   C         (k, d) float32 centroids, read only.
 *   labels    (n,) int64 output: the lowest j minimising ||x_i - c_j||^2
 *             (Gram form, float32). Also used as scratch during the call.
 *   min_dist  (n,) float32 output, or NULL to skip it: the squared distance to
 *             the chosen centroid, clamped at 0.
 * Neither an (n, k) distance matrix nor an (n, d) temporary is ever written.
 */
int kmeans_assign(const float *X, const float *C, int64_t n, int64_t k, int64_t d,
                  int64_t *labels, float *min_dist,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Centroid update for fixed labels ("Three shapes ...", section Full Lloyd
 * step; "004 ...", section Lloyd step).
 *   X       (n, d) float32 samples, read only.
 *   labels  (n,) int64, read only. A row whose label lies outside [0, k) is
 *           ignored: it is counted nowhere and added to no sum.
 *   C_old   (k, d) float32, read only: the centre kept by an empty cluster.
 *   C_new   (k, d) float32 output (may be the same pointer as C_old).
 *   counts  (k,) int64 output.
 */
int kmeans_update(const float *X, const int64_t *labels, const float *C_old,
                  int64_t n, int64_t k, int64_t d,
                  float *C_new, int64_t *counts,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * One Lloyd iteration: kmeans_assign against C_old, then kmeans_update with
 * the labels just computed ("004 ...", sections Lloyd step and Cython
 * reference). Arguments as in those two calls; labels are with respect to
 * C_old. C_new may be the same pointer as C_old. min_dist is the same
 * quantity as kmeans_assign's. When ceil(d / 256) <= k / 16 the squared
 * sample norms in it are gathered by the update while it reads X (float32
 * partial sums over 256-column chunks, combined in float64), so X is read
 * twice per step instead of three times; otherwise a separate pass computes
 * them as in kmeans_assign.
 */
int kmeans_lloyd_step(const float *X, const float *C_old, int64_t n, int64_t k, int64_t d,
                      int64_t *labels, float *min_dist, float *C_new, int64_t *counts,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * kmeans_lloyd_step for callers that cannot allocate device memory at all
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels and results, but no workspace argument. The
 * scratch lives in a static device array of KM_NOALLOC_SCRATCH_BYTES bytes
 * that each GPU the library runs on holds from the library's first use on it
 * until the process ends; its address is looked up once per device on the
 * first call there. Nothing is allocated or freed by the call itself.
 *   Shapes whose kmeans_workspace_bytes(n, k, d, KM_OP_LLOYD) exceeds
 *   KM_NOALLOC_SCRATCH_BYTES return KM_ERR_SCRATCH before any HIP call (the
 *   five workloads of the pages need at most about 22 MiB).
 *   The array is shared by every call on a GPU: two calls that may overlap
 *   on one GPU (different streams, or host threads) race on it and give
 *   undefined results; calls on one stream are ordered and safe. Every part
 *   of it a call reads is written earlier in the same call.
 *   The scratch is on the device of `stream` (the current device for NULL).
 * Other arguments, checks and return codes as in kmeans_lloyd_step.
 */
#define KM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int kmeans_lloyd_step_noalloc(const float *X, const float *C_old, int64_t n, int64_t k,
                              int64_t d, int64_t *labels, float *min_dist, float *C_new,
                              int64_t *counts, void *stream);

/*
 * Lloyd iterations from C_init: assignment, optional empty-cluster
 * relocation, update, repeated until the centre shift
 * sum_j ||C_new_j - C_old_j||^2 (float64) is <= tol or max_iter iterations
 * ran; then one more assignment against the final centres ("004 ...",
 * sections Lloyd step and Cython timing, whose Lloyd call updates the
 * centres and relocates empty clusters).
 *   max_iter  >= 1.
 *   tol       convergence threshold on the centre shift (not NaN).
 *   flags     0, or KM_FIT_RELOCATE_EMPTY: after each assignment, the
 *             min(#empty, n) samples farthest from their assigned centre
 *             (float64 distance; lower index first on ties) each become the
 *             only member of the next empty cluster in increasing index.
 *             Without it (and for a cluster a move empties) an empty
 *             cluster keeps its centre.
 *   C_out     (k, d) float32 output: the final centres. May equal C_init.
 *   labels    (n,) int64 output: assignment against the final centres.
 *   min_dist  (n,) float32 output or NULL: squared distances of that
 *             assignment (as in kmeans_assign).
 *   counts    (k,) int64 output: cluster sizes of those labels.
 *   info      device array of 3 doubles, output: iterations run, inertia
 *             (sum of the final squared distances, float64), and the centre
 *             shift of the last iteration.
 * Synchronisation: iterations are enqueued in batches, 4 first, then 8;
 * between batches the call waits on `stream` to read a 4-byte convergence
 * flag back to the host (the only entry point that ever waits). Iterations
 * enqueued after the one that converged do nothing on the GPU: every kernel
 * of an iteration returns at once once the flag is set. With max_iter <= 4
 * the call never waits.
 */
int kmeans_fit(const float *X, const float *C_init, int64_t n, int64_t k, int64_t d,
               int64_t max_iter, double tol, int flags,
               float *C_out, int64_t *labels, float *min_dist, int64_t *counts, double *info,
               void *workspace, size_t workspace_bytes, void *stream);

/*
 * Greedy k-means++ seeding ("004 ...", section k-means++: 2 + log(k) trials
 * per centre). chosen[0] = first. With D(i) the squared distance of sample i
 * to its nearest chosen centre and pot = sum_i D(i), each further centre c
 * draws `trials` candidates: trial t takes the first sample whose running
 * sum of D reaches rand[(c - 1) * trials + t] * pot (the last sample if none
 * does); the candidate with the smallest potential sum_i min(D(i),
 * |x_i - x_cand|^2) (lowest trial on ties) becomes centre c. Distances are
 * float64 in Gram form, |x|^2 + |c|^2 - 2 x.c clamped at 0, with the sample
 * norms computed once per call (the pages' faster version); the float32
 * products are exact in float64 and a sample's distance to itself is exactly
 * 0. The random draws are an input so that a run is reproducible.
 *   X        (n, d) float32 samples.
 *   k        number of centres, 1 <= k <= n.
 *   first    index of the first centre, 0 <= first < n.
 *   trials   candidates per centre, 1 <= trials <= 16.
 *   rand     device array of (k - 1) * trials float64 uniforms in [0, 1)
 *            (may be NULL when k == 1).
 *   centres  (k, d) float32 output: the chosen rows of X.
 *   chosen   (k,) int64 output: their indices.
 * Asynchronous like kmeans_assign; 2 kernel launches per centre.
 * Workspace: about (2 * 16 + 1) * n doubles (kmeans_workspace_bytes with
 * KM_OP_KMEANSPP).
 */
int kmeans_plusplus(const float *X, int64_t n, int64_t d, int64_t k, int64_t first,
                    int64_t trials, const double *rand, float *centres, int64_t *chosen,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Static, NUL-terminated description of a km_status value (never NULL). */
const char *kmeans_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KMEANS_MI355X_H */
