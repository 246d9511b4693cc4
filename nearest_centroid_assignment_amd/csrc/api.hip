// api.hip - the C ABI declared in include/kmeans_mi355x.h.
//
// Every entry point validates its arguments on the host before the first HIP
// call, carves its sections out of the caller's workspace (or, in
// kmeans_lloyd_step_noalloc, out of the static `scratch` array), and enqueues
// the kernels on the caller's stream. Nothing here allocates or frees device
// memory. kmeans_fit is the one call that may wait on its stream: it reads the
// 4-byte convergence flag back to the host between batches of iterations
// (after the first 4, then every 8). Global state:
// the assignment launcher's cached compute-unit count per device and the
// per-device address of `scratch`.
#include <atomic>

#include "../../include/kmeans_mi355x.h"
#include "kernels.h"

// Scratch of kmeans_lloyd_step_noalloc: one copy per GPU, alive until the
// process ends. In host code `scratch` only names the symbol; its device
// address comes from hipGetSymbolAddress (see noalloc_scratch below) and that
// address is what the kernels get.
__device__ __align__(256) unsigned char scratch[KM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kMaxDim = 2147483647;  // n, k, d < 2^31
constexpr size_t kAlign = 256;           // section alignment inside the workspace
constexpr int64_t kMaxGridThreads = 4294967295LL;  // one dispatch dimension, in work-items

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Whether kmeans_lloyd_step gathers the squared sample norms inside the
// update (n x ceil(d / 256) float32 partials in the workspace) instead of a
// separate pass over X: only while that buffer stays below 1/16 of an (n, k)
// float32 matrix, so the workspace never approaches the distance matrix.
bool lloyd_fuses_norms(int64_t k, int64_t d) { return km::norm_parts(d) * 16 <= k; }

struct Layout {
    size_t cn = 0, tile_hist = 0, rank = 0, cnt = 0, seg_start = 0, perm = 0, big = 0, order = 0,
           flags = 0;
    // kmeans_lloyd_step only
    size_t xn_part = 0;
    // kmeans_fit only
    size_t md = 0, dist = 0, empty = 0, sort_key = 0, sort_idx = 0,
           shift_partial = 0, scalars = 0;
    // kmeans_plusplus only
    size_t pp_buf_a = 0, pp_buf_b = 0, pp_parts_a = 0, pp_parts_b = 0, pp_cand_a = 0,
           pp_cand_b = 0, pp_state = 0, pp_xnorm = 0;
    size_t total = 0;
};

// Offsets from the first 256-byte boundary at or after the workspace start;
// total includes that much slack so any base alignment works.
Layout layout(int64_t n, int64_t k, int64_t d, int op) {
    Layout L;
    size_t off = 0;
    if (op == KM_OP_ASSIGN || op == KM_OP_LLOYD || op == KM_OP_FIT) {
        L.cn = off;
        off += round_up((size_t)k * sizeof(float));
    }
    if (op == KM_OP_UPDATE || op == KM_OP_LLOYD || op == KM_OP_FIT) {
        const int64_t n_tiles = cdiv(n, km::kSortTileRows);
        L.tile_hist = off;
        off += round_up((size_t)k * (size_t)n_tiles * sizeof(int));
        L.cnt = off;
        off += round_up((size_t)k * sizeof(int));
        L.seg_start = off;
        off += round_up((size_t)k * sizeof(int));
        L.perm = off;
        off += round_up((size_t)n * sizeof(int));
        L.big = off;
        off += round_up(((size_t)k + 1) * sizeof(int));
        L.order = off;
        off += round_up((size_t)k * sizeof(int));
        L.rank = off;
        off += round_up((size_t)n * sizeof(unsigned short));
        L.flags = off;  // no-empty flag
        off += round_up(sizeof(int));
    }
    if (op == KM_OP_LLOYD && lloyd_fuses_norms(k, d)) {
        L.xn_part = off;
        off += round_up((size_t)n * (size_t)km::norm_parts(d) * sizeof(float));
    }
    if (op == KM_OP_FIT) {
        const int64_t cap = km::reloc_sort_cap(n, k);
        L.md = off;
        off += round_up((size_t)n * sizeof(float));
        L.dist = off;
        off += round_up((size_t)n * sizeof(double));
        L.empty = off;
        off += round_up((size_t)k * sizeof(int));
        L.sort_key = off;
        off += round_up((size_t)cap * sizeof(unsigned long long));
        L.sort_idx = off;
        off += round_up((size_t)cap * sizeof(int));
        L.shift_partial = off;
        off += round_up((size_t)km::mean_blocks(k, d) * sizeof(double));
        L.scalars = off;  // num_empty, converged
        off += round_up(4 * sizeof(int));
    }
    if (op == KM_OP_KMEANSPP) {
        const size_t t = (size_t)km::pp_max_trials();
        const size_t nb = (size_t)km::pp_blocks(n);
        L.pp_buf_a = off;
        off += round_up(t * (size_t)n * sizeof(double));
        L.pp_buf_b = off;
        off += round_up(t * (size_t)n * sizeof(double));
        L.pp_parts_a = off;
        off += round_up(t * nb * sizeof(double));
        L.pp_parts_b = off;
        off += round_up(t * nb * sizeof(double));
        L.pp_cand_a = off;
        off += round_up(t * sizeof(int64_t));
        L.pp_cand_b = off;
        off += round_up(t * sizeof(int64_t));
        L.pp_state = off;
        off += round_up(km::pp_state_bytes());
        L.pp_xnorm = off;
        off += round_up((size_t)n * sizeof(double));
    }
    L.total = off + kAlign;
    return L;
}

bool shape_ok(int64_t n, int64_t k, int64_t d) {
    return n >= 0 && n <= kMaxDim && k >= 1 && k <= kMaxDim && d >= 1 && d <= kMaxDim;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi); empty when lo == hi
};

Range range(const void *p, int64_t count, size_t elem) {
    const uintptr_t lo = (uintptr_t)p;
    return Range{lo, p ? lo + (uintptr_t)count * elem : lo};
}

bool overlap(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

char *ws_base(void *workspace) {
    const uintptr_t p = (uintptr_t)workspace;
    return (char *)((p + kAlign - 1) / kAlign * kAlign);
}

bool grid_ok(int64_t n, int64_t k, int64_t d) {
    return km::assign_grid_threads(n, k, d) <= kMaxGridThreads &&
           km::update_grid_threads(n, k, d) <= kMaxGridThreads;
}

// An array argument: pointer, element count, element size.
struct Out {
    const void *p;
    int64_t count;
    size_t elem;
};

// Output `inplace_out` may coincide exactly with input `inplace_in` (C_new and
// C_old); -1 disables the exception.
int check_alias(const Out *outs, int n_outs, const Out *ins, int n_ins, int inplace_out,
                int inplace_in) {
    for (int i = 0; i < n_outs; ++i) {
        const Range ri = range(outs[i].p, outs[i].count, outs[i].elem);
        for (int j = 0; j < n_ins; ++j) {
            if (i == inplace_out && j == inplace_in && outs[i].p == ins[j].p) continue;
            if (overlap(ri, range(ins[j].p, ins[j].count, ins[j].elem))) return KM_ERR_ALIAS;
        }
        for (int j = i + 1; j < n_outs; ++j)
            if (overlap(ri, range(outs[j].p, outs[j].count, outs[j].elem))) return KM_ERR_ALIAS;
    }
    return KM_OK;
}

// The assignment. With min_dist and add_norm, min_dist receives the full
// squared distance (a separate pass computes ||x||^2 first); with min_dist
// and !add_norm it receives only the best ||c||^2 - 2 x.c, and the caller
// adds ||x||^2 later (the Lloyd step gets it from the update's reads of X).
// With count_ws the finalize also takes the update's first counting step on
// the labels it writes (per-tile histograms and ranks into count_ws). Every
// kernel is gated by `gate` (the assignment's product kernel by gate.a).
int run_assign(const float *X, const float *C, int64_t n, int64_t k, int64_t d, int64_t *labels,
               float *min_dist, bool add_norm, float *cn, const km::UpdateScratch *count_ws,
               km::Gate gate, hipStream_t s) {
    hipError_t e = km::launch_row_sqnorms(C, k, d, cn, s, gate);
    if (e == hipSuccess && !km::assign_stores_keys(X, C, n, k, d))
        e = km::launch_fill_keys((unsigned long long *)labels, n, s, gate);
    if (e == hipSuccess && min_dist && add_norm)
        e = km::launch_row_sqnorms(X, n, d, min_dist, s, gate);
    if (e == hipSuccess)
        e = km::launch_assign_tiles(X, C, cn, n, k, d, (unsigned long long *)labels, s, gate.a);
    if (e == hipSuccess)
        e = count_ws ? km::launch_finalize_rank_hist((unsigned long long *)labels, min_dist,
                                                     add_norm, n, k, *count_ws, gate, s)
                     : km::launch_finalize((unsigned long long *)labels, min_dist, add_norm, n, k,
                                           s);
    return e == hipSuccess ? KM_OK : KM_ERR_HIP;
}

// Device address of `scratch` on the device of `stream`, looked up once per
// device (with that device current) and cached.
constexpr int kMaxDevices = 64;
std::atomic<void *> g_noalloc_scratch[kMaxDevices];

int noalloc_scratch(hipStream_t stream, void **out) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return KM_ERR_HIP;
    int dev = cur;
    if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return KM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return KM_ERR_HIP;
    void *p = g_noalloc_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return KM_ERR_HIP;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return KM_ERR_HIP;
        if (e != hipSuccess || p == nullptr) return KM_ERR_HIP;
        g_noalloc_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return KM_OK;
}

km::UpdateScratch update_scratch(char *base, const Layout &L, int64_t n) {
    km::UpdateScratch ws;
    ws.tile_hist = (int *)(base + L.tile_hist);
    ws.cnt = (int *)(base + L.cnt);
    ws.seg_start = (int *)(base + L.seg_start);
    ws.perm = (int *)(base + L.perm);
    ws.big = (int *)(base + L.big);
    ws.order = (int *)(base + L.order);
    ws.rank = (unsigned short *)(base + L.rank);
    ws.no_empty = (int *)(base + L.flags);
    ws.n_tiles = cdiv(n, km::kSortTileRows);
    return ws;
}

// Argument checks of the Lloyd step. workspace == NULL means the static
// scratch of kmeans_lloyd_step_noalloc (its size is checked by the caller, and
// it cannot overlap a caller's buffer).
int check_lloyd(const float *X, const float *C_old, int64_t n, int64_t k, int64_t d,
                const int64_t *labels, const float *min_dist, const float *C_new,
                const int64_t *counts, const void *workspace, size_t workspace_bytes) {
    if (!shape_ok(n, k, d) || !grid_ok(n, k, d)) return KM_ERR_SHAPE;
    if (!C_old || !C_new || !counts || (n > 0 && (!X || !labels))) return KM_ERR_NULL;
    if (!aligned(X, 4) || !aligned(C_old, 4) || !aligned(labels, 8) || !aligned(min_dist, 4) ||
        !aligned(C_new, 4) || !aligned(counts, 8))
        return KM_ERR_ALIGN;
    if (workspace_bytes < layout(n, k, d, KM_OP_LLOYD).total) return KM_ERR_WORKSPACE;
    const Out outs[] = {{labels, n, 8},
                        {min_dist, n, 4},
                        {C_new, k * d, 4},
                        {counts, k, 8},
                        {workspace, workspace ? (int64_t)workspace_bytes : 0, 1}};
    const Out ins[] = {{X, n * d, 4}, {C_old, k * d, 4}};
    return check_alias(outs, 5, ins, 2, /*C_new*/ 2, /*C_old*/ 1);
}

// The Lloyd step's kernels, with the workspace sections at `base`.
int run_lloyd(const float *X, const float *C_old, int64_t n, int64_t k, int64_t d,
              int64_t *labels, float *min_dist, float *C_new, int64_t *counts, char *base,
              hipStream_t s) {
    const Layout L = layout(n, k, d, KM_OP_LLOYD);
    // min_dist: the assignment leaves the best ||c||^2 - 2 x.c there; the
    // update, which reads every row of X anyway, gathers the partial squared
    // norms of the rows, and a last pass adds them: X is read twice per
    // step (assignment and update), not three times.
    float *xn_part =
        (min_dist && lloyd_fuses_norms(k, d)) ? (float *)(base + L.xn_part) : nullptr;
    const km::UpdateScratch ws = update_scratch(base, L, n);
    if (n > 0) {
        const int rc = run_assign(X, C_old, n, k, d, labels, min_dist, xn_part == nullptr,
                                  (float *)(base + L.cn), &ws, km::Gate{}, s);
        if (rc != KM_OK) return rc;
    }
    hipError_t e = km::launch_update(X, labels, C_old, n, k, d, C_new, counts, xn_part, n > 0, ws, s);
    if (e == hipSuccess && xn_part) e = km::launch_add_norms(min_dist, xn_part, n, d, ws, s);
    return e == hipSuccess ? KM_OK : KM_ERR_HIP;
}

}  // namespace

extern "C" {

size_t kmeans_workspace_bytes(int64_t n, int64_t k, int64_t d, int op) {
    if (!shape_ok(n, k, d)) return 0;
    if (op < KM_OP_ASSIGN || op > KM_OP_KMEANSPP) return 0;
    // A shape whose launch grid does not fit is unsupported, as in the calls.
    if (op == KM_OP_KMEANSPP ? km::pp_blocks(n) * km::pp_block_threads() > kMaxGridThreads
                             : !grid_ok(n, k, d))
        return 0;
    return layout(n, k, d, op).total;
}

const char *kmeans_status_string(int status) {
    switch (status) {
        case KM_OK: return "ok";
        case KM_ERR_NULL: return "a required pointer is NULL";
        case KM_ERR_SHAPE: return "n, k or d outside the supported range";
        case KM_ERR_ALIGN: return "a pointer is not aligned to its element size";
        case KM_ERR_WORKSPACE: return "workspace smaller than kmeans_workspace_bytes()";
        case KM_ERR_ALIAS: return "an output overlaps an input, another output or the workspace";
        case KM_ERR_HIP: return "the HIP runtime rejected a kernel launch";
        case KM_ERR_OP: return "unknown op code or flag";
        case KM_ERR_SCRATCH:
            return "the shape needs more scratch than the static buffer of "
                   "kmeans_lloyd_step_noalloc holds";
        default: return "unknown status";
    }
}

int kmeans_assign(const float *X, const float *C, int64_t n, int64_t k, int64_t d,
                  int64_t *labels, float *min_dist, void *workspace, size_t workspace_bytes,
                  void *stream) {
    if (!shape_ok(n, k, d) || !grid_ok(n, k, d)) return KM_ERR_SHAPE;
    if (!C || !workspace || (n > 0 && (!X || !labels))) return KM_ERR_NULL;
    if (!aligned(X, 4) || !aligned(C, 4) || !aligned(labels, 8) || !aligned(min_dist, 4))
        return KM_ERR_ALIGN;
    const Layout L = layout(n, k, d, KM_OP_ASSIGN);
    if (workspace_bytes < L.total) return KM_ERR_WORKSPACE;
    const Out outs[] = {{labels, n, 8}, {min_dist, n, 4}, {workspace, (int64_t)workspace_bytes, 1}};
    const Out ins[] = {{X, n * d, 4}, {C, k * d, 4}};
    if (int rc = check_alias(outs, 3, ins, 2, -1, -1)) return rc;
    if (n == 0) return KM_OK;
    char *base = ws_base(workspace);
    return run_assign(X, C, n, k, d, labels, min_dist, true, (float *)(base + L.cn), nullptr,
                      km::Gate{}, (hipStream_t)stream);
}

int kmeans_update(const float *X, const int64_t *labels, const float *C_old, int64_t n, int64_t k,
                  int64_t d, float *C_new, int64_t *counts, void *workspace,
                  size_t workspace_bytes, void *stream) {
    if (!shape_ok(n, k, d) || !grid_ok(n, k, d)) return KM_ERR_SHAPE;
    if (!C_old || !C_new || !counts || !workspace || (n > 0 && (!X || !labels)))
        return KM_ERR_NULL;
    if (!aligned(X, 4) || !aligned(labels, 8) || !aligned(C_old, 4) || !aligned(C_new, 4) ||
        !aligned(counts, 8))
        return KM_ERR_ALIGN;
    const Layout L = layout(n, k, d, KM_OP_UPDATE);
    if (workspace_bytes < L.total) return KM_ERR_WORKSPACE;
    const Out outs[] = {{C_new, k * d, 4}, {counts, k, 8}, {workspace, (int64_t)workspace_bytes, 1}};
    const Out ins[] = {{X, n * d, 4}, {labels, n, 8}, {C_old, k * d, 4}};
    if (int rc = check_alias(outs, 3, ins, 3, /*C_new*/ 0, /*C_old*/ 2)) return rc;
    char *base = ws_base(workspace);
    const hipError_t e = km::launch_update(X, labels, C_old, n, k, d, C_new, counts, nullptr,
                                           false, update_scratch(base, L, n), (hipStream_t)stream);
    return e == hipSuccess ? KM_OK : KM_ERR_HIP;
}

int kmeans_lloyd_step(const float *X, const float *C_old, int64_t n, int64_t k, int64_t d,
                      int64_t *labels, float *min_dist, float *C_new, int64_t *counts,
                      void *workspace, size_t workspace_bytes, void *stream) {
    if (!workspace) return shape_ok(n, k, d) && grid_ok(n, k, d) ? KM_ERR_NULL : KM_ERR_SHAPE;
    if (int rc = check_lloyd(X, C_old, n, k, d, labels, min_dist, C_new, counts, workspace,
                             workspace_bytes))
        return rc;
    return run_lloyd(X, C_old, n, k, d, labels, min_dist, C_new, counts, ws_base(workspace),
                     (hipStream_t)stream);
}

int kmeans_lloyd_step_noalloc(const float *X, const float *C_old, int64_t n, int64_t k,
                              int64_t d, int64_t *labels, float *min_dist, float *C_new,
                              int64_t *counts, void *stream) {
    if (!shape_ok(n, k, d) || !grid_ok(n, k, d)) return KM_ERR_SHAPE;
    if (layout(n, k, d, KM_OP_LLOYD).total > KM_NOALLOC_SCRATCH_BYTES) return KM_ERR_SCRATCH;
    if (int rc = check_lloyd(X, C_old, n, k, d, labels, min_dist, C_new, counts, nullptr,
                             KM_NOALLOC_SCRATCH_BYTES))
        return rc;
    void *ws = nullptr;
    if (int rc = noalloc_scratch((hipStream_t)stream, &ws)) return rc;
    return run_lloyd(X, C_old, n, k, d, labels, min_dist, C_new, counts, ws_base(ws),
                     (hipStream_t)stream);
}

int kmeans_fit(const float *X, const float *C_init, int64_t n, int64_t k, int64_t d,
               int64_t max_iter, double tol, int flags, float *C_out, int64_t *labels,
               float *min_dist, int64_t *counts, double *info, void *workspace,
               size_t workspace_bytes, void *stream) {
    if (!shape_ok(n, k, d) || !grid_ok(n, k, d) || max_iter < 1 || tol != tol)
        return KM_ERR_SHAPE;
    if (flags & ~KM_FIT_RELOCATE_EMPTY) return KM_ERR_OP;
    if (!C_init || !C_out || !counts || !info || !workspace || (n > 0 && (!X || !labels)))
        return KM_ERR_NULL;
    if (!aligned(X, 4) || !aligned(C_init, 4) || !aligned(C_out, 4) || !aligned(labels, 8) ||
        !aligned(min_dist, 4) || !aligned(counts, 8) || !aligned(info, 8))
        return KM_ERR_ALIGN;
    const Layout L = layout(n, k, d, KM_OP_FIT);
    if (workspace_bytes < L.total) return KM_ERR_WORKSPACE;
    const Out outs[] = {{C_out, k * d, 4},   {labels, n, 8}, {min_dist, n, 4},
                        {counts, k, 8},      {info, 3, 8},   {workspace, (int64_t)workspace_bytes, 1}};
    const Out ins[] = {{X, n * d, 4}, {C_init, k * d, 4}};
    if (int rc = check_alias(outs, 6, ins, 2, /*C_out*/ 0, /*C_init*/ 1)) return rc;

    hipStream_t s = (hipStream_t)stream;
    char *base = ws_base(workspace);
    const km::UpdateScratch ws = update_scratch(base, L, n);
    float *cn = (float *)(base + L.cn);
    float *md = min_dist ? min_dist : (float *)(base + L.md);
    int *scalars = (int *)(base + L.scalars);
    km::RelocScratch rs;
    rs.dist = (double *)(base + L.dist);
    rs.empty = (int *)(base + L.empty);
    rs.sort_key = (unsigned long long *)(base + L.sort_key);
    rs.sort_idx = (int *)(base + L.sort_idx);
    rs.num_empty = scalars;
    int *converged = scalars + 1;
    int *iterations = scalars + 2;
    double *shift_partial = (double *)(base + L.shift_partial);
    const bool relocate = (flags & KM_FIT_RELOCATE_EMPTY) != 0;
    // Every kernel of an iteration returns at once once the converged flag
    // is set, so iterations are enqueued in batches and the host reads the
    // flag only between batches (a call of at most kFirstBatch iterations
    // never waits).
    const km::Gate loop{converged, nullptr};

    auto iteration = [&]() -> hipError_t {
        hipError_t e = hipSuccess;
        if (n > 0) {
            if (run_assign(X, C_out, n, k, d, labels, nullptr, true, cn, &ws, loop, s) != KM_OK)
                return hipErrorLaunchFailure;
        } else {
            e = km::launch_rank_hist(labels, n, k, ws, loop, s);
        }
        if (e == hipSuccess)
            e = km::launch_scan(labels, n, k, d, counts, relocate ? rs.num_empty : nullptr, ws,
                                loop, s);
        if (e == hipSuccess && relocate) {
            e = km::launch_relocate(X, C_out, labels, n, k, d, rs, ws, s, loop);
            // Count again only if a cluster was empty (something moved).
            if (e == hipSuccess)
                e = km::launch_count(labels, n, k, d, counts, nullptr, ws,
                                     km::Gate{converged, ws.no_empty}, s);
        }
        if (e == hipSuccess)
            e = km::launch_group_and_mean(X, labels, C_out, n, k, d, C_out, shift_partial, nullptr,
                                          ws, loop, s);
        if (e == hipSuccess)
            e = km::launch_shift(shift_partial, km::mean_blocks(k, d), tol, info + 2, converged,
                                 iterations, s);
        return e;
    };

    constexpr int64_t kFirstBatch = 4, kBatch = 8;
    hipError_t e = km::launch_copy_f32(C_out, C_init, k * d, s);
    if (e == hipSuccess) e = km::launch_zero_i32(scalars, 4, s);
    for (int64_t enqueued = 0; e == hipSuccess && enqueued < max_iter;) {
        const int64_t want = enqueued == 0 ? kFirstBatch : kBatch;
        const int64_t batch = want < max_iter - enqueued ? want : max_iter - enqueued;
        for (int64_t b = 0; b < batch && e == hipSuccess; ++b) e = iteration();
        enqueued += batch;
        if (e != hipSuccess || enqueued >= max_iter) break;
        int host_converged = 0;
        e = hipMemcpyAsync(&host_converged, converged, sizeof(int), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e == hipSuccess && host_converged) break;
    }
    if (e == hipSuccess && n > 0 &&
        run_assign(X, C_out, n, k, d, labels, md, true, cn, &ws, km::Gate{}, s) != KM_OK)
        return KM_ERR_HIP;
    if (e == hipSuccess && n <= 0) e = km::launch_rank_hist(labels, n, k, ws, km::Gate{}, s);
    if (e == hipSuccess) e = km::launch_scan(labels, n, k, d, counts, nullptr, ws, km::Gate{}, s);
    if (e == hipSuccess) e = km::launch_inertia(md, n, info + 1, s);
    if (e == hipSuccess) e = km::launch_store_count(info, iterations, s);
    return e == hipSuccess ? KM_OK : KM_ERR_HIP;
}

int kmeans_plusplus(const float *X, int64_t n, int64_t d, int64_t k, int64_t first,
                    int64_t trials, const double *rand, float *centres, int64_t *chosen,
                    void *workspace, size_t workspace_bytes, void *stream) {
    if (!shape_ok(n, k, d) || n < 1 || k > n || first < 0 || first >= n || trials < 1 ||
        trials > km::pp_max_trials() || km::pp_blocks(n) * km::pp_block_threads() > kMaxGridThreads)
        return KM_ERR_SHAPE;
    if (!X || !centres || !chosen || !workspace || (k > 1 && !rand)) return KM_ERR_NULL;
    if (!aligned(X, 4) || !aligned(rand, 8) || !aligned(centres, 4) || !aligned(chosen, 8))
        return KM_ERR_ALIGN;
    const Layout L = layout(n, k, d, KM_OP_KMEANSPP);
    if (workspace_bytes < L.total) return KM_ERR_WORKSPACE;
    const Out outs[] = {{centres, k * d, 4}, {chosen, k, 8}, {workspace, (int64_t)workspace_bytes, 1}};
    const Out ins[] = {{X, n * d, 4}, {rand, k > 1 ? (k - 1) * trials : 0, 8}};
    if (int rc = check_alias(outs, 3, ins, 2, -1, -1)) return rc;
    char *base = ws_base(workspace);
    km::PPScratch ws;
    ws.buf_a = (double *)(base + L.pp_buf_a);
    ws.buf_b = (double *)(base + L.pp_buf_b);
    ws.parts_a = (double *)(base + L.pp_parts_a);
    ws.parts_b = (double *)(base + L.pp_parts_b);
    ws.cand_a = (int64_t *)(base + L.pp_cand_a);
    ws.cand_b = (int64_t *)(base + L.pp_cand_b);
    ws.state = base + L.pp_state;
    ws.xnorm = (double *)(base + L.pp_xnorm);
    const hipError_t e = km::launch_kmeanspp(X, n, d, k, first, (int)trials, rand, centres, chosen,
                                             ws, (hipStream_t)stream);
    return e == hipSuccess ? KM_OK : KM_ERR_HIP;
}

}  // extern "C"
