// calib.hip - calibration kernels for the measurements (not part of the k-means
// path): a streaming copy of known size, whose HBM counters give the scale
// factor of the FETCH_SIZE / WRITE_SIZE counters and the attainable copy
// bandwidth; a streaming read (every byte read once, one float written per
// thread), which gives the attainable read bandwidth, the ceiling of kernels
// that mostly read (the update, the k-means++ distances); and a loop of nothing
// but fp32 MFMAs, which gives the attainable fp32 matrix rate under the clocks
// the chip actually holds.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/km_calib.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void copy_kernel(f32x4 *__restrict__ dst,
                                                   const f32x4 *__restrict__ src, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

// Each thread sums its share of the buffer (8 independent 16-byte loads in
// flight per loop trip) and writes one float, so the reads cannot be dropped.
// kNT: non-temporal loads (the data is not kept in the caches for reuse),
// the fastest way found to stream a buffer that is read once.
template <bool kNT>
__global__ __launch_bounds__(256) void read_kernel(const f32x4 *__restrict__ src, int64_t n,
                                                   float *__restrict__ out) {
    constexpr int U = 8;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    float a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = 0.f;
    int64_t i = tid;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = kNT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    for (; i < n; i += stride) {
        const f32x4 v = src[i];
        a[0] += (v.x + v.y) + (v.z + v.w);
    }
    float t = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) t += a[u];
    out[tid] = t;
}

// Four independent 32x32 accumulators per wave; iters x 4 MFMAs per wave.
__global__ __launch_bounds__(256) void mfma_f32_loop_kernel(float *__restrict__ out, int iters,
                                                            float seed) {
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    float a = seed * (float)(threadIdx.x + 1);
    float b = 1.0f / (float)(blockIdx.x + 1);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int km_calib_copy(void *dst, const void *src, size_t bytes, void *stream) {
    if (!dst || !src || bytes % 16 != 0 || (uintptr_t)dst % 16 || (uintptr_t)src % 16) return -1;
    const int64_t n = (int64_t)(bytes / 16);
    if (n == 0) return 0;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 256 * 32) blocks = 256 * 32;
    copy_kernel<<<(unsigned)blocks, 256, 0, (hipStream_t)stream>>>((f32x4 *)dst, (const f32x4 *)src, n);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

int km_calib_read(const void *src, size_t bytes, float *out, int blocks, int nontemporal,
                  void *stream) {
    if (!src || !out || blocks < 1 || bytes % 16 != 0 || (uintptr_t)src % 16) return -1;
    if (nontemporal)
        read_kernel<true><<<(unsigned)blocks, 256, 0, (hipStream_t)stream>>>(
            (const f32x4 *)src, (int64_t)(bytes / 16), out);
    else
        read_kernel<false><<<(unsigned)blocks, 256, 0, (hipStream_t)stream>>>(
            (const f32x4 *)src, (int64_t)(bytes / 16), out);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

int km_calib_mfma_f32(float *out, int blocks, int iters, void *stream) {
    if (!out || blocks < 1 || iters < 1) return -1;
    mfma_f32_loop_kernel<<<(unsigned)blocks, 256, 0, (hipStream_t)stream>>>(out, iters, 1e-3f);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
