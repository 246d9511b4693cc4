/*
 * km_calib.h - calibration kernels used by the measurements (libkm_calib.so).
 * Not part of the k-means computation.
 *
 * All pointers are device pointers owned by the caller; stream is a
 * hipStream_t (NULL = default stream). Calls only enqueue work.
 */
#ifndef KM_CALIB_H
#define KM_CALIB_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Copy `bytes` bytes from src to dst with 16-byte vector loads and stores
 * (a streaming kernel that reads and writes every byte exactly once). Used to
 * calibrate the HBM byte counters and to measure attainable copy bandwidth.
 * Requires bytes % 16 == 0 and 16-byte aligned, non-overlapping buffers.
 * Returns 0, -1 on invalid arguments, -6 if the launch is rejected.
 */
int km_calib_copy(void *dst, const void *src, size_t bytes, void *stream);

/*
 * Read `bytes` bytes of src once with 16-byte vector loads (blocks x 256
 * threads striding over the buffer, 8 loads in flight per thread; ordinary
 * or, with nontemporal != 0, non-temporal loads) and write one float per
 * thread to out (blocks * 256 floats): the attainable read bandwidth.
 * Requires bytes % 16 == 0, src 16-byte aligned, blocks >= 1.
 * Returns 0, -1 on invalid arguments, -6 if the launch is rejected.
 */
int km_calib_read(const void *src, size_t bytes, float *out, int blocks, int nontemporal,
                  void *stream);

/*
 * Run `blocks` blocks of 256 threads, each wave issuing iters x 4
 * v_mfma_f32_32x32x2_f32 (4096 flop each) on four independent accumulators,
 * with no memory traffic but one float per thread written to out
 * (blocks * 256 floats). Work = blocks * 4 * iters * 4 * 4096 flop.
 * Returns 0, -1 on invalid arguments, -6 if the launch is rejected.
 */
int km_calib_mfma_f32(float *out, int blocks, int iters, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KM_CALIB_H */
