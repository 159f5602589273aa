/*
 * Sliding window sums on the GPU (gfx950): the cooperative-staging example of
 * "CMU DLSys Lecture 12: GPU Acceleration", section 3 ("A sliding window
 * reveals cooperative loading"), as a C ABI.  Status codes are those of
 * sgemm.h.
 */
#ifndef TILED_FP32_WINDOW_SUM_H
#define TILED_FP32_WINDOW_SUM_H

#include <stdint.h>

#include "sgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * y[i] = sum_{d=0}^{W-1} x[i+d] for 0 <= i < n.  n counts outputs; x must hold
 * n + W - 1 valid floats (the lecture's five-wide window is W = 5, a window of
 * radius R is W = 2R + 1).  Each output adds its terms in the order
 * d = 0, 1, ..., W-1 in FP32.  x and y are device pointers owned by the caller
 * and must not overlap; y[n..] is never written and x past n + W - 1 is never
 * read.  Enqueued on `stream`, asynchronous.
 * Returns 0; SGEMM_STATUS_INVALID_SIZE for n < 0, W < 1 or W > 1024;
 * SGEMM_STATUS_SIZE_OVERFLOW when n + W - 1 overflows or the launch would need
 * more than 2^32 - 1 work-items (blocks of 256 lanes hold 1024 outputs for
 * W <= 8, 2048 for W <= 24 and 4096 for wider windows: n above about 1.7e10,
 * 3.4e10 or 6.9e10);
 * SGEMM_STATUS_NULL_POINTER for a NULL x or y with n > 0;
 * SGEMM_STATUS_LAUNCH_FAILED if HIP rejects the launch.  n == 0 enqueues
 * nothing.
 */
int window_sum(int64_t n, int64_t W, const float *x, float *y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TILED_FP32_WINDOW_SUM_H */
