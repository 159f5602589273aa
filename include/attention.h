/*
 * attention.h -- C ABI of the blockwise attention of the MI355X (gfx950)
 * library.
 *
 * Scaled dot-product attention per head, the "FlashAttention" row of the
 * tiled-kernel table in "Tiling Strategies", section 5 ("Tiling Beyond
 * GEMM": Q, K and V are tiled along the sequence, and each K/V block is reused
 * by all the query rows of a tile).  For head h < BH, query i < Sq, d < D:
 *
 *   s_ij = scale * sum_d Q[(h*Sq + i)*D + d] * K[(h*Skv + j)*D + d]
 *          over the allowed keys j: j < Skv, and j <= i when causal = 1,
 *   O[(h*Sq + i)*D + d] = sum_j exp(s_ij - max_j s_ij) V[(h*Skv + j)*D + d]
 *                         / sum_j exp(s_ij - max_j s_ij).
 *
 * Q, O: BH x Sq x D; K, V: BH x Skv x D; all FP32, contiguous (D innermost).
 * Computed in FP32 in one pass over K and V with the online softmax (a running
 * maximum and sum per query, base-2 exponentials of scores scaled by
 * scale * log2(e)); the score matrix is never stored.  The order of the sums
 * is unspecified.
 *
 * Memory and ownership: device pointers owned by the caller; O must not
 * overlap Q, K or V (not checked).  Nothing is allocated.  Work is enqueued on
 * `stream` and the call returns without waiting.
 *
 * Returns SGEMM_STATUS_SUCCESS (sgemm.h); SGEMM_STATUS_INVALID_SIZE for a
 * negative size, a head dimension other than 64 or 128, or a scale that is not
 * finite; SGEMM_STATUS_INVALID_OP for causal other than 0 or 1;
 * SGEMM_STATUS_SIZE_OVERFLOW when BH reaches 2^31, Sq or Skv exceeds
 * 2^31 - 513 or an element count overflows 64 bits (heads that need more
 * workgroups than one launch holds go over several launches);
 * SGEMM_STATUS_NULL_POINTER for a NULL O with outputs to write or a NULL Q, K
 * or V when Skv > 0; SGEMM_STATUS_LAUNCH_FAILED if HIP rejects the launch.
 * BH == 0 or Sq == 0 enqueues nothing; Skv == 0 sets O to +0.0.
 */
#ifndef TILED_FP32_ATTENTION_H
#define TILED_FP32_ATTENTION_H

#include <stdint.h>

#include "sgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

int attention_fwd(int64_t BH, int64_t Sq, int64_t Skv, int64_t D, const float *Q, const float *K,
                  const float *V, float *O, float scale, int causal, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TILED_FP32_ATTENTION_H */
