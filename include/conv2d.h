/*
 * conv2d.h -- C ABI of the 2-D convolution of the MI355X (gfx950) library.
 *
 * The convolution is the "Convolution" row of the tiled-kernel table in
 * "Tiling Strategies", section 5 ("Tiling Beyond GEMM"): input patches and
 * filter weights are the tiled operands, and every weight is reused at every
 * output position.  The pages give no formula; the usual deep-learning form is
 * computed (cross-correlation, zero padding, stride, dilation), channels
 * innermost:
 *
 *   x[((n*H + h)*W + w)*C + c]      input,   N x H x W x C (NHWC), contiguous
 *   wt[((k*R + r)*S + s)*C + c]     filters, K x R x S x C (KRSC), contiguous
 *   y[((n*P + p)*Q + q)*K + k]      output,  N x P x Q x K (NHWC), contiguous
 *
 *   P = (H + 2 pad_h - dil_h (R - 1) - 1) / stride_h + 1   (floor; 0 when negative)
 *   Q = (W + 2 pad_w - dil_w (S - 1) - 1) / stride_w + 1
 *   y[n][p][q][k] = sum_{r<R, s<S, c<C}
 *       x[n][p stride_h - pad_h + r dil_h][q stride_w - pad_w + s dil_w][c] * wt[k][r][s][c]
 *
 * with input positions outside the image reading as zero.  It runs as an
 * implicit matrix product on the same matrix-core kernel as sgemm: rows are
 * the N*P*Q output positions, columns the K output channels, the reduction
 * runs over R*S*C; the input is gathered straight into LDS tile by tile (no
 * im2col buffer), the filters are read as the N x K stored operand.  The
 * summation order is unspecified; results are FP32 (round to nearest even),
 * exact for integer-valued inputs whose partial sums stay below 2^24.  Fastest
 * when C is a multiple of 32 (each K slice then lies in one filter tap and is
 * copied straight into LDS); other C gather through registers.
 *
 * Memory and ownership: x, wt and y are device pointers owned by the caller;
 * y must not overlap x or wt (not checked).  The library allocates nothing and
 * keeps no mutable state.  Work is enqueued on `stream` and the call returns
 * without waiting.
 *
 * Status codes are those of sgemm.h.
 */
#ifndef TILED_FP32_CONV2D_H
#define TILED_FP32_CONV2D_H

#include <stdint.h>

#include "sgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * y = conv2d(x, wt) as above.
 * Returns SGEMM_STATUS_SUCCESS; SGEMM_STATUS_INVALID_SIZE for a negative size
 * or padding, or a stride or dilation below 1; SGEMM_STATUS_SIZE_OVERFLOW when
 * N*P*Q or R*S*C reaches 2^31, an element count overflows 64 bits, or
 * H + 2 pad_h, W + 2 pad_w or a dilated filter span reaches 2^29;
 * SGEMM_STATUS_NULL_POINTER for a NULL y with outputs to write, or a NULL x or
 * wt when R*S*C > 0; SGEMM_STATUS_LAUNCH_FAILED if HIP rejects the launch.
 * N*P*Q == 0 or K == 0 enqueues nothing; R*S*C == 0 sets y to +0.0.
 */
int conv2d_nhwc(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S,
                int64_t pad_h, int64_t pad_w, int64_t stride_h, int64_t stride_w, int64_t dil_h,
                int64_t dil_w, const float *x, const float *wt, float *y, hipStream_t stream);

/*
 * The same with an explicit tile configuration (an sgemm configuration index
 * for which conv2d_config_available returns 1; tests and tuning).
 * SGEMM_STATUS_INVALID_CONFIG for any other index.
 */
int conv2d_nhwc_with_config(int config, int64_t N, int64_t H, int64_t W, int64_t C, int64_t K,
                            int64_t R, int64_t S, int64_t pad_h, int64_t pad_w, int64_t stride_h,
                            int64_t stride_w, int64_t dil_h, int64_t dil_w, const float *x,
                            const float *wt, float *y, hipStream_t stream);

/*
 * Output extents P and Q (either pointer may be NULL).  Host only.
 * SGEMM_STATUS_INVALID_SIZE for negative sizes or padding, or a stride or
 * dilation below 1.
 */
int conv2d_nhwc_output_size(int64_t H, int64_t W, int64_t R, int64_t S, int64_t pad_h,
                            int64_t pad_w, int64_t stride_h, int64_t stride_w, int64_t dil_h,
                            int64_t dil_w, int64_t *P, int64_t *Q);

/* 1 if tile configuration `config` has a convolution kernel, 0 if not;
 * SGEMM_STATUS_INVALID_CONFIG for an unknown index.  Host only. */
int conv2d_config_available(int config);

/* The tile configuration conv2d_nhwc would use for this shape, or a negative
 * status for invalid arguments.  Host only. */
int conv2d_select_config(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R,
                         int64_t S, int64_t pad_h, int64_t pad_w, int64_t stride_h,
                         int64_t stride_w, int64_t dil_h, int64_t dil_w);

/*
 * y = conv2d(x, wt) as conv2d_nhwc, with the reduction over R*S*C split as in
 * sgemm_splitk: on the implicit GEMM's output tiles, each of `splits` chunks
 * of whole BK slices is reduced by its own workgroup, and the partial tiles
 * join inside the same launch in chunk order (bit-reproducible, independent
 * of timing; no workgroup waits for another).  With splits = 0 the time model
 * chooses, and may split only the tiles of the last partial layer of one tile
 * per CU, the others taking all of R*S*C ("Tiling Strategies" section 4 on
 * tail effects: a 3x3 layer of 64 x 14 x 14 outputs and 256 channels makes
 * 784 tiles of 64 x 64, three per CU and 16 more).  A chunk may start inside
 * a filter tap.
 *
 * config: a configuration with a convolution split-K kernel
 *   (conv2d_config_has_splitk), or -1 for the time model's choice (which may
 *   be the plain convolution kernel).
 * splits: 1 ... 64, or 0 for the time model's choice; the count used is at
 *   most ceil(R*S*C / BK) (conv2d_nhwc_splitk_plan reports it).
 * workspace, workspace_bytes: as for sgemm_splitk, with at least
 *   conv2d_nhwc_splitk_plan(...) bytes (NULL and 0 when the plan does not
 *   split).  The counter header must hold zeros before the first use; every
 *   completed call leaves it zero, so one workspace serves sgemm_splitk and
 *   conv2d_nhwc_splitk calls of any shape in turn.  Concurrent calls on one
 *   workspace race.
 * Errors as for conv2d_nhwc, plus SGEMM_STATUS_INVALID_CONFIG (no
 * convolution split-K kernel), SGEMM_STATUS_INVALID_SIZE (splits outside
 * 0 ... 64) and SGEMM_STATUS_INVALID_WORKSPACE; on an error nothing is
 * enqueued.
 */
int conv2d_nhwc_splitk(int config, int64_t N, int64_t H, int64_t W, int64_t C, int64_t K,
                       int64_t R, int64_t S, int64_t pad_h, int64_t pad_w, int64_t stride_h,
                       int64_t stride_w, int64_t dil_h, int64_t dil_w, const float *x,
                       const float *wt, float *y, int64_t splits, void *workspace,
                       int64_t workspace_bytes, hipStream_t stream);

/*
 * The plan conv2d_nhwc_splitk would run for these arguments: the tile
 * configuration, the chunk count and the number of output tiles that take all
 * of R*S*C without a join go to *plan_config, *plan_splits and
 * *plan_full_tiles (each may be NULL); returns the workspace bytes it needs
 * (0 when it does not split or there is nothing to compute), or a negative
 * status.  Host only.
 */
int64_t conv2d_nhwc_splitk_plan(int config, int64_t N, int64_t H, int64_t W, int64_t C,
                                int64_t K, int64_t R, int64_t S, int64_t pad_h, int64_t pad_w,
                                int64_t stride_h, int64_t stride_w, int64_t dil_h,
                                int64_t dil_w, int64_t splits, int *plan_config,
                                int64_t *plan_splits, int64_t *plan_full_tiles);

/* 1 if tile configuration `config` has a convolution split-K kernel, 0 if
 * not; SGEMM_STATUS_INVALID_CONFIG for an unknown index.  Host only. */
int conv2d_config_has_splitk(int config);

#ifdef __cplusplus
}
#endif

#endif /* TILED_FP32_CONV2D_H */
