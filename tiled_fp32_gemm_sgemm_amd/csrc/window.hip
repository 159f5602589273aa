// Host side of window_sum (include/window_sum.h): argument checks and the
// ceil(n / T)-block launch of "CMU DLSys Lecture 12: GPU Acceleration"
// sections 1 and 3 (T outputs per block, the last block guarded).
#include "window_sum.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "window_kernel.hpp"

template <int QUADS>
int launch_window(int64_t n, int W, const float* x, float* y, hipStream_t stream) {
    using WT = sgemm_dev::WindowTile<QUADS>;
    const int64_t blocks = (n + WT::T - 1) / WT::T;
    // A dispatch counts its work-items in 32 bits.
    if (blocks > (int64_t)UINT32_MAX / WT::NT) return SGEMM_STATUS_SIZE_OVERFLOW;
    void* args[] = {&x, &y, &n, &W};
    const hipError_t e = hipLaunchKernel((const void*)&sgemm_dev::window_sum_kernel<QUADS>,
                                         dim3((unsigned)blocks), dim3(WT::NT), args, 0, stream);
    return e == hipSuccess ? SGEMM_STATUS_SUCCESS : SGEMM_STATUS_LAUNCH_FAILED;
}

extern "C" int window_sum(int64_t n, int64_t W, const float* x, float* y, hipStream_t stream) {
    if (n < 0 || W < 1 || W > sgemm_dev::WindowTile<1>::MAX_W) return SGEMM_STATUS_INVALID_SIZE;
    if (n == 0) return SGEMM_STATUS_SUCCESS;
    if (n > INT64_MAX - W) return SGEMM_STATUS_SIZE_OVERFLOW;
    if (x == nullptr || y == nullptr) return SGEMM_STATUS_NULL_POINTER;
    // Outputs per workgroup by window width: more, smaller blocks for narrow
    // windows; larger ones where the halo is a bigger share of the inputs.
    if (W <= sgemm_dev::kWindowQuads1Max) return launch_window<1>(n, (int)W, x, y, stream);
    if (W <= sgemm_dev::kWindowQuads2Max) return launch_window<2>(n, (int)W, x, y, stream);
    return launch_window<4>(n, (int)W, x, y, stream);
}
