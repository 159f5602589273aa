// Host side of window_sum (include/window_sum.h): argument checks and the
// ceil(n / T)-block launch of "CMU DLSys Lecture 12: GPU Acceleration"
// sections 1 and 3 (T outputs per block, the last block guarded).
#include "window_sum.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "window_kernel.hpp"

extern "C" int window_sum(int64_t n, int64_t W, const float* x, float* y, hipStream_t stream) {
    using sgemm_dev::WindowTile;
    if (n < 0 || W < 1 || W > WindowTile::MAX_W) return SGEMM_STATUS_INVALID_SIZE;
    if (n == 0) return SGEMM_STATUS_SUCCESS;
    if (n > INT64_MAX - W) return SGEMM_STATUS_SIZE_OVERFLOW;
    const int64_t blocks = (n + WindowTile::T - 1) / WindowTile::T;
    // A dispatch counts its work-items in 32 bits.
    if (blocks > (int64_t)UINT32_MAX / WindowTile::NT) return SGEMM_STATUS_SIZE_OVERFLOW;
    if (x == nullptr || y == nullptr) return SGEMM_STATUS_NULL_POINTER;
    int w = (int)W;
    void* args[] = {&x, &y, &n, &w};
    const hipError_t e = hipLaunchKernel((const void*)&sgemm_dev::window_sum_kernel,
                                         dim3((unsigned)blocks), dim3(WindowTile::NT), args, 0,
                                         stream);
    return e == hipSuccess ? SGEMM_STATUS_SUCCESS : SGEMM_STATUS_LAUNCH_FAILED;
}
