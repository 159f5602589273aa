// Host side of attention_fwd (include/attention.h): argument checks and the
// launch of one workgroup per (head, block of queries), split over several
// launches when one dispatch cannot hold them all.
#include "attention.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "attention_kernel.hpp"

namespace {

using namespace sgemm_dev;

// O set to +0 (no keys: every output is the empty weighted sum).
__global__ void attention_zero_kernel(float* O, int64_t n) {
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x)
        O[e] = 0.0f;
}

template <class T>
int launch(int64_t BH, int64_t Sq, int64_t Skv, const float* Q, const float* K, const float* V,
           float* O, float scale, hipStream_t stream) {
    AttnArgs a;
    a.Sq = (int)Sq;
    a.Skv = (int)Skv;
    a.q_blocks = (int)((Sq + T::BQ - 1) / T::BQ);
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
    // A dispatch counts its work-items in 32 bits: the heads go over as many
    // launches as that needs (Sq < 2^31 - 512 keeps one head's query blocks
    // within one launch).
    const int64_t per_launch = (int64_t)UINT32_MAX / T::NT / a.q_blocks;
    for (int64_t h0 = 0; h0 < BH; h0 += per_launch) {
        const int64_t nh = BH - h0 < per_launch ? BH - h0 : per_launch;
        a.Q = Q + h0 * Sq * T::D;
        a.K = K + h0 * Skv * T::D;
        a.V = V + h0 * Skv * T::D;
        a.O = O + h0 * Sq * T::D;
        a.BH = nh;
        void* args[] = {&a};
        const hipError_t e =
            hipLaunchKernel((const void*)&attention_kernel<T>, dim3((unsigned)(a.q_blocks * nh)),
                            dim3(T::NT), args, 0, stream);
        if (e != hipSuccess) return SGEMM_STATUS_LAUNCH_FAILED;
    }
    return SGEMM_STATUS_SUCCESS;
}

}  // namespace

extern "C" int attention_fwd(int64_t BH, int64_t Sq, int64_t Skv, int64_t D, const float* Q,
                             const float* K, const float* V, float* O, float scale, int causal,
                             hipStream_t stream) {
    if (BH < 0 || Sq < 0 || Skv < 0 || (D != 64 && D != 128)) return SGEMM_STATUS_INVALID_SIZE;
    if (causal != 0 && causal != 1) return SGEMM_STATUS_INVALID_OP;
    // Query and key indices are 32-bit in the kernel, one block past the end
    // included.
    if (Sq > INT32_MAX - 512 || Skv > INT32_MAX - 512 || BH > INT32_MAX)
        return SGEMM_STATUS_SIZE_OVERFLOW;
    int64_t t, q_elems, kv_elems;
    if (__builtin_mul_overflow(BH, Sq, &t) || __builtin_mul_overflow(t, D, &q_elems) ||
        __builtin_mul_overflow(BH, Skv, &t) || __builtin_mul_overflow(t, D, &kv_elems))
        return SGEMM_STATUS_SIZE_OVERFLOW;
    if (BH == 0 || Sq == 0) return SGEMM_STATUS_SUCCESS;
    if (O == nullptr) return SGEMM_STATUS_NULL_POINTER;
    if (Skv == 0) {
        int64_t blocks = (q_elems + 255) / 256;
        if (blocks > 65536) blocks = 65536;
        void* args[] = {&O, &q_elems};
        const hipError_t e = hipLaunchKernel((const void*)&attention_zero_kernel,
                                             dim3((unsigned)blocks), dim3(256), args, 0, stream);
        return e == hipSuccess ? SGEMM_STATUS_SUCCESS : SGEMM_STATUS_LAUNCH_FAILED;
    }
    if (Q == nullptr || K == nullptr || V == nullptr) return SGEMM_STATUS_NULL_POINTER;
    if (!std::isfinite(scale)) return SGEMM_STATUS_INVALID_SIZE;
    if (D == 128)
        return causal ? launch<AttnTile<128, true>>(BH, Sq, Skv, Q, K, V, O, scale, stream)
                      : launch<AttnTile<128, false>>(BH, Sq, Skv, Q, K, V, O, scale, stream);
    return causal ? launch<AttnTile<64, true>>(BH, Sq, Skv, Q, K, V, O, scale, stream)
                  : launch<AttnTile<64, false>>(BH, Sq, Skv, Q, K, V, O, scale, stream);
}
