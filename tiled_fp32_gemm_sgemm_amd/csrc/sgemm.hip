// Host side of the C ABI declared in include/sgemm.h: argument validation,
// tile-configuration choice, grid arithmetic and the launch on the caller's
// stream.  Arguments are checked before anything is enqueued, and the launch
// status from HIP is returned ("CMU DLSys Lecture 12: GPU Acceleration"
// section 2: launches are asynchronous, and API and launch errors are checked).
#include "sgemm.h"
#include "conv2d.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <mutex>

#include "mfma_dl_kernel.hpp"
#include "mfma_kernel.hpp"
#include "tile_common.hpp"
#include "valu_kernel.hpp"

namespace sgemm_dev {

// C's window set to +0 (K == 0: every output is the empty sum).
__global__ void zero_fill_kernel(float* C, int64_t ldc, int64_t strideC, int M, int N,
                                 int batch) {
    const int64_t total = (int64_t)M * N * batch;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = e / ((int64_t)M * N);
        const int64_t rem = e - b * (int64_t)M * N;
        const int64_t i = rem / N;
        const int64_t j = rem - i * N;
        C[b * strideC + i * ldc + j] = 0.0f;
    }
}

// C's window scaled by beta (the general form with K == 0 or alpha == 0:
// the product term is zero).  beta == 0 writes +0 without reading C.
__global__ void scale_kernel(float* C, int64_t ldc, int64_t strideC, int M, int N, int batch,
                             float beta) {
    const int64_t total = (int64_t)M * N * batch;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = e / ((int64_t)M * N);
        const int64_t rem = e - b * (int64_t)M * N;
        const int64_t i = rem / N;
        const int64_t j = rem - i * N;
        float* const c = C + b * strideC + i * ldc + j;
        *c = beta == 0.0f ? 0.0f : beta * *c;
    }
}

// n words set to zero (n a multiple of the block size).
__global__ void clear_words_kernel(uint32_t* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

}  // namespace sgemm_dev

// The split-K workspace kept by the library for callers that cannot
// allocate device memory (sgemm_splitk_noalloc): the same layout as a
// caller's workspace (counter header, then partial tiles),
// SGEMM_SPLITK_SCRATCH_BYTES long.  Every device that loads this code object
// holds its own copy until the process ends.  In host code the name stands
// for a host-side shadow, not a device address, so it is never passed to a
// kernel or a copy: the address of each device's copy comes from
// hipGetSymbolAddress (scratch_for_stream).
static __device__ __align__(256) unsigned char scratch[SGEMM_SPLITK_SCRATCH_BYTES];

namespace {

using namespace sgemm_dev;

// Matrix-core tile configurations.  Index = config id in the ABI.
// MfmaTile<BM, BN, BK, waves along M, waves along N, MFMA edge, waves per SIMD,
//          tile-row group>
using Cfg256x128 = MfmaTile<256, 128, 16, 2, 2, 32, 2, 8>;       // 4 waves of 128x64
using Cfg128x128 = MfmaTile<128, 128, 16, 2, 2, 32, 3, 8>;       // 4 waves of 64x64
using Cfg64x64 = MfmaTile<64, 64, 16, 2, 2, 32, 4, 8>;           // 4 waves of 32x32
using Cfg256x256 = MfmaTile<256, 256, 16, 2, 4, 32, 2, 8>;       // 8 waves of 128x64
using Cfg256x256k32 = MfmaTile<256, 256, 32, 2, 4, 32, 2, 8>;    // 8 waves of 128x64
using Cfg128x128k32 = MfmaTile<128, 128, 32, 2, 2, 32, 2, 8>;    // 4 waves of 64x64
using Cfg128x128k32m16 = MfmaTile<128, 128, 32, 2, 2, 16, 2, 8>; // 4 waves of 64x64
using Cfg64x64k32m16 = MfmaTile<64, 64, 32, 2, 2, 16, 4, 8>;     // 4 waves of 32x32
// One wave per SIMD, 128x128 wave tiles, accumulators in the AGPR file.
using Cfg256x256m32w1 = MfmaTile<256, 256, 16, 2, 2, 32, 1, 8>;
using Cfg256x256k32m32w1 = MfmaTile<256, 256, 32, 2, 2, 32, 1, 8>;
// Direct global->LDS staging.
using Dl256x256k32m32 = DlTile<256, 256, 32, 2, 4, 32, 2, 8>;      // 8 waves of 128x64
using Dl256x256k16m32 = DlTile<256, 256, 16, 2, 4, 32, 2, 8>;      // 8 waves of 128x64
using Dl256x128k32m32 = DlTile<256, 128, 32, 2, 2, 32, 1, 8>;      // 4 waves of 128x64
using Dl128x128k32m32 = DlTile<128, 128, 32, 2, 2, 32, 2, 8>;      // 4 waves of 64x64
// Deeper pipelines and widths that divide ragged shapes into whole CU rounds.
using Dl128x128k32m32s4 = DlTile<128, 128, 32, 2, 2, 32, 1, 8, 4>;  // 4 waves of 64x64
using Dl64x64k32m32s4 = DlTile<64, 64, 32, 2, 2, 32, 2, 8, 4>;      // 4 waves of 32x32
using Dl256x192k32m32 = DlTile<256, 192, 32, 4, 2, 32, 2, 8>;      // 8 waves of 64x96
using Dl192x256k32m32 = DlTile<192, 256, 32, 2, 4, 32, 2, 8>;      // 8 waves of 96x64
using Dl64x64k64m32s4 = DlTile<64, 64, 64, 2, 2, 32, 1, 8, 4>;      // 4 waves of 32x32
using Dl64x64k32m32s8 = DlTile<64, 64, 32, 2, 2, 32, 1, 8, 8>;      // 4 waves of 32x32
using Dl128x64k32m32s4 = DlTile<128, 64, 32, 2, 2, 32, 1, 8, 4>;    // 4 waves of 64x32
using Dl128x128k64m32s2 = DlTile<128, 128, 64, 2, 2, 32, 1, 8, 2>;  // 4 waves of 64x64
// Two wave groups split every slice's k range (8 waves of 32x32, 2 per SIMD).
using Dl64x64k64m32s4x2 = DlTile<64, 64, 64, 2, 2, 32, 2, 8, 4, 2>;
using Dl64x64k32m32s4x2 = DlTile<64, 64, 32, 2, 2, 32, 2, 8, 4, 2>;
// Copies spread over the k steps (schedule 2): +6 % at 512 x 4096 x 4096.
using Dl128x64k64m32s2x2 =
    DlTile<128, 64, 64, 2, 2, 32, 2, 8, 2, 2, true, false, false, false, true, false, 2>;  // 8 waves of 64x32
using Dl64x128k64m32s2x2 =
    DlTile<64, 128, 64, 2, 2, 32, 2, 8, 2, 2, true, false, false, false, true, false, 2>;  // 8 waves of 32x64
// 96 x 96: one tile per CU at 1536^2 (16 x 16 tiles), 4 waves of 48 x 48 on
// 16x16x4 MFMAs (3 x 3 accumulator tiles each).
using Dl96x96k32m16 = DlTile<96, 96, 32, 2, 2, 16, 2, 8>;
// 128 x 128 with two k groups (8 waves of 64 x 64, two per SIMD) and copies
// spread over the k steps: one tile per CU at 2048^2 without dropping to one
// wave per SIMD (2048^3: 135.9 -> 138.0 TFLOP/s; 1024 x 4096 x 4096: 138.5 ->
// 142.3).  No convolution variant: with the convolution's burst copies it ran
// the 3x3 layers 1.5-2 % slower than the tile they use.
using Dl128x128k64m32s2x2 =
    DlTile<128, 128, 64, 2, 2, 32, 2, 8, 2, 2, true, false, false, false, true, false, 2>;
// 64 x 64 with BK = 128, four k groups (8 waves of 32 x 64, two per SIMD)
// and copies spread over the k steps: for one tile per CU (1024^3, the
// split-K chunks of thin products) the long slices halve the barriers per
// k: 1024^3 20.7 -> 19.9 us, 1024 x 1024 x 4096 71.3 -> 65.7 us against the
// 64 x 64 x 64 tile with two k groups.
using Dl64x64k128m32s2x4 =
    DlTile<64, 64, 128, 2, 1, 32, 2, 8, 2, 4, true, false, false, false, true, false, 2>;
// 128 x 128 x 64 with eight waves of 32 x 64 (two per SIMD) and no k
// groups, copies spread over the k steps: for one 128 x 128 tile per CU it
// avoids the k-group exchange (2048^3: 124.2 -> 121.3 us against the k-group
// tile; 2048 x 2048 x 1024: 65.5 -> 63.7).
using Dl128x128k64m32w4x2 =
    DlTile<128, 128, 64, 4, 2, 32, 2, 8, 2, 1, true, false, false, false, true, false, 2>;
// Small LDS footprints, so that three or four workgroups share a CU and
// their barriers fall at different times (4 waves of 64x64 or 32x32 each).
// The 128 x 128 x 16 tiles spread their copies over the k steps (schedule
// 2): batched 1024 x 128^3 41.9 -> 40.6 us, 8192^2 x 128 152.2 -> 145.7 us,
// 16 x 3000 x 512 x 128 on the three-stage tile 63.1 -> 55.9 us, and level to
// 1 % slower on the rest of the shapes that choose them.  The 64 x 64 x 32
// tile keeps the burst: spread, it ran 1.4-3.4 % slower (its split-K variant
// and hybrid plans included).
using Dl128x128k16o4 =  // 32 KB LDS, 4 per CU
    DlTile<128, 128, 16, 2, 2, 32, 4, 8, 2, 1, true, false, false, false, true, false, 2>;
using Dl128x128k16o3s3 =  // 48 KB LDS, 3 per CU
    DlTile<128, 128, 16, 2, 2, 32, 3, 8, 3, 1, true, false, false, false, true, false, 2>;
using Dl64x64k32o4 = DlTile<64, 64, 32, 2, 2, 32, 4, 8, 2>;         // 32 KB LDS, 4 per CU
// Control build: A stored unswizzled (bank conflicts on purpose); never chosen.
using Dl256x256k32m32Plain = DlTile<256, 256, 32, 2, 4, 32, 2, 8, 2, 1, false>;

struct ConfigEntry {
    const char* name;
    int bm, bn, bk, threads;
    int wg_per_cu;  // workgroups a CU can hold (waves and LDS)
    const void* kernel;
    // Time model for the choice of a configuration, fitted to measurements on
    // MI355X (python -m tiled_fp32_gemm_sgemm_amd.calibrate), per unit of tile
    // area in microseconds: a round of 256 tiles (one workgroup per CU) takes
    // BM*BN*(one_a + one_b*K); when w = per_cu > 1 workgroups overlap on a CU,
    // a full round of 256*w tiles takes BM*BN*(two_a + two_b*K).  per_cu = 0
    // marks a control or experimental build that is never chosen.
    int per_cu;
    double one_a, one_b, two_a, two_b;
    // General form C = alpha op(A) op(B) + beta C, by operand layout
    // (transA + 2 * transB); NULL where this tile is not built for it.
    const void* general[4];
    // Implicit-GEMM 2-D convolution; NULL where not built.
    const void* conv;
    // Split-K variant of the plain product; NULL where not built.
    const void* splitk;
    // Split-K variant of the convolution; NULL where not built.
    const void* conv_splitk;
    // Split-K variants of the general form, by operand layout; NULL where
    // not built.
    const void* general_splitk[4];
};

// The same tile with stored-operand layouts and the alpha/beta epilogue.
template <class T, bool TA, bool TB>
using DlGeneral = DlTile<T::BM, T::BN, T::BK, T::WAVES_M, T::WAVES_N, T::MI, T::OCC, T::GROUP_M,
                         T::STAGES, T::KSPLIT, T::SWIZZLE, TA, TB, true, T::BIL, false, T::SCHED>;

// The same tile as an implicit-GEMM convolution (A gathered from an NHWC
// image, B = KRSC filters stored N x K).
template <class T>
using DlConv = DlTile<T::BM, T::BN, T::BK, T::WAVES_M, T::WAVES_N, T::MI, T::OCC, T::GROUP_M,
                      T::STAGES, T::KSPLIT, T::SWIZZLE, false, true, false, T::BIL, true, T::SCHED>;

// The same tile as split-K workgroups that join through a workspace, built
// for wave tiles up to 64 x 64 (one wave tile of sums in the join) and BK of
// 32 or more: the 128 x 128 x 16 tile ran 2-4 times slower than the others
// as split-K at every shape and chunk count measured, which the time model
// does not see, so it is not offered.
template <class T>
using DlSplitK = DlTile<T::BM, T::BN, T::BK, T::WAVES_M, T::WAVES_N, T::MI, T::OCC, T::GROUP_M,
                        T::STAGES, T::KSPLIT, T::SWIZZLE, false, false, false, T::BIL, false,
                        T::SCHED, true>;

template <class T>
const void* splitk_kernel() {
    if constexpr (T::WTM * T::WTN <= 64 * 64 && T::BK >= 32)
        return (const void*)&sgemm_mfma_dl_kernel<DlSplitK<T>>;
    else
        return nullptr;
}

// The convolution's split-K variant, for the same tiles.
template <class T>
using DlConvSplitK = DlTile<T::BM, T::BN, T::BK, T::WAVES_M, T::WAVES_N, T::MI, T::OCC,
                            T::GROUP_M, T::STAGES, T::KSPLIT, T::SWIZZLE, false, true, false,
                            T::BIL, true, T::SCHED, true>;

template <class T>
const void* conv_splitk_kernel() {
    if constexpr (T::WTM * T::WTN <= 64 * 64 && T::BK >= 32)
        return (const void*)&sgemm_mfma_dl_kernel<DlConvSplitK<T>>;
    else
        return nullptr;
}

// The general form's split-K variants, for the tiles that have a plain one.
template <class T, bool TA, bool TB>
using DlGeneralSplitK = DlTile<T::BM, T::BN, T::BK, T::WAVES_M, T::WAVES_N, T::MI, T::OCC,
                               T::GROUP_M, T::STAGES, T::KSPLIT, T::SWIZZLE, TA, TB, true,
                               T::BIL, false, T::SCHED, true>;

template <class T, bool TA, bool TB>
const void* general_splitk_kernel() {
    if constexpr (T::WTM * T::WTN <= 64 * 64 && T::BK >= 32)
        return (const void*)&sgemm_mfma_dl_kernel<DlGeneralSplitK<T, TA, TB>>;
    else
        return nullptr;
}

#define SGEMM_GENERAL_SPLITK(T)                                                         \
    { general_splitk_kernel<T, false, false>(), general_splitk_kernel<T, true, false>(), \
      general_splitk_kernel<T, false, true>(), general_splitk_kernel<T, true, true>() }

#define SGEMM_CFG(T, name, per_cu, a1, b1, a2, b2) \
    { name, T::BM, T::BN, T::BK, T::NT, T::WG_PER_CU, (const void*)&sgemm_mfma_kernel<T>, per_cu, \
      a1, b1, a2, b2 }
#define SGEMM_DL_CFG(T, name, per_cu, a1, b1, a2, b2)                                        \
    { name, T::BM, T::BN, T::BK, T::NT, T::WG_PER_CU, (const void*)&sgemm_mfma_dl_kernel<T>, \
      per_cu, a1, b1, a2, b2 }
#define SGEMM_DLX_CFG(T, name, per_cu, a1, b1, a2, b2)                                       \
    { name, T::BM, T::BN, T::BK, T::NT, T::WG_PER_CU, (const void*)&sgemm_mfma_dl_kernel<T>, \
      per_cu, a1, b1, a2, b2,                                                                 \
      { (const void*)&sgemm_mfma_dl_kernel<DlGeneral<T, false, false>>,                       \
        (const void*)&sgemm_mfma_dl_kernel<DlGeneral<T, true, false>>,                        \
        (const void*)&sgemm_mfma_dl_kernel<DlGeneral<T, false, true>>,                        \
        (const void*)&sgemm_mfma_dl_kernel<DlGeneral<T, true, true>> },                        \
      (const void*)&sgemm_mfma_dl_kernel<DlConv<T>>, splitk_kernel<T>(),                     \
      conv_splitk_kernel<T>(), SGEMM_GENERAL_SPLITK(T) }
// General form, no convolution variant.
#define SGEMM_DLG_CFG(T, name, per_cu, a1, b1, a2, b2)                                       \
    { name, T::BM, T::BN, T::BK, T::NT, T::WG_PER_CU, (const void*)&sgemm_mfma_dl_kernel<T>, \
      per_cu, a1, b1, a2, b2,                                                                 \
      { (const void*)&sgemm_mfma_dl_kernel<DlGeneral<T, false, false>>,                       \
        (const void*)&sgemm_mfma_dl_kernel<DlGeneral<T, true, false>>,                        \
        (const void*)&sgemm_mfma_dl_kernel<DlGeneral<T, false, true>>,                        \
        (const void*)&sgemm_mfma_dl_kernel<DlGeneral<T, true, true>> },                        \
      nullptr, splitk_kernel<T>(), nullptr, SGEMM_GENERAL_SPLITK(T) }

const ConfigEntry kConfigs[] = {
    SGEMM_CFG(Cfg256x128, "mfma32_256x128x16_w2x2", 1, 3.6505e-04, 4.2029e-06, 4.1134e-04, 8.0806e-06),
    SGEMM_CFG(Cfg128x128, "mfma32_128x128x16_w2x2", 3, 4.3004e-04, 4.5225e-06, 6.6566e-04, 1.2010e-05),
    SGEMM_CFG(Cfg64x64, "mfma32_64x64x16_w2x2", 4, 0.0000e+00, 8.9392e-06, 1.5698e-03, 1.7660e-05),
    SGEMM_CFG(Cfg256x256, "mfma32_256x256x16_w2x4", 1, 1.9697e-04, 3.7832e-06, 3.4747e-04, 7.5724e-06),
    SGEMM_CFG(Cfg256x256k32, "mfma32_256x256x32_w2x4", 1, 2.0272e-04, 3.7449e-06, 3.6204e-04, 7.4854e-06),
    SGEMM_CFG(Cfg128x128k32, "mfma32_128x128x32_w2x2", 2, 4.0454e-04, 4.5185e-06, 5.8699e-04, 7.7883e-06),
    SGEMM_CFG(Cfg128x128k32m16, "mfma16_128x128x32_w2x2", 2, 3.8094e-04, 4.7398e-06, 5.6840e-04, 8.1136e-06),
    SGEMM_CFG(Cfg64x64k32m16, "mfma16_64x64x32_w2x2", 4, 6.8628e-04, 6.4584e-06, 1.5598e-03, 1.8572e-05),
    SGEMM_CFG(Cfg256x256m32w1, "mfma32_256x256x16_w2x2", 1, 2.1097e-04, 3.9263e-06, 3.9320e-04, 7.8470e-06),
    SGEMM_CFG(Cfg256x256k32m32w1, "mfma32_256x256x32_w2x2", 1, 2.2194e-04, 3.8922e-06, 4.1654e-04, 7.7681e-06),
    SGEMM_DLX_CFG(Dl256x256k32m32, "dl32_256x256x32_w2x4", 1, 2.7056e-04, 3.3635e-06, 3.9211e-04, 6.7493e-06),
    SGEMM_DL_CFG(Dl256x256k16m32, "dl32_256x256x16_w2x4", 1, 2.2059e-04, 3.3829e-06, 3.7041e-04, 6.7868e-06),
    SGEMM_DL_CFG(Dl256x128k32m32, "dl32_256x128x32_w2x2", 1, 3.2052e-04, 3.7135e-06, 4.3937e-04, 7.4384e-06),
    SGEMM_DLX_CFG(Dl128x128k32m32, "dl32_128x128x32_w2x2", 2, 3.9893e-04, 3.8925e-06, 5.5372e-04, 6.8583e-06),
    SGEMM_DL_CFG(Dl256x256k32m32Plain, "dl32_256x256x32_w2x4_unswizzled", 0, 0, 0, 0, 0),
    SGEMM_DL_CFG(Dl128x128k32m32s4, "dl32_128x128x32_w2x2_s4", 1, 4.1409e-04, 4.0347e-06, 5.8961e-04, 8.0769e-06),
    SGEMM_DLX_CFG(Dl64x64k32m32s4, "dl32_64x64x32_w2x2_s4", 2, 7.5517e-04, 4.8253e-06, 1.0738e-03, 7.8416e-06),
    SGEMM_DLX_CFG(Dl256x192k32m32, "dl32_256x192x32_w4x2", 1, 2.1273e-04, 3.4836e-06, 3.5937e-04, 6.9587e-06),
    SGEMM_DLX_CFG(Dl192x256k32m32, "dl32_192x256x32_w2x4", 1, 2.1856e-04, 3.4304e-06, 3.6343e-04, 6.8644e-06),
    SGEMM_DL_CFG(Dl64x64k64m32s4, "dl32_64x64x64_w2x2_s4", 1, 7.7140e-04, 4.8489e-06, 1.2493e-03, 9.6503e-06),
    SGEMM_DL_CFG(Dl64x64k32m32s8, "dl32_64x64x32_w2x2_s8", 1, 8.4332e-04, 4.8843e-06, 1.3606e-03, 9.7563e-06),
    SGEMM_DL_CFG(Dl128x64k32m32s4, "dl32_128x64x32_w2x2_s4", 1, 4.9721e-04, 4.5194e-06, 8.1195e-04, 9.0356e-06),
    SGEMM_DL_CFG(Dl128x128k64m32s2, "dl32_128x128x64_w2x2", 1, 4.4267e-04, 3.9188e-06, 6.5237e-04, 7.8463e-06),
    SGEMM_DLX_CFG(Dl64x64k64m32s4x2, "dl32_64x64x64_w2x2_s4_k2", 1, 8.9272e-04, 4.1196e-06, 1.5031e-03, 8.1286e-06),
    SGEMM_DL_CFG(Dl64x64k32m32s4x2, "dl32_64x64x32_w2x2_s4_k2", 2, 8.4842e-04, 4.9353e-06, 1.1928e-03, 8.4095e-06),
    SGEMM_DLX_CFG(Dl128x64k64m32s2x2, "dl32_128x64x64_w2x2_s2_k2", 1, 5.7303e-04, 3.7133e-06, 1.0005e-03, 7.3913e-06),
    SGEMM_DLX_CFG(Dl128x128k16o4, "dl32_128x128x16_w2x2_o4", 4, 3.7798e-04, 3.8163e-06, 7.8534e-04, 1.3933e-05),
    SGEMM_DL_CFG(Dl128x128k16o3s3, "dl32_128x128x16_w2x2_s3_o3", 3, 3.7375e-04, 4.0480e-06, 5.7368e-04, 1.0599e-05),
    SGEMM_DLX_CFG(Dl64x64k32o4, "dl32_64x64x32_w2x2_o4", 4, 7.5602e-04, 4.4574e-06, 1.4899e-03, 1.4845e-05),
    SGEMM_DLX_CFG(Dl64x128k64m32s2x2, "dl32_64x128x64_w2x2_s2_k2", 1, 5.6513e-04, 3.6309e-06, 9.9029e-04, 7.2336e-06),
    SGEMM_DL_CFG(Dl96x96k32m16, "dl16_96x96x32_w2x2", 3, 5.7956e-04, 4.1848e-06, 8.6320e-04, 1.0753e-05),
    SGEMM_DLG_CFG(Dl128x128k64m32s2x2, "dl32_128x128x64_w2x2_s2_k2", 1, 5.9521e-04, 3.4661e-06, 7.0309e-04, 6.9811e-06),
    SGEMM_DLG_CFG(Dl64x64k128m32s2x4, "dl32_64x64x128_w2x1_s2_k4", 1, 1.1211e-03, 3.6461e-06, 1.8864e-03, 7.2474e-06),
    SGEMM_DLG_CFG(Dl128x128k64m32w4x2, "dl32_128x128x64_w4x2_s2", 1, 3.3451e-04, 3.4895e-06, 6.3514e-04, 6.9657e-06),
};
#undef SGEMM_CFG
#undef SGEMM_DL_CFG
#undef SGEMM_DLX_CFG
#undef SGEMM_DLG_CFG
#undef SGEMM_GENERAL_SPLITK
constexpr int kNumConfigs = (int)(sizeof(kConfigs) / sizeof(kConfigs[0]));
constexpr int kNumCu = 256;  // MI355X compute units

constexpr int64_t kMaxDim = INT32_MAX;
// A dispatch counts its work-items in 32 bits: one launch holds at most
// UINT32_MAX / threads workgroups.
constexpr int64_t kMaxWorkItems = UINT32_MAX;

bool mul_add_overflows(int64_t a, int64_t b, int64_t c, int64_t* out) {
    int64_t t;
    if (__builtin_mul_overflow(a, b, &t)) return true;
    return __builtin_add_overflow(t, c, out);
}

// Highest element index touched in a rows x cols matrix with leading dim ld,
// plus (batch-1)*stride; -1 means the call overflows int64.
int64_t span_end(int64_t rows, int64_t cols, int64_t ld, int64_t stride, int64_t batch) {
    if (rows == 0 || cols == 0) return 0;
    int64_t last;
    if (mul_add_overflows(rows - 1, ld, cols, &last)) return -1;
    int64_t boff;
    if (mul_add_overflows(batch - 1, stride, last, &boff)) return -1;
    return boff;
}

// Argument checks for C = alpha op(A) op(B) + beta C; the plain product is
// transA = transB = 0 with alpha = 1 (A and B needed whenever K > 0).  A is
// stored M x K (lda >= K) or, transposed, K x M (lda >= M); B is stored K x N
// (ldb >= N) or N x K (ldb >= K).
int validate_general(int transA, int transB, int64_t M, int64_t N, int64_t K, float alpha,
                     const float* A, int64_t lda, int64_t strideA, const float* B, int64_t ldb,
                     int64_t strideB, const float* C, int64_t ldc, int64_t strideC,
                     int64_t batch) {
    if ((transA != 0 && transA != 1) || (transB != 0 && transB != 1))
        return SGEMM_STATUS_INVALID_OP;
    if (M < 0 || N < 0 || K < 0 || batch < 0) return SGEMM_STATUS_INVALID_SIZE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim || batch > kMaxDim)
        return SGEMM_STATUS_SIZE_OVERFLOW;
    const int64_t a_rows = transA ? K : M, a_cols = transA ? M : K;
    const int64_t b_rows = transB ? N : K, b_cols = transB ? K : N;
    if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1) ||
        ldc < (N > 1 ? N : 1))
        return SGEMM_STATUS_INVALID_LD;
    if (strideA < 0 || strideB < 0 || strideC < 0) return SGEMM_STATUS_INVALID_STRIDE;
    if (M == 0 || N == 0 || batch == 0) return SGEMM_STATUS_SUCCESS;
    if (batch > 1) {
        const int64_t one_c = span_end(M, N, ldc, 0, 1);
        if (one_c < 0) return SGEMM_STATUS_SIZE_OVERFLOW;
        if (strideC < one_c) return SGEMM_STATUS_INVALID_STRIDE;
    }
    if (C == nullptr) return SGEMM_STATUS_NULL_POINTER;
    const bool reads_ab = K > 0 && alpha != 0.0f;
    if (reads_ab && (A == nullptr || B == nullptr)) return SGEMM_STATUS_NULL_POINTER;
    if (span_end(a_rows, a_cols, lda, strideA, batch) < 0 ||
        span_end(b_rows, b_cols, ldb, strideB, batch) < 0 ||
        span_end(M, N, ldc, strideC, batch) < 0)
        return SGEMM_STATUS_SIZE_OVERFLOW;
    return SGEMM_STATUS_SUCCESS;
}

int validate(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, int64_t strideA,
             const float* B, int64_t ldb, int64_t strideB, const float* C, int64_t ldc,
             int64_t strideC, int64_t batch) {
    return validate_general(0, 0, M, N, K, 1.0f, A, lda, strideA, B, ldb, strideB, C, ldc,
                            strideC, batch);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Predicted time of one launch: whole rounds of 256 * per_cu tiles at the
// fitted full-round time; a last, partial round that puts j of the w
// workgroups on the busiest CU takes the one-per-CU time plus (j - 1) / (w - 1)
// of the difference to a full round.
double predict_us(const ConfigEntry& c, int64_t M, int64_t N, int64_t K, int64_t batch) {
    const double tiles = (double)(ceil_div(M, c.bm) * ceil_div(N, c.bn)) * (double)batch;
    const double area = (double)c.bm * c.bn;
    const double one = area * (c.one_a + c.one_b * (double)K);
    const double full_t = area * (c.two_a + c.two_b * (double)K);
    const int w = c.per_cu;
    if (w < 2) return std::ceil(tiles / kNumCu) * one;
    const double full = std::floor(tiles / ((double)w * kNumCu));
    const double rest = tiles - full * (double)w * kNumCu;
    double last = 0.0;
    if (rest > 0.0) {
        const double j = std::ceil(rest / kNumCu);
        last = one + (full_t - one) * (j - 1.0) / (double)(w - 1);
    }
    return full * full_t + last;
}

// Shape -> configuration: the smallest predicted time; control builds are
// never chosen.  `general` restricts the choice to tiles built for the
// general form (every layout is built for the same tiles).
int choose_config(int64_t M, int64_t N, int64_t K, int64_t batch, bool general = false) {
    int best = -1;
    double best_us = 0.0;
    for (int idx = 0; idx < kNumConfigs; ++idx) {
        const ConfigEntry& c = kConfigs[idx];
        if (c.per_cu == 0 || (general && c.general[0] == nullptr)) continue;
        const double t = predict_us(c, M, N, K, batch);
        if (best < 0 || t < best_us * (1.0 - 1e-9)) {
            best_us = t;
            best = idx;
        }
    }
    return best;
}

// Convolution tiles: the smallest predicted time for the implicit GEMM
// (M = N*P*Q, N = output channels, K = R*S*C); a tile whose BK does not divide
// C gathers through registers and is counted four times slower.
int choose_conv_config(int64_t M, int64_t N, int64_t K, int64_t C) {
    int best = -1;
    double best_us = 0.0;
    for (int idx = 0; idx < kNumConfigs; ++idx) {
        const ConfigEntry& c = kConfigs[idx];
        if (c.per_cu == 0 || c.conv == nullptr) continue;
        const double t = predict_us(c, M, N, K, 1) * (C % c.bk == 0 ? 1.0 : 4.0);
        if (best < 0 || t < best_us * (1.0 - 1e-9)) {
            best_us = t;
            best = idx;
        }
    }
    return best;
}

int launch_gemm(const void* kernel, int bm, int bn, int threads, int64_t M, int64_t N, int64_t K,
                const float* A, int64_t lda, int64_t strideA, const float* B, int64_t ldb,
                int64_t strideB, float* C, int64_t ldc, int64_t strideC, int64_t batch,
                hipStream_t stream, float alpha = 1.0f, float beta = 0.0f,
                const ConvGeom* conv = nullptr) {
    if (K == 0) {
        const int64_t total = M * N * batch;
        int64_t blocks = ceil_div(total, 256);
        if (blocks > 65536) blocks = 65536;
        void* args[] = {&C, &ldc, &strideC, nullptr, nullptr, nullptr};
        int Mi = (int)M, Ni = (int)N, bi = (int)batch;
        // batch may exceed int range only with M*N tiny; the fill loops in int64
        // over M*N*batch, and batch < 2^31 is validated.
        args[3] = &Mi;
        args[4] = &Ni;
        args[5] = &bi;
        hipError_t e = hipLaunchKernel((const void*)&zero_fill_kernel, dim3((unsigned)blocks),
                                       dim3(256), args, 0, stream);
        return e == hipSuccess ? SGEMM_STATUS_SUCCESS : SGEMM_STATUS_LAUNCH_FAILED;
    }
    const int64_t tiles_m = ceil_div(M, bm);
    const int64_t tiles_n = ceil_div(N, bn);
    const int64_t per_matrix = tiles_m * tiles_n;
    const int64_t max_blocks = kMaxWorkItems / threads;
    if (per_matrix > max_blocks) return SGEMM_STATUS_SIZE_OVERFLOW;
    const int64_t per_launch = max_blocks / per_matrix;  // batch members per launch
    for (int64_t b0 = 0; b0 < batch; b0 += per_launch) {
        const int64_t nb = (batch - b0) < per_launch ? (batch - b0) : per_launch;
        GemmArgs p = {};
        if (conv != nullptr) p.conv = *conv;
        p.A = A;
        p.B = B;
        p.C = C;
        p.lda = lda;
        p.ldb = ldb;
        p.ldc = ldc;
        p.strideA = strideA;
        p.strideB = strideB;
        p.strideC = strideC;
        p.M = (int)M;
        p.N = (int)N;
        p.K = (int)K;
        p.tiles_m = (int)tiles_m;
        p.tiles_n = (int)tiles_n;
        p.batch_base = (int)b0;
        p.batch_count = (int)nb;
        p.alpha = alpha;
        p.beta = beta;
        void* args[] = {&p};
        hipError_t e = hipLaunchKernel(kernel, dim3((unsigned)(per_matrix * nb)), dim3(threads),
                                       args, 0, stream);
        if (e != hipSuccess) return SGEMM_STATUS_LAUNCH_FAILED;
    }
    return SGEMM_STATUS_SUCCESS;
}

int run_mfma(int config, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
             int64_t strideA, const float* B, int64_t ldb, int64_t strideB, float* C, int64_t ldc,
             int64_t strideC, int64_t batch, hipStream_t stream) {
    const int st = validate(M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    if (M == 0 || N == 0 || batch == 0) return SGEMM_STATUS_SUCCESS;
    if (config < 0) config = choose_config(M, N, K, batch);
    const ConfigEntry& c = kConfigs[config];
    return launch_gemm(c.kernel, c.bm, c.bn, c.threads, M, N, K, A, lda, strideA, B, ldb,
                       strideB, C, ldc, strideC, batch, stream);
}

// ------------------------------------------------------------------ split-K
// Split-K: the k range is cut into `splits` chunks of whole BK slices, each
// reduced by its own workgroup per output tile; the partial tiles join in the
// kernel (the last workgroup of a tile to arrive adds them in split order).
// A hybrid plan splits only the tiles past the last whole layer of one tile
// per CU: the first F = tiles - tiles % 256 take all of K with no join, and
// the chunks of the other R tiles fill one more layer, so every CU gets F / 256
// tiles plus about one chunk instead of some CUs one tile more than others.
// Workspace: a header of kSplitMaxTiles uint32 arrival counters, counter t
// for output tile t whatever the shape, then splits * BM * BN floats per
// tile.  The header's place and size do not depend on the call, so the zeros
// that every completed call leaves there serve the next call of any shape;
// products with more output tiles than the header holds are not split.
constexpr int64_t kMaxSplits = 64;
constexpr int64_t kSplitMaxTiles = SGEMM_SPLITK_MAX_TILES;
constexpr int64_t kSplitHeaderBytes = kSplitMaxTiles * 4;
// Join cost in the plan: the partial tiles are written once and read back
// once (device-coherent accesses that stay mostly in the MALL), at
// kJoinBytesPerUs, plus a fixed kJoinFixedUs for the counter round trip and
// the last workgroup's serial sum.  Set so that on a sweep of thin shapes
// (256 and 512 x 4096 x 4096, 512 x 512 x 8192, 128 x 4096 x 8192, 768^3 to
// 2048^3) the plan lands on the measured fastest choice or within 5 % of it.
constexpr double kJoinBytesPerUs = 4.0e6;
constexpr double kJoinFixedUs = 2.0;
// Hybrid plans: a chunk workgroup pays about kHybridChunkUs beyond its
// slices (first-slice latency, k-group exchange, partial write and arrival),
// and the join on the launch's tail path kHybridJoinUs.  Set so that on
// 12544 x 256 x 2304, 50176 x 128 x 1152, 12544 x 512 x 4608 (hybrid 8-23 %
// faster) and 3000 x 2000 x 1000, 2100 x 1000 x 1000 (2-8 % slower) the plan
// takes the faster kind.
constexpr double kHybridChunkUs = 3.0;
constexpr double kHybridJoinUs = 3.0;

struct SplitPlan {
    int config;          // tile configuration
    int64_t splits;      // effective number of k chunks (1: the plain kernel)
    int64_t kchunk;      // k values per chunk, a multiple of BK
    int64_t ws_bytes;    // workspace needed (0 when splits == 1)
    int64_t full_tiles;  // hybrid: tiles that take all of K (0: every tile splits)
};

SplitPlan make_split_plan(const ConfigEntry& c, int config, int64_t M, int64_t N, int64_t K,
                          int64_t want) {
    SplitPlan sp;
    sp.config = config;
    const int64_t slices = ceil_div(K, c.bk);
    const int64_t tiles = ceil_div(M, c.bm) * ceil_div(N, c.bn);
    int64_t s = want < 1 ? 1 : want;
    if (s > slices) s = slices;
    if (tiles > kSplitMaxTiles || s < 1) s = 1;
    sp.kchunk = (slices > 0 ? ceil_div(slices, s) : 1) * c.bk;
    sp.splits = K > 0 ? ceil_div(K, sp.kchunk) : 1;
    sp.ws_bytes = sp.splits > 1 ? kSplitHeaderBytes + tiles * sp.splits * c.bm * c.bn * 4 : 0;
    sp.full_tiles = 0;
    return sp;
}

// The hybrid plan with `want` chunks per split tile; false when the shape has
// no partial layer of tiles, no whole one, or the chunks do not spread evenly
// over the 8 XCDs.
bool make_hybrid_plan(const ConfigEntry& c, int config, int64_t M, int64_t N, int64_t K,
                      int64_t want, SplitPlan* out) {
    const int64_t tiles = ceil_div(M, c.bm) * ceil_div(N, c.bn);
    const int64_t rest = tiles % kNumCu, full = tiles - rest;
    if (tiles > kSplitMaxTiles || rest == 0 || full == 0) return false;
    SplitPlan sp = make_split_plan(c, config, M, N, K, want);
    if (sp.splits < 2 || (rest * sp.splits) % kNumXcd != 0) return false;
    sp.full_tiles = full;
    sp.ws_bytes = kSplitHeaderBytes + rest * sp.splits * c.bm * c.bn * 4;
    *out = sp;
    return true;
}

// Workgroups of a split launch: every chunk of every split tile, plus the
// hybrid's whole tiles.
int64_t split_blocks(const SplitPlan& sp, int64_t tiles) {
    return sp.full_tiles + (tiles - sp.full_tiles) * sp.splits;
}

double predict_split_us(const ConfigEntry& c, const SplitPlan& sp, int64_t M, int64_t N,
                        int64_t K) {
    const double tiles = (double)(ceil_div(M, c.bm) * ceil_div(N, c.bn));
    const double joined = tiles - (double)sp.full_tiles;  // tiles whose chunks join
    const double join_bytes = joined * (double)c.bm * c.bn * 4.0 * 2.0 * (double)sp.splits;
    if (sp.full_tiles > 0) {
        // Each CU runs full_tiles / 256 whole tiles and ceil(chunks / 256)
        // chunks; a chunk counts as its own one-tile time over a whole
        // tile's in the model's interpolation between one and w tiles per CU.
        const double area = (double)c.bm * c.bn;
        const double one = area * (c.one_a + c.one_b * (double)K);
        const double full_t = area * (c.two_a + c.two_b * (double)K);
        const double one_chunk = area * (c.one_a + c.one_b * (double)sp.kchunk) + kHybridChunkUs;
        const double chunks_per_cu = std::ceil(joined * (double)sp.splits / kNumCu);
        const double e = (double)sp.full_tiles / kNumCu + chunks_per_cu * one_chunk / one;
        const int w = c.per_cu < 1 ? 1 : c.per_cu;
        double t;
        if (w < 2) {
            t = e * one;
        } else {
            const double rounds = std::floor(e / w);
            const double rest = e - rounds * w;
            double last = 0.0;
            if (rest >= 1.0)
                last = one + (full_t - one) * (rest - 1.0) / (w - 1);
            else if (rest > 0.0)
                last = rest * one;
            t = rounds * full_t + last;
        }
        return t + kHybridJoinUs + join_bytes / kJoinBytesPerUs;
    }
    // One chunk is the plain kernel over all of K.
    const double t = predict_us(c, M, N, sp.splits == 1 ? K : sp.kchunk, sp.splits);
    if (sp.splits == 1) return t;
    return t + kJoinFixedUs + join_bytes / kJoinBytesPerUs;
}

// config < 0: every tile with a split-K variant (and the automatic plain
// choice); splits == 0: every split count up to kMaxSplits.  Plans whose
// workspace exceeds max_ws are left out.  The smallest predicted time wins.
// conv_c > 0: the product is a convolution's implicit GEMM over conv_c input
// channels; the tiles are those with a convolution split-K kernel, and a BK
// that does not divide conv_c (slices gathered through registers) counts
// four times slower, as in choose_conv_config.
// layout >= 0: the general form in that operand layout (transA + 2 transB);
// the tiles are those with its split-K kernel, and the unsplit choice is
// the general form's.
int plan_splitk(int config, int64_t M, int64_t N, int64_t K, int64_t splits, SplitPlan* out,
                int64_t max_ws = INT64_MAX, int64_t conv_c = 0, int layout = -1) {
    auto kernel_of = [&](const ConfigEntry& c) {
        return conv_c > 0 ? c.conv_splitk : layout >= 0 ? c.general_splitk[layout] : c.splitk;
    };
    if (config >= kNumConfigs) return SGEMM_STATUS_INVALID_CONFIG;
    if (config >= 0 && kernel_of(kConfigs[config]) == nullptr) return SGEMM_STATUS_INVALID_CONFIG;
    if (splits < 0 || splits > kMaxSplits) return SGEMM_STATUS_INVALID_SIZE;
    bool have = false;
    double best_us = 0.0;
    auto take = [&](const ConfigEntry& c, const SplitPlan& sp) {
        if (sp.ws_bytes > max_ws) return;
        const double t = predict_split_us(c, sp, M, N, K) *
                         (conv_c > 0 && conv_c % c.bk != 0 ? 4.0 : 1.0);
        if (!have || t < best_us * (1.0 - 1e-9)) {
            have = true;
            best_us = t;
            *out = sp;
        }
    };
    auto consider = [&](int idx, int64_t want) {
        const ConfigEntry& c = kConfigs[idx];
        take(c, make_split_plan(c, idx, M, N, K, want));
        // The library's own choice (splits == 0) may also split only the
        // last partial layer of tiles.
        SplitPlan hp;
        if (splits == 0 && make_hybrid_plan(c, idx, M, N, K, want, &hp)) take(c, hp);
    };
    if (config < 0 && splits == 0 && M > 0 && N > 0 && K > 0)
        consider(conv_c > 0 ? choose_conv_config(M, N, K, conv_c)
                            : choose_config(M, N, K, 1, layout >= 0), 1);
    for (int idx = 0; idx < kNumConfigs; ++idx) {
        if (config >= 0 ? idx != config : (kernel_of(kConfigs[idx]) == nullptr ||
                                           kConfigs[idx].per_cu == 0))
            continue;
        if (splits > 0) {
            consider(idx, splits);
        } else {
            for (int64_t s = 1; s <= kMaxSplits; ++s) consider(idx, s);
        }
    }
    if (have) return SGEMM_STATUS_SUCCESS;
    return max_ws < INT64_MAX ? SGEMM_STATUS_SCRATCH_TOO_SMALL : SGEMM_STATUS_INVALID_CONFIG;
}

// Arguments checked and the plan made, nothing enqueued yet: *needs_ws is
// set when the plan joins chunks through a workspace.
int prepare_splitk(int config, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                   const float* B, int64_t ldb, float* C, int64_t ldc, int64_t splits,
                   int64_t max_ws, SplitPlan* sp, bool* needs_ws) {
    int st = validate(M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, 1);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    st = plan_splitk(config, M, N, K, splits, sp, max_ws);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    *needs_ws = M > 0 && N > 0 && K > 0 && sp->splits > 1;
    if (*needs_ws) {
        const ConfigEntry& c = kConfigs[sp->config];
        const int64_t blocks = split_blocks(*sp, ceil_div(M, c.bm) * ceil_div(N, c.bn));
        if (blocks > kMaxWorkItems / c.threads) return SGEMM_STATUS_SIZE_OVERFLOW;
    }
    return SGEMM_STATUS_SUCCESS;
}

// Enqueues a prepared plan; the workspace is used only when the plan splits.
// conv: the product is that convolution's implicit GEMM (A the NHWC image,
// B the filters stored N x K).
int launch_splitk(const SplitPlan& sp, int64_t M, int64_t N, int64_t K, const float* A,
                  int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                  void* workspace, hipStream_t stream, const ConvGeom* conv = nullptr) {
    if (M == 0 || N == 0) return SGEMM_STATUS_SUCCESS;
    const ConfigEntry& c = kConfigs[sp.config];
    if (K == 0 || sp.splits == 1)
        return launch_gemm(conv != nullptr ? c.conv : c.kernel, c.bm, c.bn, c.threads, M, N, K,
                           A, lda, 0, B, ldb, 0, C, ldc, 0, 1, stream, 1.0f, 0.0f, conv);
    const int64_t tiles_m = ceil_div(M, c.bm), tiles_n = ceil_div(N, c.bn);
    const int64_t blocks = split_blocks(sp, tiles_m * tiles_n);
    GemmArgs p = {};
    if (conv != nullptr) p.conv = *conv;
    p.A = A;
    p.B = B;
    p.C = C;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    // Split b starts at column b * kchunk of A (the convolution's gather
    // adds it itself) and at row b * kchunk of B (column, for the filters).
    p.strideA = conv != nullptr ? 0 : sp.kchunk;
    p.strideB = conv != nullptr ? sp.kchunk : sp.kchunk * ldb;
    p.strideC = 0;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.tiles_m = (int)tiles_m;
    p.tiles_n = (int)tiles_n;
    p.batch_base = 0;
    p.batch_count = (int)sp.splits;
    p.alpha = 1.0f;
    p.beta = 0.0f;
    p.counters = (uint32_t*)workspace;
    p.ws = (float*)((char*)workspace + kSplitHeaderBytes);
    p.kchunk = (int)sp.kchunk;
    p.splits = (int)sp.splits;
    p.full_tiles = (int)sp.full_tiles;
    void* args[] = {&p};
    hipError_t e = hipLaunchKernel(conv != nullptr ? c.conv_splitk : c.splitk,
                                   dim3((unsigned)blocks), dim3(c.threads), args, 0, stream);
    return e == hipSuccess ? SGEMM_STATUS_SUCCESS : SGEMM_STATUS_LAUNCH_FAILED;
}

int run_splitk(int config, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
               const float* B, int64_t ldb, float* C, int64_t ldc, int64_t splits,
               void* workspace, int64_t workspace_bytes, hipStream_t stream) {
    SplitPlan sp;
    bool needs_ws = false;
    const int st = prepare_splitk(config, M, N, K, A, lda, B, ldb, C, ldc, splits, INT64_MAX,
                                  &sp, &needs_ws);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    if (needs_ws && (workspace == nullptr || workspace_bytes < sp.ws_bytes))
        return SGEMM_STATUS_INVALID_WORKSPACE;
    return launch_splitk(sp, M, N, K, A, lda, B, ldb, C, ldc, workspace, stream);
}

// ------------------------------------------------- split-K without allocation
// The device addresses of `scratch` (declared at file scope above), one per
// GPU, each looked up once with that device current.
constexpr int kMaxScratchDevices = 64;
struct ScratchState {
    void* ptr;     // device address of this device's scratch
    bool cleared;  // its counter header zeroed by a kernel that has run eagerly
};
std::mutex g_scratch_mutex;
ScratchState g_scratch[kMaxScratchDevices];

// The scratch of the device that `stream` runs on, its counter header
// zeroed on `stream` until one clearing launch has been made outside graph
// capture (zeros after loading are then not relied on; every completed call
// leaves the header zero again).
int scratch_for_stream(hipStream_t stream, void** out) {
    int dev = -1;
    if (stream != nullptr) {
        if (hipStreamGetDevice(stream, &dev) != hipSuccess) return SGEMM_STATUS_LAUNCH_FAILED;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return SGEMM_STATUS_LAUNCH_FAILED;
    }
    if (dev < 0 || dev >= kMaxScratchDevices) return SGEMM_STATUS_LAUNCH_FAILED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    ScratchState& st = g_scratch[dev];
    if (st.ptr == nullptr) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return SGEMM_STATUS_LAUNCH_FAILED;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return SGEMM_STATUS_LAUNCH_FAILED;
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return SGEMM_STATUS_LAUNCH_FAILED;
        if (e != hipSuccess || ptr == nullptr) return SGEMM_STATUS_LAUNCH_FAILED;
        st.ptr = ptr;
    }
    if (!st.cleared) {
        uint32_t* words = (uint32_t*)st.ptr;
        int64_t n = kSplitHeaderBytes / 4;
        void* args[] = {&words, &n};
        if (hipLaunchKernel((const void*)&clear_words_kernel, dim3((unsigned)(n / 256)), dim3(256),
                            args, 0, stream) != hipSuccess)
            return SGEMM_STATUS_LAUNCH_FAILED;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone)
            st.cleared = true;
    }
    *out = st.ptr;
    return SGEMM_STATUS_SUCCESS;
}

int run_splitk_noalloc(int config, int64_t M, int64_t N, int64_t K, const float* A,
                       int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                       int64_t splits, hipStream_t stream) {
    SplitPlan sp;
    bool needs_ws = false;
    int st = prepare_splitk(config, M, N, K, A, lda, B, ldb, C, ldc, splits,
                            SGEMM_SPLITK_SCRATCH_BYTES, &sp, &needs_ws);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    void* ws = nullptr;
    if (needs_ws) {
        st = scratch_for_stream(stream, &ws);
        if (st != SGEMM_STATUS_SUCCESS) return st;
    }
    return launch_splitk(sp, M, N, K, A, lda, B, ldb, C, ldc, ws, stream);
}

// C = beta * C over the M x N windows (+0 when beta == 0, C not read).
int launch_scale(int64_t M, int64_t N, float* C, int64_t ldc, int64_t strideC, int64_t batch,
                 float beta, hipStream_t stream) {
    int64_t blocks = ceil_div(M * N * batch, 256);
    if (blocks > 65536) blocks = 65536;
    int Mi = (int)M, Ni = (int)N, bi = (int)batch;
    void* args[] = {&C, &ldc, &strideC, &Mi, &Ni, &bi, &beta};
    hipError_t e = hipLaunchKernel((const void*)&scale_kernel, dim3((unsigned)blocks), dim3(256),
                                   args, 0, stream);
    return e == hipSuccess ? SGEMM_STATUS_SUCCESS : SGEMM_STATUS_LAUNCH_FAILED;
}

int run_general(int config, int transA, int transB, int64_t M, int64_t N, int64_t K,
                float alpha, const float* A, int64_t lda, int64_t strideA, const float* B,
                int64_t ldb, int64_t strideB, float beta, float* C, int64_t ldc,
                int64_t strideC, int64_t batch, hipStream_t stream) {
    const int st = validate_general(transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb,
                                    strideB, C, ldc, strideC, batch);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    const int layout = transA + 2 * transB;
    if (config >= 0 && (config >= kNumConfigs || kConfigs[config].general[layout] == nullptr))
        return SGEMM_STATUS_INVALID_CONFIG;
    if (M == 0 || N == 0 || batch == 0) return SGEMM_STATUS_SUCCESS;
    if (K == 0 || alpha == 0.0f) {
        // No product term: C = beta * C (nothing to do for beta == 1).
        if (beta == 1.0f) return SGEMM_STATUS_SUCCESS;
        return launch_scale(M, N, C, ldc, strideC, batch, beta, stream);
    }
    if (config < 0) config = choose_config(M, N, K, batch, true);
    const ConfigEntry& c = kConfigs[config];
    return launch_gemm(c.general[layout], c.bm, c.bn, c.threads, M, N, K, A, lda, strideA, B,
                       ldb, strideB, C, ldc, strideC, batch, stream, alpha, beta);
}

// The general form with its reduction split as in run_splitk: the chunks'
// operands start kchunk further along k (a row of A stored K x M, a column
// of B stored N x K), and the join's stores apply alpha and beta.
int run_ex_splitk(int config, int transA, int transB, int64_t M, int64_t N, int64_t K,
                  float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                  float beta, float* C, int64_t ldc, int64_t splits, void* workspace,
                  int64_t workspace_bytes, hipStream_t stream) {
    int st = validate_general(transA, transB, M, N, K, alpha, A, lda, 0, B, ldb, 0, C, ldc, 0, 1);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    const int layout = transA + 2 * transB;
    if (config >= kNumConfigs || (config >= 0 && kConfigs[config].general_splitk[layout] == nullptr))
        return SGEMM_STATUS_INVALID_CONFIG;
    if (splits < 0 || splits > kMaxSplits) return SGEMM_STATUS_INVALID_SIZE;
    if (M == 0 || N == 0) return SGEMM_STATUS_SUCCESS;
    if (K == 0 || alpha == 0.0f) {
        if (beta == 1.0f) return SGEMM_STATUS_SUCCESS;
        return launch_scale(M, N, C, ldc, 0, 1, beta, stream);
    }
    SplitPlan sp;
    st = plan_splitk(config, M, N, K, splits, &sp, INT64_MAX, 0, layout);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    const ConfigEntry& c = kConfigs[sp.config];
    if (sp.splits == 1)
        return launch_gemm(c.general[layout], c.bm, c.bn, c.threads, M, N, K, A, lda, 0, B, ldb,
                           0, C, ldc, 0, 1, stream, alpha, beta);
    const int64_t tiles_m = ceil_div(M, c.bm), tiles_n = ceil_div(N, c.bn);
    const int64_t blocks = split_blocks(sp, tiles_m * tiles_n);
    if (blocks > kMaxWorkItems / c.threads) return SGEMM_STATUS_SIZE_OVERFLOW;
    if (workspace == nullptr || workspace_bytes < sp.ws_bytes)
        return SGEMM_STATUS_INVALID_WORKSPACE;
    GemmArgs p = {};
    p.A = A;
    p.B = B;
    p.C = C;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    p.strideA = transA ? sp.kchunk * lda : sp.kchunk;
    p.strideB = transB ? sp.kchunk : sp.kchunk * ldb;
    p.strideC = 0;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.tiles_m = (int)tiles_m;
    p.tiles_n = (int)tiles_n;
    p.batch_base = 0;
    p.batch_count = (int)sp.splits;
    p.alpha = alpha;
    p.beta = beta;
    p.counters = (uint32_t*)workspace;
    p.ws = (float*)((char*)workspace + kSplitHeaderBytes);
    p.kchunk = (int)sp.kchunk;
    p.splits = (int)sp.splits;
    p.full_tiles = (int)sp.full_tiles;
    void* args[] = {&p};
    hipError_t e = hipLaunchKernel(c.general_splitk[layout], dim3((unsigned)blocks),
                                   dim3(c.threads), args, 0, stream);
    return e == hipSuccess ? SGEMM_STATUS_SUCCESS : SGEMM_STATUS_LAUNCH_FAILED;
}

// Output extent of a convolution along one axis; -1 for invalid arguments.
int64_t conv_extent(int64_t in, int64_t pad, int64_t f, int64_t stride, int64_t dil) {
    if (in < 0 || pad < 0 || f < 0 || stride < 1 || dil < 1) return -1;
    const int64_t span = in + 2 * pad - dil * (f - 1) - 1;
    return span < 0 ? 0 : span / stride + 1;
}

constexpr int64_t kConvMaxExtent = (int64_t)1 << 29;  // image extents and padded spans

// Checked sizes of a convolution run as an implicit GEMM.
struct ConvPlan {
    int64_t P, Q, Mg, Kg, x_elems;
};

int conv_plan(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S,
              int64_t pad_h, int64_t pad_w, int64_t stride_h, int64_t stride_w, int64_t dil_h,
              int64_t dil_w, ConvPlan* out) {
    if (N < 0 || H < 0 || W < 0 || C < 0 || K < 0 || R < 0 || S < 0 || pad_h < 0 || pad_w < 0 ||
        stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1)
        return SGEMM_STATUS_INVALID_SIZE;
    // Every in-kernel index (p * stride - pad + r * dil, and the like) stays
    // inside int32 when the padded spans are below 2^29.
    if (H + 2 * pad_h >= kConvMaxExtent || W + 2 * pad_w >= kConvMaxExtent ||
        (R > 0 && (R - 1) > kConvMaxExtent / dil_h) || (S > 0 && (S - 1) > kConvMaxExtent / dil_w) ||
        stride_h >= kConvMaxExtent || stride_w >= kConvMaxExtent || N > kMaxDim || C > kMaxDim ||
        K > kMaxDim)
        return SGEMM_STATUS_SIZE_OVERFLOW;
    ConvPlan pl;
    pl.P = conv_extent(H, pad_h, R, stride_h, dil_h);
    pl.Q = conv_extent(W, pad_w, S, stride_w, dil_w);
    int64_t t, y_elems, w_elems;
    if (__builtin_mul_overflow(N, pl.P, &t) || __builtin_mul_overflow(t, pl.Q, &pl.Mg) ||
        __builtin_mul_overflow(R, S, &t) || __builtin_mul_overflow(t, C, &pl.Kg) ||
        __builtin_mul_overflow(N, H, &t) || __builtin_mul_overflow(t, W, &t) ||
        __builtin_mul_overflow(t, C, &pl.x_elems) || __builtin_mul_overflow(K, pl.Kg, &w_elems) ||
        __builtin_mul_overflow(pl.Mg, K, &y_elems) || pl.Mg > kMaxDim || pl.Kg > kMaxDim)
        return SGEMM_STATUS_SIZE_OVERFLOW;
    *out = pl;
    return SGEMM_STATUS_SUCCESS;
}

ConvGeom conv_geom(int64_t H, int64_t W, int64_t C, int64_t S, int64_t pad_h, int64_t pad_w,
                   int64_t stride_h, int64_t stride_w, int64_t dil_h, int64_t dil_w,
                   const ConvPlan& pl) {
    ConvGeom g;
    g.H = (int)H;
    g.W = (int)W;
    g.C = (int)C;
    g.P = (int)pl.P;
    g.Q = (int)pl.Q;
    g.S = (int)S;
    g.pad_h = (int)pad_h;
    g.pad_w = (int)pad_w;
    g.stride_h = (int)stride_h;
    g.stride_w = (int)stride_w;
    g.dil_h = (int)dil_h;
    g.dil_w = (int)dil_w;
    return g;
}

int run_conv(int config, int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R,
             int64_t S, int64_t pad_h, int64_t pad_w, int64_t stride_h, int64_t stride_w,
             int64_t dil_h, int64_t dil_w, const float* x, const float* w, float* y,
             hipStream_t stream) {
    ConvPlan pl;
    const int st = conv_plan(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w,
                             &pl);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    if (config >= 0 && (config >= kNumConfigs || kConfigs[config].conv == nullptr))
        return SGEMM_STATUS_INVALID_CONFIG;
    if (pl.Mg == 0 || K == 0) return SGEMM_STATUS_SUCCESS;
    if (y == nullptr) return SGEMM_STATUS_NULL_POINTER;
    if (pl.Kg == 0)  // every output is the empty sum: +0
        return launch_gemm(nullptr, 1, 1, 1, pl.Mg, K, 0, nullptr, 1, 0, nullptr, 1, 0, y, K, 0,
                           1, stream);
    if (x == nullptr || w == nullptr) return SGEMM_STATUS_NULL_POINTER;
    if (config < 0) config = choose_conv_config(pl.Mg, K, pl.Kg, C);
    const ConfigEntry& c = kConfigs[config];
    const ConvGeom g = conv_geom(H, W, C, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, pl);
    return launch_gemm(c.conv, c.bm, c.bn, c.threads, pl.Mg, K, pl.Kg, x, pl.Kg, 0, w, pl.Kg, 0, y,
                       K, 0, 1, stream, 1.0f, 0.0f, &g);
}

// The convolution's implicit GEMM with its reduction split as in
// sgemm_splitk.  *sp gets the plan; nothing is enqueued.
int plan_conv_splitk(int config, int64_t N, int64_t H, int64_t W, int64_t C, int64_t K,
                     int64_t R, int64_t S, int64_t pad_h, int64_t pad_w, int64_t stride_h,
                     int64_t stride_w, int64_t dil_h, int64_t dil_w, int64_t splits,
                     ConvPlan* pl, SplitPlan* sp) {
    const int st = conv_plan(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w,
                             pl);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    if (config >= 0 && (config >= kNumConfigs || kConfigs[config].conv_splitk == nullptr))
        return SGEMM_STATUS_INVALID_CONFIG;
    if (splits < 0 || splits > kMaxSplits) return SGEMM_STATUS_INVALID_SIZE;
    if (pl->Mg == 0 || K == 0 || pl->Kg == 0) {  // nothing to split
        const int idx = config >= 0 ? config
                                    : choose_conv_config(pl->Mg > 0 ? pl->Mg : 1, K > 0 ? K : 1,
                                                         pl->Kg > 0 ? pl->Kg : 1, C);
        *sp = SplitPlan{idx, 1, 0, 0, 0};
        return SGEMM_STATUS_SUCCESS;
    }
    return plan_splitk(config, pl->Mg, K, pl->Kg, splits, sp, INT64_MAX, C);
}

int run_conv_splitk(int config, int64_t N, int64_t H, int64_t W, int64_t C, int64_t K,
                    int64_t R, int64_t S, int64_t pad_h, int64_t pad_w, int64_t stride_h,
                    int64_t stride_w, int64_t dil_h, int64_t dil_w, const float* x,
                    const float* w, float* y, int64_t splits, void* workspace,
                    int64_t workspace_bytes, hipStream_t stream) {
    ConvPlan pl;
    SplitPlan sp;
    const int st = plan_conv_splitk(config, N, H, W, C, K, R, S, pad_h, pad_w, stride_h,
                                    stride_w, dil_h, dil_w, splits, &pl, &sp);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    if (pl.Mg == 0 || K == 0) return SGEMM_STATUS_SUCCESS;
    if (y == nullptr) return SGEMM_STATUS_NULL_POINTER;
    if (pl.Kg == 0)  // every output is the empty sum: +0
        return launch_gemm(nullptr, 1, 1, 1, pl.Mg, K, 0, nullptr, 1, 0, nullptr, 1, 0, y, K, 0,
                           1, stream);
    if (x == nullptr || w == nullptr) return SGEMM_STATUS_NULL_POINTER;
    if (sp.splits > 1) {
        const ConfigEntry& c = kConfigs[sp.config];
        const int64_t blocks = split_blocks(sp, ceil_div(pl.Mg, c.bm) * ceil_div(K, c.bn));
        if (blocks > kMaxWorkItems / c.threads) return SGEMM_STATUS_SIZE_OVERFLOW;
        if (workspace == nullptr || workspace_bytes < sp.ws_bytes)
            return SGEMM_STATUS_INVALID_WORKSPACE;
    }
    const ConvGeom g = conv_geom(H, W, C, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, pl);
    return launch_splitk(sp, pl.Mg, K, pl.Kg, x, pl.Kg, w, pl.Kg, y, K, workspace, stream, &g);
}

int run_valu(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, int64_t strideA,
             const float* B, int64_t ldb, int64_t strideB, float* C, int64_t ldc,
             int64_t strideC, int64_t batch, hipStream_t stream) {
    const int st = validate(M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    if (M == 0 || N == 0 || batch == 0) return SGEMM_STATUS_SUCCESS;
    return launch_gemm((const void*)&sgemm_valu_kernel, ValuTile::BM, ValuTile::BN,
                       ValuTile::NT, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                       batch, stream);
}

}  // namespace

extern "C" {

int sgemm(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
          int64_t ldb, float* C, int64_t ldc, hipStream_t stream) {
    return run_mfma(-1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, 1, stream);
}

int sgemm_strided_batched(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                          int64_t strideA, const float* B, int64_t ldb, int64_t strideB,
                          float* C, int64_t ldc, int64_t strideC, int64_t batch,
                          hipStream_t stream) {
    return run_mfma(-1, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch,
                    stream);
}

int sgemm_valu(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
               int64_t ldb, float* C, int64_t ldc, hipStream_t stream) {
    return run_valu(M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, 1, stream);
}

int sgemm_valu_strided_batched(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                               int64_t strideA, const float* B, int64_t ldb, int64_t strideB,
                               float* C, int64_t ldc, int64_t strideC, int64_t batch,
                               hipStream_t stream) {
    return run_valu(M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, stream);
}

int sgemm_with_config(int config, int64_t M, int64_t N, int64_t K, const float* A,
                      int64_t lda, int64_t strideA, const float* B, int64_t ldb,
                      int64_t strideB, float* C, int64_t ldc, int64_t strideC, int64_t batch,
                      hipStream_t stream) {
    if (config < 0 || config >= kNumConfigs) return SGEMM_STATUS_INVALID_CONFIG;
    return run_mfma(config, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch,
                    stream);
}

int sgemm_splitk(int config, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                 const float* B, int64_t ldb, float* C, int64_t ldc, int64_t splits,
                 void* workspace, int64_t workspace_bytes, hipStream_t stream) {
    return run_splitk(config, M, N, K, A, lda, B, ldb, C, ldc, splits, workspace,
                      workspace_bytes, stream);
}

int sgemm_splitk_noalloc(int config, int64_t M, int64_t N, int64_t K, const float* A,
                         int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                         int64_t splits, hipStream_t stream) {
    return run_splitk_noalloc(config, M, N, K, A, lda, B, ldb, C, ldc, splits, stream);
}

int64_t sgemm_splitk_plan(int config, int64_t M, int64_t N, int64_t K, int64_t splits,
                          int* plan_config, int64_t* plan_splits) {
    if (M < 0 || N < 0 || K < 0) return SGEMM_STATUS_INVALID_SIZE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return SGEMM_STATUS_SIZE_OVERFLOW;
    SplitPlan sp;
    const int st = plan_splitk(config, M, N, K, splits, &sp);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    if (plan_config != nullptr) *plan_config = sp.config;
    if (plan_splits != nullptr) *plan_splits = sp.splits;
    return (M == 0 || N == 0 || K == 0) ? 0 : sp.ws_bytes;
}

int64_t sgemm_splitk_plan_full_tiles(int config, int64_t M, int64_t N, int64_t K,
                                      int64_t splits) {
    if (M < 0 || N < 0 || K < 0) return SGEMM_STATUS_INVALID_SIZE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return SGEMM_STATUS_SIZE_OVERFLOW;
    SplitPlan sp;
    const int st = plan_splitk(config, M, N, K, splits, &sp);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    return sp.splits > 1 ? sp.full_tiles : 0;
}

int sgemm_ex_splitk(int config, int transA, int transB, int64_t M, int64_t N, int64_t K,
                    float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                    float beta, float* C, int64_t ldc, int64_t splits, void* workspace,
                    int64_t workspace_bytes, hipStream_t stream) {
    return run_ex_splitk(config, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                         splits, workspace, workspace_bytes, stream);
}

int64_t sgemm_ex_splitk_plan(int config, int transA, int transB, int64_t M, int64_t N,
                             int64_t K, int64_t splits, int* plan_config, int64_t* plan_splits) {
    if ((transA != 0 && transA != 1) || (transB != 0 && transB != 1))
        return SGEMM_STATUS_INVALID_OP;
    if (M < 0 || N < 0 || K < 0) return SGEMM_STATUS_INVALID_SIZE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return SGEMM_STATUS_SIZE_OVERFLOW;
    const int layout = transA + 2 * transB;
    if (config >= kNumConfigs || (config >= 0 && kConfigs[config].general_splitk[layout] == nullptr))
        return SGEMM_STATUS_INVALID_CONFIG;
    SplitPlan sp;
    const int st = plan_splitk(config, M, N, K, splits, &sp, INT64_MAX, 0, layout);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    if (plan_config != nullptr) *plan_config = sp.config;
    if (plan_splits != nullptr) *plan_splits = sp.splits;
    return (M == 0 || N == 0 || K == 0) ? 0 : sp.ws_bytes;
}

int64_t sgemm_ex_splitk_plan_full_tiles(int config, int transA, int transB, int64_t M,
                                        int64_t N, int64_t K, int64_t splits) {
    int plan_config = -1;
    int64_t plan_splits = 0;
    const int64_t st = sgemm_ex_splitk_plan(config, transA, transB, M, N, K, splits,
                                            &plan_config, &plan_splits);
    if (st < 0) return st;
    SplitPlan sp;
    const int r = plan_splitk(config, M, N, K, splits, &sp, INT64_MAX, 0, transA + 2 * transB);
    if (r != SGEMM_STATUS_SUCCESS) return r;
    return sp.splits > 1 ? sp.full_tiles : 0;
}

int sgemm_config_has_general_splitk(int config) {
    if (config < 0 || config >= kNumConfigs) return SGEMM_STATUS_INVALID_CONFIG;
    return kConfigs[config].general_splitk[0] != nullptr ? 1 : 0;
}

int sgemm_config_has_splitk(int config) {
    if (config < 0 || config >= kNumConfigs) return SGEMM_STATUS_INVALID_CONFIG;
    return kConfigs[config].splitk != nullptr ? 1 : 0;
}

int sgemm_num_configs(void) { return kNumConfigs; }

int sgemm_config_info(int config, char* buf, int64_t len, int* bm, int* bn, int* bk,
                      int* threads) {
    if (config < 0 || config >= kNumConfigs) return SGEMM_STATUS_INVALID_CONFIG;
    const ConfigEntry& c = kConfigs[config];
    if (buf != nullptr && len > 0) snprintf(buf, (size_t)len, "%s", c.name);
    if (bm) *bm = c.bm;
    if (bn) *bn = c.bn;
    if (bk) *bk = c.bk;
    if (threads) *threads = c.threads;
    return SGEMM_STATUS_SUCCESS;
}

int sgemm_select_config(int64_t M, int64_t N, int64_t K, int64_t batch) {
    if (M < 0 || N < 0 || K < 0 || batch < 0) return SGEMM_STATUS_INVALID_SIZE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim || batch > kMaxDim)
        return SGEMM_STATUS_SIZE_OVERFLOW;
    if (M == 0 || N == 0 || batch == 0) return 0;
    return choose_config(M, N, K, batch);
}

int sgemm_ex(int transA, int transB, int64_t M, int64_t N, int64_t K, float alpha,
             const float* A, int64_t lda, const float* B, int64_t ldb, float beta, float* C,
             int64_t ldc, hipStream_t stream) {
    return run_general(-1, transA, transB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc,
                       0, 1, stream);
}

int sgemm_ex_strided_batched(int transA, int transB, int64_t M, int64_t N, int64_t K,
                             float alpha, const float* A, int64_t lda, int64_t strideA,
                             const float* B, int64_t ldb, int64_t strideB, float beta, float* C,
                             int64_t ldc, int64_t strideC, int64_t batch, hipStream_t stream) {
    return run_general(-1, transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB,
                       beta, C, ldc, strideC, batch, stream);
}

int sgemm_ex_with_config(int config, int transA, int transB, int64_t M, int64_t N, int64_t K,
                         float alpha, const float* A, int64_t lda, int64_t strideA,
                         const float* B, int64_t ldb, int64_t strideB, float beta, float* C,
                         int64_t ldc, int64_t strideC, int64_t batch, hipStream_t stream) {
    if (config < 0 || config >= kNumConfigs) return SGEMM_STATUS_INVALID_CONFIG;
    return run_general(config, transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb,
                       strideB, beta, C, ldc, strideC, batch, stream);
}

int sgemm_config_has_general_form(int config) {
    if (config < 0 || config >= kNumConfigs) return SGEMM_STATUS_INVALID_CONFIG;
    return kConfigs[config].general[0] != nullptr ? 1 : 0;
}

int sgemm_select_general_config(int64_t M, int64_t N, int64_t K, int64_t batch) {
    if (M < 0 || N < 0 || K < 0 || batch < 0) return SGEMM_STATUS_INVALID_SIZE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim || batch > kMaxDim)
        return SGEMM_STATUS_SIZE_OVERFLOW;
    return choose_config(M, N, K, batch, true);
}

int sgemm_config_workgroups_per_cu(int config) {
    if (config < 0 || config >= kNumConfigs) return SGEMM_STATUS_INVALID_CONFIG;
    const ConfigEntry& c = kConfigs[config];
    // The runtime's answer counts the registers the compiler actually used;
    // the launch bound in the table is only the floor it guarantees.
    // A failed lookup clears only an error of its own: one the caller had
    // pending (an earlier asynchronous launch failure, say) stays in place.
    const hipError_t before = hipPeekAtLastError();
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, c.kernel, c.threads, 0) ==
            hipSuccess &&
        blocks > 0)
        return blocks;
    if (before == hipSuccess) (void)hipGetLastError();
    return c.wg_per_cu;
}

int sgemm_config_selectable(int config) {
    if (config < 0 || config >= kNumConfigs) return SGEMM_STATUS_INVALID_CONFIG;
    return kConfigs[config].per_cu > 0 ? 1 : 0;
}

double sgemm_config_predict_us(int config, int64_t M, int64_t N, int64_t K, int64_t batch) {
    if (config < 0 || config >= kNumConfigs) return (double)SGEMM_STATUS_INVALID_CONFIG;
    if (M < 0 || N < 0 || K < 0 || batch < 0) return (double)SGEMM_STATUS_INVALID_SIZE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim || batch > kMaxDim)
        return (double)SGEMM_STATUS_SIZE_OVERFLOW;
    if (kConfigs[config].per_cu == 0) return (double)SGEMM_STATUS_INVALID_CONFIG;
    return predict_us(kConfigs[config], M, N, K, batch);
}

int sgemm_autotune(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                   int64_t strideA, const float* B, int64_t ldb, int64_t strideB, float* C,
                   int64_t ldc, int64_t strideC, int64_t batch, hipStream_t stream, int reps,
                   int* best_config, float* best_ms) {
    if (best_config == nullptr) return SGEMM_STATUS_NULL_POINTER;
    if (reps < 1) return SGEMM_STATUS_INVALID_SIZE;
    const int st = validate(M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    *best_config = (M == 0 || N == 0 || batch == 0) ? 0 : choose_config(M, N, K, batch);
    if (best_ms) *best_ms = 0.0f;
    if (M == 0 || N == 0 || batch == 0 || K == 0) return SGEMM_STATUS_SUCCESS;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return SGEMM_STATUS_LAUNCH_FAILED;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return SGEMM_STATUS_LAUNCH_FAILED;
    }
    int status = SGEMM_STATUS_SUCCESS;
    float best = -1.0f;
    for (int idx = 0; idx < kNumConfigs && status == SGEMM_STATUS_SUCCESS; ++idx) {
        const ConfigEntry& c = kConfigs[idx];
        if (c.per_cu == 0) continue;
        auto launch = [&]() {
            return launch_gemm(c.kernel, c.bm, c.bn, c.threads, M, N, K, A, lda, strideA, B,
                               ldb, strideB, C, ldc, strideC, batch, stream);
        };
        status = launch();  // warm-up
        if (status != SGEMM_STATUS_SUCCESS) break;
        if (hipEventRecord(e0, stream) != hipSuccess) status = SGEMM_STATUS_LAUNCH_FAILED;
        for (int r = 0; r < reps && status == SGEMM_STATUS_SUCCESS; ++r) status = launch();
        if (status != SGEMM_STATUS_SUCCESS) break;
        float ms = 0.0f;
        if (hipEventRecord(e1, stream) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
            hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
            status = SGEMM_STATUS_LAUNCH_FAILED;
            break;
        }
        ms /= (float)reps;
        if (best < 0.0f || ms < best) {
            best = ms;
            *best_config = idx;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (status != SGEMM_STATUS_SUCCESS) return status;
    // Leave C holding the product of the chosen configuration.
    const ConfigEntry& c = kConfigs[*best_config];
    status = launch_gemm(c.kernel, c.bm, c.bn, c.threads, M, N, K, A, lda, strideA, B, ldb,
                         strideB, C, ldc, strideC, batch, stream);
    if (best_ms) *best_ms = best;
    return status;
}

int conv2d_nhwc(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S,
                int64_t pad_h, int64_t pad_w, int64_t stride_h, int64_t stride_w, int64_t dil_h,
                int64_t dil_w, const float* x, const float* w, float* y, hipStream_t stream) {
    return run_conv(-1, N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, x,
                    w, y, stream);
}

int conv2d_nhwc_with_config(int config, int64_t N, int64_t H, int64_t W, int64_t C, int64_t K,
                            int64_t R, int64_t S, int64_t pad_h, int64_t pad_w, int64_t stride_h,
                            int64_t stride_w, int64_t dil_h, int64_t dil_w, const float* x,
                            const float* w, float* y, hipStream_t stream) {
    if (config < 0 || config >= kNumConfigs) return SGEMM_STATUS_INVALID_CONFIG;
    return run_conv(config, N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w,
                    x, w, y, stream);
}

int conv2d_nhwc_output_size(int64_t H, int64_t W, int64_t R, int64_t S, int64_t pad_h,
                            int64_t pad_w, int64_t stride_h, int64_t stride_w, int64_t dil_h,
                            int64_t dil_w, int64_t* P, int64_t* Q) {
    const int64_t p = conv_extent(H, pad_h, R, stride_h, dil_h);
    const int64_t q = conv_extent(W, pad_w, S, stride_w, dil_w);
    if (p < 0 || q < 0) return SGEMM_STATUS_INVALID_SIZE;
    if (P) *P = p;
    if (Q) *Q = q;
    return SGEMM_STATUS_SUCCESS;
}

int conv2d_config_available(int config) {
    if (config < 0 || config >= kNumConfigs) return SGEMM_STATUS_INVALID_CONFIG;
    return kConfigs[config].conv != nullptr ? 1 : 0;
}

int conv2d_select_config(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R,
                         int64_t S, int64_t pad_h, int64_t pad_w, int64_t stride_h,
                         int64_t stride_w, int64_t dil_h, int64_t dil_w) {
    ConvPlan pl;
    const int st = conv_plan(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w,
                             &pl);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    return choose_conv_config(pl.Mg > 0 ? pl.Mg : 1, K > 0 ? K : 1, pl.Kg > 0 ? pl.Kg : 1, C);
}

int conv2d_nhwc_splitk(int config, int64_t N, int64_t H, int64_t W, int64_t C, int64_t K,
                       int64_t R, int64_t S, int64_t pad_h, int64_t pad_w, int64_t stride_h,
                       int64_t stride_w, int64_t dil_h, int64_t dil_w, const float* x,
                       const float* wt, float* y, int64_t splits, void* workspace,
                       int64_t workspace_bytes, hipStream_t stream) {
    return run_conv_splitk(config, N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h,
                           dil_w, x, wt, y, splits, workspace, workspace_bytes, stream);
}

int64_t conv2d_nhwc_splitk_plan(int config, int64_t N, int64_t H, int64_t W, int64_t C,
                                int64_t K, int64_t R, int64_t S, int64_t pad_h, int64_t pad_w,
                                int64_t stride_h, int64_t stride_w, int64_t dil_h,
                                int64_t dil_w, int64_t splits, int* plan_config,
                                int64_t* plan_splits, int64_t* plan_full_tiles) {
    ConvPlan pl;
    SplitPlan sp;
    const int st = plan_conv_splitk(config, N, H, W, C, K, R, S, pad_h, pad_w, stride_h,
                                    stride_w, dil_h, dil_w, splits, &pl, &sp);
    if (st != SGEMM_STATUS_SUCCESS) return st;
    if (plan_config != nullptr) *plan_config = sp.config;
    if (plan_splits != nullptr) *plan_splits = sp.splits;
    if (plan_full_tiles != nullptr) *plan_full_tiles = sp.splits > 1 ? sp.full_tiles : 0;
    return sp.splits > 1 ? sp.ws_bytes : 0;
}

int conv2d_config_has_splitk(int config) {
    if (config < 0 || config >= kNumConfigs) return SGEMM_STATUS_INVALID_CONFIG;
    return kConfigs[config].conv_splitk != nullptr ? 1 : 0;
}

const char* sgemm_status_string(int status) {
    switch (status) {
        case SGEMM_STATUS_SUCCESS: return "success";
        case SGEMM_STATUS_INVALID_SIZE: return "invalid size: M, N, K or batch is negative";
        case SGEMM_STATUS_INVALID_LD: return "invalid leading dimension";
        case SGEMM_STATUS_NULL_POINTER: return "null operand pointer";
        case SGEMM_STATUS_SIZE_OVERFLOW: return "size overflow";
        case SGEMM_STATUS_INVALID_STRIDE: return "invalid batch stride";
        case SGEMM_STATUS_LAUNCH_FAILED: return "kernel launch failed";
        case SGEMM_STATUS_INVALID_CONFIG: return "unknown tile configuration";
        case SGEMM_STATUS_INVALID_OP: return "invalid transpose flag (must be 0 or 1)";
        case SGEMM_STATUS_INVALID_WORKSPACE:
            return "split-K workspace is NULL or smaller than sgemm_splitk_plan reports";
        case SGEMM_STATUS_SCRATCH_TOO_SMALL:
            return "split-K plan needs more workspace than the library's scratch "
                   "(SGEMM_SPLITK_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

}  // extern "C"
