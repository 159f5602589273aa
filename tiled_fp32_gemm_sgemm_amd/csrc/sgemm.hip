// Host side of the C ABI declared in include/sgemm.h: argument validation,
// tile-configuration choice, grid arithmetic and the launch on the caller's
// stream.  Arguments are checked before anything is enqueued, and the launch
// status from HIP is returned ("CMU DLSys Lecture 12: GPU Acceleration"
// section 2: launches are asynchronous, and API and launch errors are checked).
#include "sgemm.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mfma_dl_kernel.hpp"
#include "mfma_kernel.hpp"
#include "tile_common.hpp"
#include "valu_kernel.hpp"

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
// Control build: A stored unswizzled (bank conflicts on purpose); never chosen.
using Dl256x256k32m32Plain = DlTile<256, 256, 32, 2, 4, 32, 2, 8, 2, false>;

struct ConfigEntry {
    const char* name;
    int bm, bn, bk, threads;
    const void* kernel;
    double tile_efficiency;  // relative per-CU throughput of a full tile (tuning input)
    int blocks_per_cu;       // workgroups that fit on one CU at once
};

#define SGEMM_CFG(T, name, eff, per_cu) \
    { name, T::BM, T::BN, T::BK, T::NT, (const void*)&sgemm_mfma_kernel<T>, eff, per_cu }
#define SGEMM_DL_CFG(T, name, eff, per_cu) \
    { name, T::BM, T::BN, T::BK, T::NT, (const void*)&sgemm_mfma_dl_kernel<T>, eff, per_cu }

const ConfigEntry kConfigs[] = {
    SGEMM_CFG(Cfg256x128, "mfma32_256x128x16_w2x2", 0.94, 2),
    SGEMM_CFG(Cfg128x128, "mfma32_128x128x16_w2x2", 0.90, 3),
    SGEMM_CFG(Cfg64x64, "mfma32_64x64x16_w2x2", 0.60, 8),
    SGEMM_CFG(Cfg256x256, "mfma32_256x256x16_w2x4", 0.96, 1),
    SGEMM_CFG(Cfg256x256k32, "mfma32_256x256x32_w2x4", 1.00, 1),
    SGEMM_CFG(Cfg128x128k32, "mfma32_128x128x32_w2x2", 0.90, 2),
    SGEMM_CFG(Cfg128x128k32m16, "mfma16_128x128x32_w2x2", 0.90, 2),
    SGEMM_CFG(Cfg64x64k32m16, "mfma16_64x64x32_w2x2", 0.60, 4),
    SGEMM_CFG(Cfg256x256m32w1, "mfma32_256x256x16_w2x2", 0.98, 1),
    SGEMM_CFG(Cfg256x256k32m32w1, "mfma32_256x256x32_w2x2", 0.98, 1),
    SGEMM_DL_CFG(Dl256x256k32m32, "dl32_256x256x32_w2x4", 1.04, 1),
    SGEMM_DL_CFG(Dl256x256k16m32, "dl32_256x256x16_w2x4", 1.02, 1),
    SGEMM_DL_CFG(Dl256x128k32m32, "dl32_256x128x32_w2x2", 0.96, 1),
    SGEMM_DL_CFG(Dl128x128k32m32, "dl32_128x128x32_w2x2", 0.92, 2),
    SGEMM_DL_CFG(Dl256x256k32m32Plain, "dl32_256x256x32_w2x4_unswizzled", 0.0, 1),
    SGEMM_DL_CFG(Dl128x128k32m32s4, "dl32_128x128x32_w2x2_s4", 0.92, 1),
    SGEMM_DL_CFG(Dl64x64k32m32s4, "dl32_64x64x32_w2x2_s4", 0.60, 2),
    SGEMM_DL_CFG(Dl256x192k32m32, "dl32_256x192x32_w4x2", 1.00, 1),
    SGEMM_DL_CFG(Dl192x256k32m32, "dl32_192x256x32_w2x4", 1.00, 1),
};
#undef SGEMM_CFG
#undef SGEMM_DL_CFG
constexpr int kNumConfigs = (int)(sizeof(kConfigs) / sizeof(kConfigs[0]));
constexpr int kNumCu = 256;  // MI355X compute units

constexpr int64_t kMaxDim = INT32_MAX;
constexpr int64_t kMaxGridX = INT32_MAX;

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

int validate(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, int64_t strideA,
             const float* B, int64_t ldb, int64_t strideB, const float* C, int64_t ldc,
             int64_t strideC, int64_t batch) {
    if (M < 0 || N < 0 || K < 0 || batch < 0) return SGEMM_STATUS_INVALID_SIZE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim || batch > kMaxDim)
        return SGEMM_STATUS_SIZE_OVERFLOW;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1))
        return SGEMM_STATUS_INVALID_LD;
    if (strideA < 0 || strideB < 0 || strideC < 0) return SGEMM_STATUS_INVALID_STRIDE;
    if (M == 0 || N == 0 || batch == 0) return SGEMM_STATUS_SUCCESS;
    if (batch > 1) {
        const int64_t one_c = span_end(M, N, ldc, 0, 1);
        if (one_c < 0) return SGEMM_STATUS_SIZE_OVERFLOW;
        if (strideC < one_c) return SGEMM_STATUS_INVALID_STRIDE;
    }
    if (C == nullptr) return SGEMM_STATUS_NULL_POINTER;
    if (K > 0 && (A == nullptr || B == nullptr)) return SGEMM_STATUS_NULL_POINTER;
    if (span_end(M, K, lda, strideA, batch) < 0 || span_end(K, N, ldb, strideB, batch) < 0 ||
        span_end(M, N, ldc, strideC, batch) < 0)
        return SGEMM_STATUS_SIZE_OVERFLOW;
    return SGEMM_STATUS_SUCCESS;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shape -> configuration.  Score = useful fraction of the padded tiles x how
// evenly the tiles fill the CUs' resident slots x a per-tile efficiency.
// Control builds (efficiency 0) are never chosen.
int choose_config(int64_t M, int64_t N, int64_t K, int64_t batch) {
    (void)K;
    int best = 0;
    double best_score = -1.0;
    for (int idx = 0; idx < kNumConfigs; ++idx) {
        const ConfigEntry& c = kConfigs[idx];
        if (c.tile_efficiency <= 0.0) continue;
        const int64_t tiles = ceil_div(M, c.bm) * ceil_div(N, c.bn) * batch;
        const double useful = (double)M * N * batch / ((double)tiles * c.bm * c.bn);
        const int64_t slots = (int64_t)kNumCu * c.blocks_per_cu;
        const int64_t rounds = ceil_div(tiles, slots);
        const double fill = (double)tiles / (double)(rounds * slots);
        const double score = useful * fill * c.tile_efficiency;
        if (score > best_score + 1e-9) {
            best_score = score;
            best = idx;
        }
    }
    return best;
}

int launch_gemm(const void* kernel, int bm, int bn, int threads, int64_t M, int64_t N, int64_t K,
                const float* A, int64_t lda, int64_t strideA, const float* B, int64_t ldb,
                int64_t strideB, float* C, int64_t ldc, int64_t strideC, int64_t batch,
                hipStream_t stream) {
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
    if (per_matrix > kMaxGridX) return SGEMM_STATUS_SIZE_OVERFLOW;
    const int64_t per_launch = kMaxGridX / per_matrix;  // batch members per launch
    for (int64_t b0 = 0; b0 < batch; b0 += per_launch) {
        const int64_t nb = (batch - b0) < per_launch ? (batch - b0) : per_launch;
        GemmArgs p;
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
        default: return "unknown status";
    }
}

}  // extern "C"
