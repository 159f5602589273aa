// FP32 GEMM on the vector ALUs with per-lane register tiles, C = A x B,
// row-major, beta = 0.  This is the thread-tile design the pages describe,
// sized for wave64:
//  * 128 x 128 block tile, 256 threads (4 waves), each lane owns an 8 x 8
//    output tile: "Tiling Hierarchy on GPUs" ("Register Tiling": 8 A values
//    and 8 B values per k feed 64 FMAs; "Reducing Overhead Slots": a 128x128
//    block at 8x8 per thread takes 256 threads) and "Tiling Strategies"
//    section 4 ("Register Tiling": 128x128 block tile, 8x8 per thread).
//  * Register prefetching ("Tiling Hierarchy on GPUs", "Register
//    prefetching"): the LDS reads for step k+1 are issued before the FMAs of
//    step k, so each lane holds two operand sets.
//  * Double-buffered LDS slices with the next slice's global loads staged in
//    registers ("Tiling Strategies" section 3), zero-filled masked tails
//    ("CMU DLSys Lecture 12: GPU Acceleration" section 5).
//
// Layout: the outer product wants a column of A per k ("Outer Product"), so
// the A slice is transposed on its way into LDS, As[k][m] (pitch BM + 4, which
// spreads the transposing 4-byte writes of one half-wave over all banks); B is
// kept as Bs[k][n].  A lane's 8 rows are 4ty..4ty+3 and 64+4ty..64+4ty+3 and
// its 8 columns 4tx..4tx+3 and 64+4tx..64+4tx+3, so each k step is four
// ds_read_b128 from contiguous, conflict-free runs.
//
// The FMAs are plain FP32 v_fmac_f32, one multiply-add per lane per
// instruction: a wave64 instruction is 64 FMAs and takes a SIMD's issue
// quad-cycle.  gfx950 issues two VALU instructions from two waves in one
// quad-cycle (counted on the SIMD as a dual issue), so the bound is the full
// FP32 peak of 157.3 TFLOP/s, with every issue slot an FMA; at 8 x 8 per
// lane the operand reads and loop overhead keep this path near half of it
// (counters: about 84 % of quad-cycles issue VALU work, 30 % of them two
// instructions).  The matrix-core path is the fast one.
#pragma once

#include "tile_common.hpp"

namespace sgemm_dev {

struct ValuTile {
    static constexpr int BM = 128, BN = 128, BK = 8;
    static constexpr int NT = 256;
    static constexpr int GROUP_M = 8;
    static constexpr int LDA = BM + 4;  // LDS pitch of a transposed A row (one k)
    static constexpr int LDB = BN + 4;
    static constexpr int A_FLOATS = BK * LDA;
    static constexpr int B_FLOATS = BK * LDB;
};

__global__ __launch_bounds__(256) void sgemm_valu_kernel(GemmArgs p) {
    using T = ValuTile;
    __shared__ __attribute__((aligned(16))) float smem[2 * (T::A_FLOATS + T::B_FLOATS)];
    float* const As0 = smem;
    float* const Bs0 = smem + 2 * T::A_FLOATS;

    const TileCoord tc = map_block(p, T::GROUP_M);
    const int m0 = tc.tm * T::BM;
    const int n0 = tc.tn * T::BN;
    const float* const A = p.A + (int64_t)tc.b * p.strideA + (int64_t)m0 * p.lda;
    const float* const B = p.B + (int64_t)tc.b * p.strideB + n0;
    float* const C = p.C + (int64_t)tc.b * p.strideC + (int64_t)m0 * p.ldc + n0;
    const int rows_left = p.M - m0;
    const int cols_left = p.N - n0;
    const bool full_mn = rows_left >= T::BM && cols_left >= T::BN;

    const int tid = threadIdx.x;
    // A slice 128 x 8 = 256 quads: row tid/2, k quad tid%2.
    const int a_r = tid >> 1;
    const int a_kq = tid & 1;
    // B slice 8 x 128 = 256 quads: k row tid/32, n quad tid%32.
    const int b_k = tid >> 5;
    const int b_nq = tid & 31;

    f32x4 ra, rb;
    auto load_slice = [&](int k0) {
        if (full_mn && k0 + T::BK <= p.K) {
            ra = ldg4(A + (int64_t)a_r * p.lda + k0 + 4 * a_kq);
            rb = ldg4(B + (int64_t)(k0 + b_k) * p.ldb + 4 * b_nq);
        } else {
            ra = ldg4_masked(A + (int64_t)a_r * p.lda + k0 + 4 * a_kq,
                             a_r < rows_left ? p.K - (k0 + 4 * a_kq) : 0);
            rb = ldg4_masked(B + (int64_t)(k0 + b_k) * p.ldb + 4 * b_nq,
                             k0 + b_k < p.K ? cols_left - 4 * b_nq : 0);
        }
    };
    auto store_slice = [&](int buf) {
        float* const As = As0 + buf * T::A_FLOATS;
        float* const Bs = Bs0 + buf * T::B_FLOATS;
        As[(4 * a_kq + 0) * T::LDA + a_r] = ra.x;
        As[(4 * a_kq + 1) * T::LDA + a_r] = ra.y;
        As[(4 * a_kq + 2) * T::LDA + a_r] = ra.z;
        As[(4 * a_kq + 3) * T::LDA + a_r] = ra.w;
        *(f32x4*)(Bs + b_k * T::LDB + 4 * b_nq) = rb;
    };

    const int tx = tid & 15;
    const int ty = tid >> 4;
    float c[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) c[i][j] = 0.0f;

    auto read_operands = [&](const float* As, const float* Bs, int k, float (&a)[8],
                             float (&b)[8]) {
        const f32x4 a0 = *(const f32x4*)(As + k * T::LDA + 4 * ty);
        const f32x4 a1 = *(const f32x4*)(As + k * T::LDA + 64 + 4 * ty);
        const f32x4 b0 = *(const f32x4*)(Bs + k * T::LDB + 4 * tx);
        const f32x4 b1 = *(const f32x4*)(Bs + k * T::LDB + 64 + 4 * tx);
        a[0] = a0.x; a[1] = a0.y; a[2] = a0.z; a[3] = a0.w;
        a[4] = a1.x; a[5] = a1.y; a[6] = a1.z; a[7] = a1.w;
        b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w;
        b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
    };

    auto compute_slice = [&](int buf) {
        const float* const As = As0 + buf * T::A_FLOATS;
        const float* const Bs = Bs0 + buf * T::B_FLOATS;
        float a[2][8], b[2][8];
        read_operands(As, Bs, 0, a[0], b[0]);
#pragma unroll
        for (int k = 0; k < T::BK; ++k) {
            const int cur = k & 1;
            if (k + 1 < T::BK) read_operands(As, Bs, k + 1, a[cur ^ 1], b[cur ^ 1]);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) c[i][j] = __builtin_fmaf(a[cur][i], b[cur][j], c[i][j]);
        }
    };

    const int nslices = (p.K + T::BK - 1) / T::BK;
    if constexpr (kRaceCheck) {
        poison_lds(smem, 2 * (T::A_FLOATS + T::B_FLOATS), threadIdx.x, T::NT);
        __syncthreads();
    }
    load_slice(0);
    store_slice(0);
    __syncthreads();
    for (int s = 0; s < nslices; ++s) {
        const int cur = s & 1;
        const bool more = s + 1 < nslices;
        if (more) load_slice((s + 1) * T::BK);
        compute_slice(cur);
        if (more) store_slice(cur ^ 1);
        __syncthreads();
        if constexpr (kRaceCheck) {
            // Slice s is consumed: its buffers are refilled only after this.
            poison_lds(As0 + cur * T::A_FLOATS, T::A_FLOATS, threadIdx.x, T::NT);
            poison_lds(Bs0 + cur * T::B_FLOATS, T::B_FLOATS, threadIdx.x, T::NT);
            __syncthreads();
        }
    }

#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = (i < 4 ? 0 : 64) + 4 * ty + (i & 3);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int col = 64 * h + 4 * tx;
            const f32x4 v = {c[i][4 * h + 0], c[i][4 * h + 1], c[i][4 * h + 2], c[i][4 * h + 3]};
            float* const dst = C + (int64_t)row * p.ldc + col;
            if (full_mn)
                *(f32x4_u*)dst = (f32x4_u)v;
            else
                stg4_masked(dst, v, row < rows_left ? cols_left - col : 0);
        }
    }
}

}  // namespace sgemm_dev
