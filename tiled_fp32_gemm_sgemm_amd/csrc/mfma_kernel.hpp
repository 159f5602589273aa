// FP32 GEMM on the gfx950 matrix cores: C = A x B, row-major, beta = 0.
//
// Structure (one workgroup per BM x BN output tile, loop over K in BK slices):
//  * Block tile and K-slice loop: "Tiling Strategies" section 2 ("The Tiled
//    Solution") and "CMU DLSys Lecture 12: GPU Acceleration" section 5 (a block
//    owns an output tile, stages two operand slabs per reduction stage,
//    cooperative strided copy q = tid, tid + nt, ...).
//  * Double buffering: "Tiling Strategies" section 3.  Two LDS buffers; the
//    global loads of slice s+1 are issued into registers before slice s is
//    computed and written to the other buffer afterwards, so one barrier per
//    slice suffices.
//  * Register tiles: "Tiling Hierarchy on GPUs" ("Outer Product", "Register
//    Tiling").  Here the outer product of one k step is done by the matrix
//    core: v_mfma_f32_32x32x2_f32 adds a 32x2 by 2x32 product to a 32x32 FP32
//    accumulator tile held across the 64 lanes (16 values per lane).  A wave
//    owns a WTM x WTN tile = TM x TN such accumulator tiles.
//  * Tails: zero-filled masked loads and valid-only stores (Lecture 12,
//    section 5 schedule), never reading padding.
//
// LDS layouts (the "Warp Tiling" concern of "Tiling Hierarchy on GPUs": the
// lanes' LDS reads must not collide in banks):
//  * A slice kept as read from memory, As[m][k] (k contiguous), one row = BK
//    floats = BK/4 16-byte quads, quads XOR-swizzled by row.  Each lane reads
//    its own k values with ds_read_b128; the eight rows read together by one
//    8-lane group land in eight different quad columns.
//  * B slice kept as Bs[k][n] with a row pitch of BN + 4 floats; 32 lanes read
//    32 consecutive n of one k row (ds_read_b32), so they hit 32 banks.
//
// Reduction order inside a slice: the MFMA reduces over a k pair held by the
// two lane halves (lanes 0-31 and 32-63).  Lane half h takes k = h*BK/2 + s at
// step s, so each lane's A values for the slice are BK/2 consecutive floats.
// Every k of the slice still meets every (i, j) exactly once; only the order
// of the FP32 additions differs from a plain k loop.
#pragma once

#include "tile_common.hpp"

namespace sgemm_dev {

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int GROUP_M_>
struct MfmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int GROUP_M = GROUP_M_;
    static constexpr int NT = 64 * WAVES_M * WAVES_N;   // threads per workgroup
    static constexpr int WTM = BM / WAVES_M;            // wave tile rows
    static constexpr int WTN = BN / WAVES_N;            // wave tile columns
    static constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA tiles per wave
    static constexpr int QPR = BK / 4;                  // 16-byte quads per A row
    static constexpr int KH = BK / 2;                   // k values per lane half
    static constexpr int A_VEC = BM * QPR / NT;         // A quads per thread per slice
    static constexpr int B_QPR = BN / 4;                // 16-byte quads per B row
    static constexpr int B_VEC = BK * B_QPR / NT;       // B quads per thread per slice
    static constexpr int LDB = BN + 4;                  // LDS pitch of a B row (floats)
    static constexpr int A_FLOATS = BM * BK;            // one A buffer
    static constexpr int B_FLOATS = BK * LDB;           // one B buffer
    static constexpr int RPB = QPR >= 8 ? 1 : 8 / QPR;  // A rows per 128-byte bank row
    static constexpr int LDS_BYTES = 2 * (A_FLOATS + B_FLOATS) * 4;

    static_assert(BK == 8 || BK == 16 || BK == 32, "BK must be 8, 16 or 32");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32x32 multiples");
    static_assert((BM * QPR) % NT == 0 && NT % QPR == 0, "A slice must split evenly");
    static_assert((BK * B_QPR) % NT == 0 && NT % B_QPR == 0, "B slice must split evenly");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

    // Physical quad of logical quad `kq` in A row `r`.
    static __device__ __forceinline__ int swz(int r) { return (r / RPB) % QPR; }
};

template <class T>
__global__ __launch_bounds__(T::NT) void sgemm_mfma_kernel(GemmArgs p) {
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

    // Cooperative copy: thread tid moves quads q = tid + v*NT of each slab.
    const int a_kq = tid % T::QPR;
    const int a_r0 = tid / T::QPR;
    constexpr int A_RSTEP = T::NT / T::QPR;
    const int b_nq = tid % T::B_QPR;
    const int b_k0 = tid / T::B_QPR;
    constexpr int B_KSTEP = T::NT / T::B_QPR;

    f32x4 ra[T::A_VEC];
    f32x4 rb[T::B_VEC];

    auto load_slice = [&](int k0) {
        if (full_mn && k0 + T::BK <= p.K) {
#pragma unroll
            for (int v = 0; v < T::A_VEC; ++v)
                ra[v] = ldg4(A + (int64_t)(a_r0 + v * A_RSTEP) * p.lda + k0 + 4 * a_kq);
#pragma unroll
            for (int v = 0; v < T::B_VEC; ++v)
                rb[v] = ldg4(B + (int64_t)(k0 + b_k0 + v * B_KSTEP) * p.ldb + 4 * b_nq);
        } else {
            const int kvalid = p.K - (k0 + 4 * a_kq);
#pragma unroll
            for (int v = 0; v < T::A_VEC; ++v) {
                const int r = a_r0 + v * A_RSTEP;
                ra[v] = ldg4_masked(A + (int64_t)r * p.lda + k0 + 4 * a_kq,
                                    r < rows_left ? kvalid : 0);
            }
            const int nvalid = cols_left - 4 * b_nq;
#pragma unroll
            for (int v = 0; v < T::B_VEC; ++v) {
                const int k = k0 + b_k0 + v * B_KSTEP;
                rb[v] = ldg4_masked(B + (int64_t)k * p.ldb + 4 * b_nq, k < p.K ? nvalid : 0);
            }
        }
    };

    auto store_slice = [&](int buf) {
        float* const As = As0 + buf * T::A_FLOATS;
        float* const Bs = Bs0 + buf * T::B_FLOATS;
#pragma unroll
        for (int v = 0; v < T::A_VEC; ++v) {
            const int r = a_r0 + v * A_RSTEP;
            *(f32x4*)(As + r * T::BK + ((a_kq ^ T::swz(r)) << 2)) = ra[v];
        }
#pragma unroll
        for (int v = 0; v < T::B_VEC; ++v)
            *(f32x4*)(Bs + (b_k0 + v * B_KSTEP) * T::LDB + 4 * b_nq) = rb[v];
    };

    const int lane = tid % 64;
    const int wave = tid / 64;
    const int wy = wave / T::WAVES_N;
    const int wx = wave % T::WAVES_N;
    const int li = lane % 32;  // row of the A operand / column of the B operand
    const int lh = lane / 32;  // which k of the pair

    f32x16 acc[T::TM][T::TN];
#pragma unroll
    for (int mi = 0; mi < T::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < T::TN; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

    const int a_row = wy * T::WTM + li;  // + 32*mi
    const int a_swz = T::swz(a_row);     // 32*mi leaves the swizzle unchanged

    auto compute_slice = [&](int buf) {
        const float* const As = As0 + buf * T::A_FLOATS;
        const float* const Bs = Bs0 + buf * T::B_FLOATS;
        float a_op[T::TM][T::KH];
#pragma unroll
        for (int mi = 0; mi < T::TM; ++mi) {
#pragma unroll
            for (int qq = 0; qq < T::QPR / 2; ++qq) {
                const int quad = lh * (T::QPR / 2) + qq;
                const f32x4 v =
                    *(const f32x4*)(As + (a_row + 32 * mi) * T::BK + ((quad ^ a_swz) << 2));
                a_op[mi][4 * qq + 0] = v.x;
                a_op[mi][4 * qq + 1] = v.y;
                a_op[mi][4 * qq + 2] = v.z;
                a_op[mi][4 * qq + 3] = v.w;
            }
        }
        const float* const Bl = Bs + (lh * T::KH) * T::LDB + wx * T::WTN + li;
#pragma unroll
        for (int s = 0; s < T::KH; ++s) {
            float b_op[T::TN];
#pragma unroll
            for (int ni = 0; ni < T::TN; ++ni) b_op[ni] = Bl[s * T::LDB + 32 * ni];
#pragma unroll
            for (int mi = 0; mi < T::TM; ++mi)
#pragma unroll
                for (int ni = 0; ni < T::TN; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(a_op[mi][s], b_op[ni],
                                                                       acc[mi][ni], 0, 0, 0);
        }
    };

    const int nslices = (p.K + T::BK - 1) / T::BK;
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
    }

    // Epilogue.  Accumulator register r of lane (li, lh) in MFMA tile (mi, ni)
    // holds row 8*(r/4) + 4*lh + r%4 and column li of that 32x32 tile.
#pragma unroll
    for (int mi = 0; mi < T::TM; ++mi) {
#pragma unroll
        for (int ni = 0; ni < T::TN; ++ni) {
            const int col = wx * T::WTN + 32 * ni + li;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wy * T::WTM + 32 * mi + 8 * (r / 4) + 4 * lh + (r % 4);
                if (full_mn || (row < rows_left && col < cols_left))
                    C[(int64_t)row * p.ldc + col] = acc[mi][ni][r];
            }
        }
    }
}

}  // namespace sgemm_dev
