// FP32 GEMM on the gfx950 matrix cores: C = A x B, row-major, beta = 0.
//
// Structure (one workgroup per BM x BN output tile, loop over K in BK slices):
//  * Block tile and K-slice loop: "Tiling Strategies" section 2 ("The Tiled
//    Solution") and "CMU DLSys Lecture 12: GPU Acceleration" section 5 (a block
//    owns an output tile, stages two operand slabs per reduction stage,
//    cooperative strided copy q = tid, tid + nt, ...).
//  * Double buffering: "Tiling Strategies" section 3.  Two LDS buffers; the
//    global loads of slice s+1 are issued into registers before slice s is
//    computed and written to the other buffer while it is computed, so one
//    barrier per slice suffices.
//  * Register tiles: "Tiling Hierarchy on GPUs" ("Outer Product", "Register
//    Tiling").  The outer-product updates are done by the matrix core, one
//    MFMA instruction per MI x MI accumulator tile and k step:
//      MI = 32: v_mfma_f32_32x32x2_f32, 2 k per step, 16 accumulators per lane;
//      MI = 16: v_mfma_f32_16x16x4_f32, 4 k per step,  4 accumulators per lane.
//    The 64 lanes form 64/MI lane groups; lane (li, lg) supplies row li of the
//    A operand and column li of the B operand at the k held by group lg.  A
//    wave owns a WTM x WTN tile = TM x TN accumulator tiles.
//  * Tails: zero-filled masked loads and valid-only stores (Lecture 12,
//    section 5 schedule), never reading padding.
//
// LDS layouts (the "Warp Tiling" concern of "Tiling Hierarchy on GPUs": the
// lanes' LDS accesses must not collide in banks).  gfx950's LDS has 64 banks
// of 4 bytes; a ds_read_b128 / ds_write_b128 is served 16 lanes per pass (a
// pass is conflict-free when its 16 lanes hit 16 different 16-byte bank quads)
// and a ds_read_b32 32 lanes per pass.
//  * A slice kept as read from memory, As[m][k] (k contiguous), one row = BK
//    floats = BK/4 16-byte quads; 16/(BK/4) rows share one 256-byte bank row.
//    Quad kq of row r is stored at quad kq ^ ((r / rows_per_bank_row) % (BK/4)),
//    so the 16 consecutive rows one pass reads at the same logical quad land
//    in 16 different bank quads, and so do the 16 quads one pass writes.
//  * B slice kept as Bs[k][n] (n contiguous).  A 32-lane pass of ds_read_b32
//    covers 32/MI k rows, MI consecutive n each, and the compiler pairs the
//    reads of two column tiles into one ds_read2_b32 (8 bytes per lane, so
//    each k row then spans 2*MI banks).  With MI = 16 the row pitch BN + PADB
//    puts the two k rows of a pass 32 banks apart, so the pass touches 64
//    different banks; with MI = 32 a pass reads one row and needs no padding.
//
// Reduction order inside a slice: lane group lg takes k = lg*KPL + s at step
// s (KPL = BK*MI/64 k values per lane and slice), so each lane's A values for
// the slice are KPL consecutive floats read as 16-byte quads.  Every k of the
// slice meets every (i, j) exactly once; only the order of the FP32 additions
// differs from a plain k loop.
#pragma once

#include <type_traits>

#include "tile_common.hpp"

namespace sgemm_dev {

// The FP32 matrix instruction and its register layout.
template <int MI>
struct MfmaOp;

template <>
struct MfmaOp<32> {
    typedef f32x16 acc_t;
    static constexpr int ACC = 16;  // accumulators per lane
    static __device__ __forceinline__ acc_t mma(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    // Row inside the 32x32 tile of accumulator r held by lane group lg.
    static __device__ __forceinline__ int row(int r, int lg) {
        return 8 * (r / 4) + 4 * lg + (r % 4);
    }
};

template <>
struct MfmaOp<16> {
    typedef f32x4 acc_t;
    static constexpr int ACC = 4;
    static __device__ __forceinline__ acc_t mma(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int row(int r, int lg) { return 4 * lg + r; }
};

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int MI_, int OCC_, int GROUP_M_>
struct MfmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int MI = MI_;                       // MFMA tile edge (16 or 32)
    static constexpr int GROUP_M = GROUP_M_;
    static constexpr int OCC = OCC_;                     // waves per SIMD the registers allow
    static constexpr int NT = 64 * WAVES_M * WAVES_N;    // threads per workgroup
    static constexpr int WTM = BM / WAVES_M;             // wave tile rows
    static constexpr int WTN = BN / WAVES_N;             // wave tile columns
    static constexpr int TM = WTM / MI, TN = WTN / MI;   // MFMA tiles per wave
    static constexpr int LG = 64 / MI;                   // lane groups = k per MFMA
    static constexpr int KPL = BK / LG;                  // k values per lane per slice
    static constexpr int QPR = BK / 4;                   // 16-byte quads per A row
    static constexpr int A_VEC = BM * QPR / NT;          // A quads per thread per slice
    static constexpr int B_QPR = BN / 4;                 // 16-byte quads per B row
    static constexpr int B_VEC = BK * B_QPR / NT;        // B quads per thread per slice
    static constexpr int PADB = MI == 32 ? 0 : 32 / KPL; // see the B layout note
    static constexpr int LDB = BN + PADB;                // LDS pitch of a B row (floats)
    static constexpr int A_FLOATS = BM * BK;             // one A buffer
    static constexpr int B_FLOATS = BK * LDB;            // one B buffer
    static constexpr int RPB = 16 / QPR;                 // A rows per 256-byte bank row
    static constexpr int KG = 4;                         // k steps per operand group
    static constexpr int NKG = KPL / KG;                 // operand groups per slice
    static constexpr int HOLD = 2;                       // k steps issued after the barrier
    static constexpr int LDS_BYTES = 2 * (A_FLOATS + B_FLOATS) * 4;
    // Workgroups one CU can hold: by waves per SIMD (OCC, the launch bound)
    // and by the 160 KB of LDS.
    static constexpr int WG_PER_CU = (4 * OCC * 64 / NT) < (160 * 1024 / LDS_BYTES)
                                         ? (4 * OCC * 64 / NT) : (160 * 1024 / LDS_BYTES);

    static_assert(MI == 16 || MI == 32, "MFMA tile edge");
    static_assert(BK == 8 || BK == 16 || BK == 32, "BK must be 8, 16 or 32");
    static_assert(KPL % KG == 0, "a lane's k range must be whole 16-byte quads");
    static_assert(WTM % MI == 0 && WTN % MI == 0, "wave tile must be MFMA tile multiples");
    static_assert((BM * QPR) % NT == 0 && NT % QPR == 0, "A slice must split evenly");
    static_assert((BK * B_QPR) % NT == 0 && NT % B_QPR == 0, "B slice must split evenly");
    static_assert(BN % 64 == 0, "B rows must span whole bank rows");
    static_assert(MI == 32 || (KPL * LDB) % 64 == 32,
                  "B rows read in one pass must not share banks");
    static_assert(LDB % 4 == 0, "B rows must stay 16-byte aligned");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

    // Physical quad of logical quad `kq` in A row `r` is kq ^ swz(r).
    static __device__ __forceinline__ int swz(int r) { return (r / RPB) % QPR; }
};

template <class T>
__global__ __launch_bounds__(T::NT) __attribute__((amdgpu_waves_per_eu(T::OCC)))
void sgemm_mfma_kernel(GemmArgs p) {
    using Op = MfmaOp<T::MI>;
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
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // uniform per wave
    const int wy = wave / T::WAVES_N;
    const int wx = wave % T::WAVES_N;
    const int li = lane % T::MI;  // row of the A operand / column of the B operand
    const int lg = lane / T::MI;  // lane group: which k of the step

    typename Op::acc_t acc[T::TM][T::TN];
#pragma unroll
    for (int mi = 0; mi < T::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < T::TN; ++ni)
#pragma unroll
            for (int r = 0; r < Op::ACC; ++r) acc[mi][ni][r] = 0.0f;

    const int a_row = wy * T::WTM + li;  // + MI*mi
    const int a_swz = T::swz(a_row);     // MI*mi leaves the swizzle unchanged

    // One operand group = KG consecutive MFMA steps: one 16-byte quad of A per
    // row tile and KG values of B per column tile.  The operands of group g+1
    // are read from LDS before the MFMAs of group g are issued ("Tiling
    // Hierarchy on GPUs", "Register prefetching").
    const float* const Bl0 = Bs0 + (lg * T::KPL) * T::LDB + wx * T::WTN + li;
    auto read_group = [&](int buf, int g, f32x4 (&a)[T::TM], float (&b)[T::TN][T::KG]) {
        const float* const As = As0 + buf * T::A_FLOATS;
        const float* const Bl = Bl0 + buf * T::B_FLOATS + g * T::KG * T::LDB;
        const int quad = lg * (T::KPL / 4) + g;
#pragma unroll
        for (int mi = 0; mi < T::TM; ++mi)
            a[mi] = *(const f32x4*)(As + (a_row + T::MI * mi) * T::BK + ((quad ^ a_swz) << 2));
#pragma unroll
        for (int s = 0; s < T::KG; ++s)
#pragma unroll
            for (int ni = 0; ni < T::TN; ++ni) b[ni][s] = Bl[s * T::LDB + T::MI * ni];
    };

    auto mfma_steps = [&](const f32x4 (&a)[T::TM], const float (&b)[T::TN][T::KG], int s0,
                          int s1) {
#pragma unroll
        for (int s = s0; s < s1; ++s)
#pragma unroll
            for (int mi = 0; mi < T::TM; ++mi)
#pragma unroll
                for (int ni = 0; ni < T::TN; ++ni)
                    acc[mi][ni] = Op::mma(a[mi][s], b[ni][s], acc[mi][ni]);
    };

    // Operand registers, two groups' worth.  Group g of slice s uses set
    // (s*NKG + g) & 1; slices are processed in pairs so that the set index is
    // a compile-time constant.
    f32x4 opa[2][T::TM];
    float opb[2][T::TN][T::KG];
    const int nslices = (p.K + T::BK - 1) / T::BK;

    // One K slice held in LDS buffer `buf`.
    //  * The global loads of slice s+1 are issued first; their data is written
    //    to the other LDS buffer at the start of the slice's last operand group,
    //    so the writes complete under that group's MFMAs instead of stalling
    //    the wave right before the barrier.  That buffer was last read in slice
    //    s-1, and every wave finished those reads before the previous barrier.
    //  * The last HOLD k steps of the MFMAs are issued after the barrier that
    //    publishes slice s+1, behind the LDS reads of slice s+1's first operand
    //    group, so the matrix core keeps working while the waves synchronise and
    //    those reads are in flight.
    // SET0 is the operand set of the slice's first group (group g uses set
    // (SET0 + g) & 1, and the next slice starts on the set after the last).
    auto slice = [&](auto set0, int buf, int s) {
        constexpr int SET0 = decltype(set0)::value;
        const bool more = s + 1 < nslices;
        if (more) load_slice((s + 1) * T::BK);
#pragma unroll
        for (int g = 0; g < T::NKG; ++g) {
            const int set = (SET0 + g) & 1;
            if (g + 1 < T::NKG) {
                if (set == 0)
                    read_group(buf, g + 1, opa[1], opb[1]);
                else
                    read_group(buf, g + 1, opa[0], opb[0]);
            }
            if (T::NKG > 1 && g + 1 == T::NKG && more) store_slice(buf ^ 1);
            __builtin_amdgcn_sched_barrier(0);
            const int s1 = g + 1 < T::NKG ? T::KG : T::KG - T::HOLD;
            if (set == 0)
                mfma_steps(opa[0], opb[0], 0, s1);
            else
                mfma_steps(opa[1], opb[1], 0, s1);
            __builtin_amdgcn_sched_barrier(0);
        }
        constexpr int LAST = (SET0 + T::NKG - 1) & 1;
        if (more) {
            if (T::NKG == 1) store_slice(buf ^ 1);
            __syncthreads();
            if constexpr (kRaceCheck) {
                // Slice s is consumed: its buffers are refilled only after this.
                poison_lds(As0 + buf * T::A_FLOATS, T::A_FLOATS, threadIdx.x, T::NT);
                poison_lds(Bs0 + buf * T::B_FLOATS, T::B_FLOATS, threadIdx.x, T::NT);
                __syncthreads();
            }
            read_group(buf ^ 1, 0, opa[LAST ^ 1], opb[LAST ^ 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_steps(opa[LAST], opb[LAST], T::KG - T::HOLD, T::KG);
        __builtin_amdgcn_sched_barrier(0);
    };

    if constexpr (kRaceCheck) {
        poison_lds(smem, 2 * (T::A_FLOATS + T::B_FLOATS), threadIdx.x, T::NT);
        __syncthreads();
    }
    load_slice(0);
    store_slice(0);
    __syncthreads();
    read_group(0, 0, opa[0], opb[0]);
    if constexpr (T::NKG % 2 == 0) {
        // Every slice starts on operand set 0.
        for (int s = 0; s < nslices; ++s) slice(std::integral_constant<int, 0>(), s & 1, s);
    } else {
        // Odd group count: consecutive slices start on alternating sets.
        for (int s = 0; s < nslices; s += 2) {
            slice(std::integral_constant<int, 0>(), 0, s);
            if (s + 1 < nslices) slice(std::integral_constant<int, 1>(), 1, s + 1);
        }
    }

    // Epilogue: accumulator r of lane (li, lg) in MFMA tile (mi, ni) is row
    // Op::row(r, lg) and column li of that tile.
#pragma unroll
    for (int mi = 0; mi < T::TM; ++mi) {
#pragma unroll
        for (int ni = 0; ni < T::TN; ++ni) {
            const int col = wx * T::WTN + T::MI * ni + li;
#pragma unroll
            for (int r = 0; r < Op::ACC; ++r) {
                const int row = wy * T::WTM + T::MI * mi + Op::row(r, lg);
                if (full_mn || (row < rows_left && col < cols_left))
                    C[(int64_t)row * p.ldc + col] = acc[mi][ni][r];
            }
        }
    }
}

}  // namespace sgemm_dev
