// FP32 GEMM on the gfx950 matrix cores with direct global->LDS staging.
//
// Same product, tiling, register tiles and reduction order as mfma_kernel.hpp
// (C = A x B, row-major, beta = 0; one workgroup per BM x BN tile; K in BK
// slices; "Tiling Strategies" sections 2-3, "CMU DLSys Lecture 12: GPU
// Acceleration" section 5, "Tiling Hierarchy on GPUs" "Register Tiling" and
// "Register prefetching"), with a different global->LDS loader:
//
//  * Each slice is copied by buffer_load_dwordx4 ... lds: one instruction moves
//    64 lanes x 16 bytes from global memory straight into a contiguous 1 KB
//    chunk of LDS (lane L fills bytes 16L..16L+15), with no VGPR staging and
//    no ds_write.  On gfx950 a vector-memory or LDS-write instruction issued
//    between MFMAs costs matrix-core cycles, so this halves the instructions
//    that feed the matrix core.
//  * The layout in LDS is fixed by lane order, so each lane's global source
//    is chosen to realise the bank-conflict-free layouts: lane L of chunk c
//    fills physical quad q = 64c + L; its source is the logical quad that the
//    swizzle maps there.  Per-lane source offsets are computed once per block
//    and stay in VGPRs; the per-slice advance lives in the scalar buffer
//    descriptor, and the wave index is made wave-uniform so that every LDS
//    destination (M0) is computed on the scalar unit: the loop spends no VALU
//    instructions on the copies.
//  * Masking: a quad that lies wholly outside the matrix gets an offset past
//    the descriptor's range, and the buffer unit writes zeros for it (the
//    zero-filled masked load of Lecture 12 section 5).  Slices with quads that
//    straddle an edge (the last slice when BK does not divide K, or N not a
//    multiple of 4) are copied with masked loads through registers.
//
// LDS layouts.  gfx950 serves ds_read_b128 16 lanes per pass over 64 banks of
// 4 bytes, and ds_read_b32 32 lanes per pass over 32 banks (measured):
//  * A slice As[m][k], BK floats per row, quad kq of row r stored at
//    kq ^ ((r / rows_per_256_bytes) % (BK/4)) (as in mfma_kernel.hpp): the 16
//    rows of a b128 pass hit 16 distinct quads of the bank row.  With BK = 128
//    (512-byte rows) the flip is kq ^ (r % 16), inside each 16-quad half.
//  * B slice Bs[k][n], BN floats per row, unpadded.  The output columns are
//    interleaved over a wave's column tiles (DlTile::bcol): lane li of column
//    tile ni owns column li * BV + ni % BV of each BV-tile run, so the BV
//    values a lane needs at one k are adjacent and come in one ds_read_b64
//    (BV = 2) or ds_read_b128 (BV = 4), and a pass reads one contiguous run of
//    a k row, all 64 banks once.  Against one ds_read_b32 per column tile
//    (BV = 1, same banks) this halves the B read instructions and lets the
//    epilogue store BV adjacent outputs per lane at once: 1.8 % faster at
//    4096^3 (same-process A/B).  With MI = 16 and BV = 1 a ds_read_b32 pass
//    covers two lane groups from rows KPL apart; those rows are stored with
//    their quads flipped by 4 (16 floats) so the halves use disjoint banks.
//  * SWIZZLE = false stores A unswizzled: a control build whose A reads
//    conflict, used to show that the bank-conflict counter sees the layout.
#pragma once

#include <type_traits>

#include "mfma_kernel.hpp"
#include "tile_common.hpp"

namespace sgemm_dev {

typedef __attribute__((address_space(3))) void lds_void_t;

// Byte offset that is outside every descriptor range used here: the buffer
// unit returns zeros for it.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Four floats held as one operand group: an f32x4 for operands read as
// 16-byte quads, this for operands read one float per k step.
struct F4 {
    float v[4];
    __device__ __forceinline__ float& operator[](int i) { return v[i]; }
    __device__ __forceinline__ const float& operator[](int i) const { return v[i]; }
};

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int MI_, int OCC_, int GROUP_M_,
          int STAGES_ = 2, int KSPLIT_ = 1, bool SWIZZLE_ = true, bool TA_ = false,
          bool TB_ = false, bool EX_ = false, bool BIL_ = true, bool CONV_ = false,
          int SCHED_ = 1, bool SK_ = false>
struct DlTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int MI = MI_;
    static constexpr int OCC = OCC_;
    static constexpr int GROUP_M = GROUP_M_;
    static constexpr int STAGES = STAGES_;               // LDS slice buffers in flight
    static constexpr int KSPLIT = KSPLIT_;               // wave groups splitting each slice's k
    static constexpr bool SWIZZLE = SWIZZLE_;
    // Stored layouts: A is M x K (TA = false) or K x M (TA = true, op(A) = A^T);
    // B is K x N (TB = false) or N x K (TB = true).  An operand whose k runs
    // along its stored rows ("k-contiguous": A with TA = false, B with TB =
    // true) is staged as [mn][k] and read as swizzled 16-byte quads; the other
    // kind is staged as [k][mn] and read one float per k step.
    static constexpr bool TA = TA_, TB = TB_;
    static constexpr bool A_KC = !TA, B_KC = TB;
    static constexpr bool EX = EX_;                      // alpha/beta epilogue
    // CONV: A is the implicit im2col matrix of an NHWC image (GemmArgs::conv):
    // row m = output position (n, p, q), k = (r, s, c); B holds KRSC filters,
    // stored N x K.
    static constexpr bool CONV = CONV_;
    static constexpr int NWMN = WAVES_M * WAVES_N;       // waves per k group
    static constexpr int NW = NWMN * KSPLIT;             // waves per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int KSUB = BK / KSPLIT;             // k values of a slice per k group
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int TM = WTM / MI, TN = WTN / MI;
    static constexpr int LG = 64 / MI;
    static constexpr int KPL = KSUB / LG;
    static constexpr int QPR = BK / 4;                   // quads per k-contiguous LDS row
    static constexpr int A_QPR = A_KC ? BK / 4 : BM / 4; // quads per LDS row of A
    static constexpr int B_QPR = B_KC ? BK / 4 : BN / 4; // quads per LDS row of B
    static constexpr int LDA_S = BM;                     // LDS row length of A staged [k][m]
    static constexpr int LDB = BN;                       // LDS row length of B staged [k][n]
    static constexpr int A_FLOATS = BM * BK;
    static constexpr int B_FLOATS = BK * BN;
    static constexpr int BUF_FLOATS = A_FLOATS + B_FLOATS;
    static constexpr int RPB = QPR >= 16 ? 1 : 16 / QPR;  // stored rows per 256 bytes
    static constexpr int KG = 4;
    static constexpr int NKG = KPL / KG;
    static constexpr int HOLD = 2;                       // k steps issued after the barrier
    static constexpr int A_CH = BM * BK / 256;           // 1 KB chunks per A slice
    static constexpr int B_CH = BK * BN / 256;           // 1 KB chunks per B slice
    static constexpr int A_CHW = A_CH / NW;              // chunks per wave
    static constexpr int B_CHW = B_CH / NW;
    // Column interleave of a B operand staged [k][n] (BIL): lane li of column
    // tile ni owns output column (ni / BV) * MI * BV + li * BV + ni % BV of the
    // wave tile, so the BV values a lane needs at one k are adjacent in LDS and
    // come in one ds_read_b64 / ds_read_b128, and the lane's outputs in one row
    // are BV adjacent columns (one vector store).  Each k row of a pass is then
    // read as one contiguous run: 32 lanes x 8 bytes or 16 lanes x 16 bytes,
    // all 64 banks once.  With MI = 16 only BV = 4 keeps a pass inside one k
    // row; other widths keep BV = 1 and the row flip below.
    // A B operand staged [n][k] (stored N x K) takes the same interleave for
    // its stores: its quad reads stay at rows MI * ni + li, and the copies
    // place logical column bcol(ni, li) there (bkc_row).
    static constexpr bool BIL = BIL_;
    // Slice schedule (see the kernel body):
    //   SCHED = 0: the next operand group's LDS reads go out at once, before
    //              the current group's MFMAs; the slice copies in one burst;
    //   SCHED = 1: the reads go out a part at a time, one after each k step of
    //              the current group's MFMAs; the copies in one burst;
    //   SCHED = 2: as 1, and the copies one after each k step from the start
    //              of the slice (a convolution keeps the burst: its copy
    //              offsets are rebuilt per filter tap).
    static constexpr int SCHED = SCHED_;
    // Split-K (SK): the workgroups of one output tile each reduce a k range
    // and join through a workspace (see the end of the kernel body).
    static constexpr bool SK = SK_;
    static constexpr bool ILV = SCHED >= 1;
    static constexpr bool SPREAD_COPIES = SCHED >= 2 && !CONV_;
    static constexpr int BV = !BIL ? 1
                              : MI == 16 ? (TN % 4 == 0 ? 4 : 1)
                                         : (TN % 4 == 0 ? 4 : TN % 2 == 0 ? 2 : 1);
    // The same interleave for an A operand staged [k][m] (A^T stored): lane
    // li of row tile mi supplies wave-tile row (mi / AV) * MI * AV + li * AV +
    // mi % AV, so the AV values of A a lane needs at one k are adjacent and
    // come in one ds_read_b64 / ds_read_b128 (a pass again reads one
    // contiguous run of a k row), and the output rows of the AV tiles
    // interleave the same way.
    static constexpr int AV = (A_KC || !BIL) ? 1
                              : MI == 16 ? (TM % 4 == 0 ? 4 : 1)
                                         : (TM % 4 == 0 ? 4 : TM % 2 == 0 ? 2 : 1);
    // Quad flip on odd lane-group row blocks of an operand staged [k][mn].
    static constexpr int AFLIP = (MI == 16 && AV == 1) ? 4 : 0;
    static constexpr int BFLIP = (MI == 16 && BV == 1) ? 4 : 0;
    // Register-staged fallback: quads per thread per slice.
    static constexpr int A_VEC = BM * BK / 4 / NT;
    static constexpr int B_VEC = BK * BN / 4 / NT;
    static constexpr int LDS_BYTES = STAGES * BUF_FLOATS * 4;
    static constexpr int LPS = A_CHW + B_CHW;            // copy instructions per wave per slice
    // Workgroups one CU can hold: by waves per SIMD (OCC, the launch bound)
    // and by the 160 KB of LDS.
    static constexpr int WG_PER_CU = (4 * OCC * 64 / NT) < (160 * 1024 / LDS_BYTES)
                                         ? (4 * OCC * 64 / NT) : (160 * 1024 / LDS_BYTES);
    // Spread copies issued from a main loop specialised for whole direct
    // slices: buffer descriptors built once per slice, no branch per copy.
    // Taken by tiles that run one workgroup per CU (512 x 4096 x 4096: 123.0
    // -> 120.5 us; 1024^3 19.5 -> 19.15; 2048^3 121.5 -> 119.7).  Tiles that
    // share a CU between several workgroups keep the branch per copy: with
    // the copies issued back to back after the k steps they ran 4-15 % slower
    // (batched 1024 x 128^3 39.6 -> 41.0 us, 8192^2 x 128 134 -> 155), and
    // no placement of them inside the slice recovered it on every shape.
    static constexpr bool HOIST_SPREAD = SPREAD_COPIES && WG_PER_CU == 1;

    static_assert(MI == 16 || MI == 32, "MFMA tile edge");
    static_assert(BK == 16 || BK == 32 || BK == 64 || BK == 128, "BK must be 16, 32, 64 or 128");
    static_assert(KPL % KG == 0 && NKG % 2 == 0, "whole, even number of A operand groups");
    static_assert(WTM % MI == 0 && WTN % MI == 0, "wave tile must be MFMA tile multiples");
    static_assert(A_CH % NW == 0 && B_CH % NW == 0, "slice chunks must split over the waves");
    static_assert(BN % 32 == 0 && BM % 32 == 0, "[k][mn] rows must start on bank 0");
    static_assert(STAGES >= 2 && LPS * (STAGES - 2) <= 63, "vmcnt holds at most 63");
    static_assert((BM * BK / 4) % NT == 0 && (BK * BN / 4) % NT == 0, "fallback copy must split");
    static_assert(MI == 32 || (BN >= 32 && BM >= 32), "the flip needs 32-float rows");
    static_assert(TN % BV == 0, "whole vectors of column tiles");
    static_assert(TM % AV == 0, "whole vectors of row tiles");
    static_assert(!CONV || (A_KC && B_KC && !EX), "convolution: k-contiguous A and B, beta = 0");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(SCHED >= 0 && SCHED <= 2, "slice schedule");
    static_assert(SCHED < 2 || LPS <= NKG * KG - HOLD, "one copy per k step fits in a slice");
    static_assert((KSPLIT - 1) * BM * BN <= STAGES * BUF_FLOATS, "k-group exchange fits in LDS");
    static_assert(!SK || !CONV || (A_KC && B_KC && !EX),
                  "split-K convolution: k-contiguous operands, beta = 0");
    static_assert(!SK || WTM * WTN <= 64 * 64, "split-K join holds one wave tile of sums");

    // Quad swizzle of k-contiguous row r.  Rows of at most 256 bytes: the 16
    // rows of a b128 pass fill one 256-byte bank row each, so each takes a
    // different quad of it.  Rows of 512 bytes (BK = 128): quads are flipped
    // within their half by r % 16, so the 16 rows of a pass again cover all
    // 16 quads of a 256-byte span.
    static __device__ __forceinline__ int swz(int r) {
        return SWIZZLE ? (QPR >= 16 ? r % 16 : (r / RPB) % QPR) : 0;
    }
    // Physical quad of logical quad q in row k of an operand staged [k][mn] is
    // q ^ flip(k).
    static __device__ __forceinline__ int flipA(int k) { return ((k / KPL) & 1) * AFLIP; }
    static __device__ __forceinline__ int flipB(int k) { return ((k / KPL) & 1) * BFLIP; }
    // Wave-tile column of lane li in column tile ni (see BIL).
    static __device__ __forceinline__ int bcol(int ni, int li) {
        return (ni / BV) * MI * BV + li * BV + ni % BV;
    }
    // Logical column held by row `slot` of a B operand staged [n][k]: within
    // each run of MI * BV rows, row MI * c + l holds column l * BV + c (so the
    // rows MI * ni + li that tile ni reads hold the columns bcol(ni, li)).
    static __device__ __forceinline__ int bkc_row(int slot) {
        if constexpr (BV == 1) {
            return slot;
        } else {
            const int run = slot / (MI * BV), s = slot % (MI * BV);
            return run * MI * BV + (s % MI) * BV + s / MI;
        }
    }
    // Wave-tile row of row i (the lane that supplies it) in row tile mi (see AV).
    static __device__ __forceinline__ int arow(int mi, int i) {
        return (mi / AV) * MI * AV + i * AV + mi % AV;
    }
    using AReg = std::conditional_t<A_KC, f32x4, F4>;
    using BReg = std::conditional_t<B_KC, f32x4, F4>;
};

// A 64-bit value that is the same in every lane, moved to scalar registers
// (free when it already is scalar).
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Waits until at most N vector-memory operations of this wave are still
// outstanding; the export and LDS counters are left alone.  (s_waitcnt
// immediate: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Waits until at most LPS * min(d, MAXD) operations are outstanding: the
// copies of the d slices issued after the one that must have landed.
template <int LPS, int MAXD>
__device__ __forceinline__ void wait_slices_after(int d) {
    if constexpr (MAXD == 0) {
        wait_vmcnt<0>();
    } else {
        if (d >= MAXD)
            wait_vmcnt<LPS * MAXD>();
        else
            wait_slices_after<LPS, MAXD - 1>(d);
    }
}

// Workgroup barrier that leaves the direct copies of later slices in flight.
// __syncthreads() (and any release fence that covers LDS) waits for every
// outstanding vector-memory operation of the wave, because the direct copies
// count as pending LDS writes; here the caller waits for the copies it needs
// with wait_vmcnt, this waits for the wave's own LDS accesses (lgkmcnt 0).
// The empty asm statements with a memory clobber keep the compiler from
// moving memory accesses across (they emit nothing), and the scheduling
// barriers keep the machine scheduler from moving any instruction across.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((15 << 0) | (3 << 14) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// f(std::integral_constant<int, g>()) for the runtime value g in [G, N): a
// wave-uniform index turned into a compile-time one, so that register
// arrays are indexed with constants.
template <int G, int N, class F>
__device__ __forceinline__ void for_group(int g, F&& f) {
    if constexpr (G < N) {
        if (g == G)
            f(std::integral_constant<int, G>());
        else
            for_group<G + 1, N>(g, f);
    }
}

// The kernel body lives in a device function: it uses device-only builtins
// and types, and keeping them out of the __global__ function's own body lets
// the host compilation pass emit the launch stub.
template <class T>
__device__ __forceinline__ void sgemm_mfma_dl_body(const GemmArgs& p) {
    using Op = MfmaOp<T::MI>;
    __shared__ __attribute__((aligned(16))) float smem[T::STAGES * T::BUF_FLOATS];

    // Split-K: the tile, the chunk (tc.b) and whether the tile is split.
    TileCoord tc;
    int sk_tail = 0;
    bool sk_full = false;
    if constexpr (T::SK) {
        const SplitCoord sc = map_split_block(p, T::GROUP_M);
        tc = sc.tc;
        sk_tail = sc.tail;
        sk_full = sc.full;
    } else {
        tc = map_block(p, T::GROUP_M);
    }
    const int m0 = tc.tm * T::BM;
    const int n0 = tc.tn * T::BN;
    // Tile origin in each stored operand (element offsets); k advances along
    // rows (k-contiguous) or down rows.  The offsets are wave-uniform; saying
    // so keeps them, and the buffer descriptors built from them, in SGPRs.
    const int64_t a_org = T::CONV ? 0
                                  : uniform_i64((int64_t)tc.b * p.strideA +
                                                (T::A_KC ? (int64_t)m0 * p.lda : (int64_t)m0));
    const int64_t b_org = uniform_i64((int64_t)tc.b * p.strideB +
                                      (T::B_KC ? (int64_t)n0 * p.ldb : (int64_t)n0));
    const float* const A = p.A + a_org;
    const float* const B = p.B + b_org;
    float* const C = p.C + (int64_t)tc.b * p.strideC + (int64_t)m0 * p.ldc + n0;
    const int rows_left = p.M - m0;
    const int cols_left = p.N - n0;
    const bool full_mn = rows_left >= T::BM && cols_left >= T::BN;
    // The k range this workgroup reduces: all of K, or one split's part,
    // which starts at kbeg (the operand pointers above are already moved
    // there; only the convolution's gather works in absolute k).
    const int Kd = T::SK && !sk_full ? min(p.kchunk, p.K - tc.b * p.kchunk) : p.K;
    const int kbeg = T::SK ? tc.b * p.kchunk : 0;
    const int nslices = (Kd + T::BK - 1) / T::BK;

    const int tid = threadIdx.x;
    const int lane = tid % 64;
    // The wave index is uniform across the wave; saying so keeps every
    // per-wave address (LDS chunk bases for M0 in particular) in SGPRs.
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);

    // ---------------------------------------------------------------- loader
    // A k-contiguous slice for k0 is a descriptor over BM stored rows from
    // column k0; an [k][mn] one is a descriptor over BK stored rows from row k0.
    const int64_t a_span64 = T::A_KC ? (int64_t)(T::BM - 1) * p.lda + T::BK
                                     : (int64_t)(T::BK - 1) * p.lda + T::BM;
    const int64_t b_span64 = T::B_KC ? (int64_t)(T::BN - 1) * p.ldb + T::BK
                                     : (int64_t)(T::BK - 1) * p.ldb + T::BN;
    const uint32_t a_span = (uint32_t)(a_span64 * 4);
    const uint32_t b_span = (uint32_t)(b_span64 * 4);

    uint32_t a_off[T::A_CHW];
    uint32_t b_off[T::B_CHW];
    // Per-lane source offsets of this wave's chunks, fixed for the block;
    // quads outside the matrix point out of range and load as zeros.
    auto make_offsets = [&](int kleft) {
#pragma unroll
        for (int j = 0; j < T::A_CHW && !T::CONV; ++j) {
            const int q = 64 * (wave * T::A_CHW + j) + lane;
            const int r = q / T::A_QPR;
            if constexpr (T::A_KC) {
                const int kq = (q % T::A_QPR) ^ T::swz(r);
                const bool ok = r < rows_left && 4 * kq < kleft;
                a_off[j] = ok ? (uint32_t)(((int64_t)r * p.lda + 4 * kq) * 4) : kOutOfRange;
            } else {
                const int mq = (q % T::A_QPR) ^ T::flipA(r);
                const bool ok = r < kleft && 4 * mq < rows_left;
                a_off[j] = ok ? (uint32_t)(((int64_t)r * p.lda + 4 * mq) * 4) : kOutOfRange;
            }
        }
#pragma unroll
        for (int j = 0; j < T::B_CHW; ++j) {
            const int q = 64 * (wave * T::B_CHW + j) + lane;
            const int r = q / T::B_QPR;
            if constexpr (T::B_KC) {
                const int kq = (q % T::B_QPR) ^ T::swz(r);
                const int n = T::bkc_row(r);
                const bool ok = n < cols_left && 4 * kq < kleft;
                b_off[j] = ok ? (uint32_t)(((int64_t)n * p.ldb + 4 * kq) * 4) : kOutOfRange;
            } else {
                const int nq = (q % T::B_QPR) ^ T::flipB(r);
                const bool ok = r < kleft && 4 * nq < cols_left;
                b_off[j] = ok ? (uint32_t)(((int64_t)r * p.ldb + 4 * nq) * 4) : kOutOfRange;
            }
        }
    };

    // Convolution gather ("Tiling Strategies" section 5: input patches are the
    // tiled operand).  Each of this wave's A chunks fills one row m of the tile
    // at logical quad kq of the slice; the row's output position (n, p, q) is
    // decoded once per block.  A slice lies inside one filter tap (r, s) when
    // C is a multiple of BK, so its quads are c0 + 4 kq .. + 3 of the input
    // pixel (p sh - ph + r dh, q sw - pw + s dw): per-lane offsets for c0 = 0
    // are rebuilt when a slice starts a new tap, and c0 goes into the
    // descriptor base.  Pixels outside the image get an out-of-range offset
    // and load as zeros (the zero padding).  The descriptor starts at the
    // first image the tile's rows fall in and ends after the last one, so the
    // byte offsets only have to span those images, not the whole input.
    const ConvGeom& cg = p.conv;
    int64_t cv_base[T::A_CHW];  // (n - first image) * H * W * C + 4 kq
    int cv_ih0[T::A_CHW], cv_iw0[T::A_CHW];
    bool cv_row[T::A_CHW];
    int64_t cv_org = 0, cv_span = 0;  // first element and element count of the tile's images
    if constexpr (T::CONV) {
        const int64_t hwc = (int64_t)cg.H * cg.W * cg.C;
        const int pq = cg.P * cg.Q;
        const int img0 = m0 / pq;
        const int img1 = (min(p.M, m0 + T::BM) - 1) / pq;
        cv_org = uniform_i64((int64_t)img0 * hwc);
        cv_span = uniform_i64((int64_t)(img1 - img0 + 1) * hwc);
#pragma unroll
        for (int j = 0; j < T::A_CHW; ++j) {
            const int q = 64 * (wave * T::A_CHW + j) + lane;
            const int r = q / T::A_QPR;
            const int kq = (q % T::A_QPR) ^ T::swz(r);
            cv_row[j] = r < rows_left;
            const int m = cv_row[j] ? m0 + r : m0;
            const int oq = m % cg.Q;
            const int t = m / cg.Q;
            const int op = t % cg.P;
            const int n = t / cg.P;
            cv_base[j] = (int64_t)(n - img0) * hwc + 4 * kq;
            cv_ih0[j] = op * cg.stride_h - cg.pad_h;
            cv_iw0[j] = oq * cg.stride_w - cg.pad_w;
        }
    }
    auto conv_offsets = [&](int tap) {
        const int fr = tap / cg.S;
        const int fs = tap - fr * cg.S;
#pragma unroll
        for (int j = 0; j < T::A_CHW; ++j) {
            const int ih = cv_ih0[j] + fr * cg.dil_h;
            const int iw = cv_iw0[j] + fs * cg.dil_w;
            const bool ok = cv_row[j] && (unsigned)ih < (unsigned)cg.H && (unsigned)iw < (unsigned)cg.W;
            a_off[j] = ok ? (uint32_t)((cv_base[j] + ((int64_t)ih * cg.W + iw) * cg.C) * 4)
                          : kOutOfRange;
        }
    };

    // The copies of a direct slice with index j in [lo, hi): this wave's A
    // chunks are j < A_CHW, its B chunks the rest.  Schedule 2 issues them
    // one per k step; otherwise (and always for a convolution, whose offsets
    // are rebuilt at a new filter tap) all at once.
    auto load_direct_part = [&](int k0, int buf, int lo, int hi) {
        float* const dstA = smem + buf * T::BUF_FLOATS;
        float* const dstB = dstA + T::A_FLOATS;
        int a_range = (int)a_span;
        int64_t a_step = T::A_KC ? (int64_t)k0 : (int64_t)k0 * p.lda;
        if constexpr (T::CONV) {
            // Slices are copied in k order, so the offsets are rebuilt at a
            // new tap and at the first slice (a split-K chunk may start
            // inside a tap).
            const int kg = kbeg + k0;
            const int tap = __builtin_amdgcn_readfirstlane(kg / cg.C);
            const int c0 = kg - tap * cg.C;
            if (c0 == 0 || k0 == 0) conv_offsets(tap);
            a_step = cv_org + c0;
            a_range = (int)((cv_span - c0) * 4);
        }
        const float* const a_base = p.A + uniform_i64(a_org + a_step);
        const float* const b_base =
            p.B + uniform_i64(b_org + (T::B_KC ? (int64_t)k0 : (int64_t)k0 * p.ldb));
        const __amdgpu_buffer_rsrc_t ra =
            __builtin_amdgcn_make_buffer_rsrc((void*)a_base, (short)0, a_range, 0x00020000);
        const __amdgpu_buffer_rsrc_t rb =
            __builtin_amdgcn_make_buffer_rsrc((void*)b_base, (short)0, (int)b_span, 0x00020000);
#pragma unroll
        for (int j = 0; j < T::LPS; ++j) {
            if (j < lo || j >= hi) continue;
            if (j < T::A_CHW)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    ra, (lds_void_t*)(dstA + 256 * (wave * T::A_CHW + j)), 16, a_off[j], 0, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rb, (lds_void_t*)(dstB + 256 * (wave * T::B_CHW + j - T::A_CHW)), 16,
                    b_off[j - T::A_CHW], 0, 0, 0);
        }
    };
    auto load_direct = [&](int k0, int buf) { load_direct_part(k0, buf, 0, T::LPS); };

    // Fallback for slices with quads that straddle the matrix edge: masked
    // element loads through registers, written to the same layout.
    auto load_staged = [&](int k0, int buf) {
        float* const As = smem + buf * T::BUF_FLOATS;
        float* const Bs = As + T::A_FLOATS;
        // One quad at a time: slow, but holds no registers across the slice.
#pragma unroll 1
        for (int v = 0; v < T::A_VEC; ++v) {
            const int q = tid + v * T::NT;
            const int r = q / T::A_QPR;
            f32x4 x;
            if constexpr (T::CONV) {
                // Element by element: the four k of a quad may straddle taps.
                const int kq = (q % T::A_QPR) ^ T::swz(r);
                x = f32x4{0.f, 0.f, 0.f, 0.f};
                if (r < rows_left) {
                    const int m = m0 + r;
                    const int oq = m % cg.Q;
                    const int t = m / cg.Q;
                    const int op = t % cg.P;
                    const int n = t / cg.P;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int k = k0 + 4 * kq + e;
                        if (k < Kd) {
                            const int tap = (kbeg + k) / cg.C;
                            const int c = kbeg + k - tap * cg.C;
                            const int fr = tap / cg.S;
                            const int fs = tap - fr * cg.S;
                            const int ih = op * cg.stride_h - cg.pad_h + fr * cg.dil_h;
                            const int iw = oq * cg.stride_w - cg.pad_w + fs * cg.dil_w;
                            if ((unsigned)ih < (unsigned)cg.H && (unsigned)iw < (unsigned)cg.W)
                                x[e] = p.A[(((int64_t)n * cg.H + ih) * cg.W + iw) * cg.C + c];
                        }
                    }
                }
            } else if constexpr (T::A_KC) {
                const int kq = (q % T::A_QPR) ^ T::swz(r);
                x = ldg4_masked(A + (int64_t)r * p.lda + k0 + 4 * kq,
                                r < rows_left ? Kd - (k0 + 4 * kq) : 0);
            } else {
                const int mq = (q % T::A_QPR) ^ T::flipA(r);
                x = ldg4_masked(A + (int64_t)(k0 + r) * p.lda + 4 * mq,
                                k0 + r < Kd ? rows_left - 4 * mq : 0);
            }
            *(f32x4*)(As + 4 * q) = x;
        }
#pragma unroll 1
        for (int v = 0; v < T::B_VEC; ++v) {
            const int q = tid + v * T::NT;
            const int r = q / T::B_QPR;
            f32x4 x;
            if constexpr (T::B_KC) {
                const int kq = (q % T::B_QPR) ^ T::swz(r);
                const int n = T::bkc_row(r);
                x = ldg4_masked(B + (int64_t)n * p.ldb + k0 + 4 * kq,
                                n < cols_left ? Kd - (k0 + 4 * kq) : 0);
            } else {
                const int nq = (q % T::B_QPR) ^ T::flipB(r);
                x = ldg4_masked(B + (int64_t)(k0 + r) * p.ldb + 4 * nq,
                                k0 + r < Kd ? cols_left - 4 * nq : 0);
            }
            *(f32x4*)(Bs + 4 * q) = x;
        }
    };

    // Direct staging needs 31-bit descriptor spans and, for an operand staged
    // [k][mn], whole quads along its m or n edge; a partial K slice (the last
    // one when BK does not divide K) goes through registers, so the offsets
    // stay fixed for the whole loop.
    // A convolution stages directly when every slice lies inside one filter
    // tap (C a multiple of BK) and the byte offsets into the tile's images fit
    // 31 bits.
    const bool direct_ok = (T::CONV ? (cg.C % T::BK == 0 && cv_span * 4 < (int64_t)kOutOfRange)
                                    : a_span64 * 4 < (int64_t)kOutOfRange) &&
                           b_span64 * 4 < (int64_t)kOutOfRange &&
                           (T::A_KC || rows_left >= T::BM || p.M % 4 == 0) &&
                           (T::B_KC || cols_left >= T::BN || p.N % 4 == 0);
    const int full_slices = Kd / T::BK;

    make_offsets(T::BK);
    auto load_slice = [&](int s) {
        const int k0 = s * T::BK;
        const int buf = s % T::STAGES;
        if (direct_ok && s < full_slices)
            load_direct(k0, buf);
        else
            load_staged(k0, buf);
    };
    // Slice t has landed in this wave's part of LDS once only the direct
    // copies of later slices (issued up to slice `last`) are outstanding; a
    // register-staged slice is complete when load_staged returns.
    auto wait_slice = [&](int t, int last) {
        const int direct_last = (direct_ok ? full_slices : 0) - 1;
        const int d = (last < direct_last ? last : direct_last) - t;
        wait_slices_after<T::LPS, T::STAGES - 2>(d);
    };

    // --------------------------------------------------------------- compute
    const int wave_mn = wave % T::NWMN;
    const int kgrp = wave / T::NWMN;  // which KSUB-wide part of every slice this wave reduces
    const int wy = wave_mn / T::WAVES_N;
    const int wx = wave_mn % T::WAVES_N;
    const int li = lane % T::MI;
    const int lg = lane / T::MI;

    typename Op::acc_t acc[T::TM][T::TN];
#pragma unroll
    for (int mi = 0; mi < T::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < T::TN; ++ni)
#pragma unroll
            for (int r = 0; r < Op::ACC; ++r) acc[mi][ni][r] = 0.0f;

    // Row (k-contiguous) or column ([k][mn]) of this lane in each MFMA tile.
    // The swizzle of a k-contiguous row is the same for every tile of the
    // wave (tiles are MI rows apart); a [k][mn] column carries the row-block
    // flip of the k values this lane reads (all with k / KPL = kgrp * LG + lg).
    const int a_row = wy * T::WTM + li;
    const int a_swz = T::swz(a_row);
    const int b_row = wx * T::WTN + li;
    const int b_swz = T::swz(b_row);
    const int kfirst = kgrp * T::KSUB + lg * T::KPL;
    const int kflip_a = 4 * T::flipA(kfirst);
    const int kflip_b = 4 * T::flipB(kfirst);
    // First row of each AV-wide run of row tiles (AV = 1: every tile).
    constexpr int NAV = T::TM / T::AV;
    int a_col[NAV];
#pragma unroll
    for (int h = 0; h < NAV; ++h) a_col[h] = (wy * T::WTM + T::arow(h * T::AV, li)) ^ kflip_a;
    // First column of each BV-wide run of column tiles (BV = 1: every tile).
    constexpr int NBV = T::TN / T::BV;
    int b_col[NBV];
#pragma unroll
    for (int h = 0; h < NBV; ++h) b_col[h] = (wx * T::WTN + T::bcol(h * T::BV, li)) ^ kflip_b;

    // One operand group = KG consecutive k steps: one 16-byte quad of A per
    // row tile and KG values of B per column tile.  The operands of group g+1
    // are read while the MFMAs of group g are issued ("Tiling Hierarchy on
    // GPUs", "Register prefetching").  A group is a list of LDS reads: the A
    // items first (one quad per row tile, or one float per k step and row
    // tile for A staged [k][m]), then the B items (one quad per column tile,
    // one float per k step and column tile, or one BV-vector per k step and
    // run of column tiles); read_items issues those with index in [lo, hi).
    using AReg = typename T::AReg;
    using BReg = typename T::BReg;
    constexpr int NA_ITEMS = T::A_KC ? T::TM : T::KG * NAV;
    constexpr int NB_ITEMS = T::B_KC ? T::TN : T::KG * NBV;
    constexpr int N_ITEMS = NA_ITEMS + NB_ITEMS;
    auto read_items = [&](int buf, int g, int lo, int hi, AReg (&a)[T::TM], BReg (&b)[T::TN]) {
        const float* const As = smem + buf * T::BUF_FLOATS;
        const float* const Bs = As + T::A_FLOATS;
        const int krow = kgrp * T::KSUB + lg * T::KPL + g * T::KG;  // first k of the group
        const int quad = krow / 4;
#pragma unroll
        for (int i = 0; i < N_ITEMS; ++i) {
            if (i < lo || i >= hi) continue;
            if (i < NA_ITEMS) {
                if constexpr (T::A_KC) {
                    a[i] = *(const f32x4*)(As + (a_row + T::MI * i) * T::BK + ((quad ^ a_swz) << 2));
                } else if constexpr (T::AV == 1) {
                    const int st = i / T::TM, mi = i % T::TM;
                    a[mi][st] = As[(krow + st) * T::LDA_S + a_col[mi]];
                } else {
                    typedef float avec_t __attribute__((ext_vector_type(T::AV)));
                    const int st = i / NAV, h = i % NAV;
                    const avec_t v = *(const avec_t*)(As + (krow + st) * T::LDA_S + a_col[h]);
#pragma unroll
                    for (int u = 0; u < T::AV; ++u) a[h * T::AV + u][st] = v[u];
                }
            } else {
                const int j = i - NA_ITEMS;
                if constexpr (T::B_KC) {
                    b[j] = *(const f32x4*)(Bs + (b_row + T::MI * j) * T::BK + ((quad ^ b_swz) << 2));
                } else if constexpr (T::BV == 1) {
                    const int st = j / T::TN, ni = j % T::TN;
                    b[ni][st] = Bs[(krow + st) * T::LDB + b_col[ni]];
                } else {
                    typedef float bvec_t __attribute__((ext_vector_type(T::BV)));
                    const int st = j / NBV, h = j % NBV;
                    const bvec_t v = *(const bvec_t*)(Bs + (krow + st) * T::LDB + b_col[h]);
#pragma unroll
                    for (int u = 0; u < T::BV; ++u) b[h * T::BV + u][st] = v[u];
                }
            }
        }
    };
    auto read_group = [&](int buf, int g, AReg (&a)[T::TM], BReg (&b)[T::TN]) {
        read_items(buf, g, 0, N_ITEMS, a, b);
    };
    // Part `part` of KG: the items [part, part + 1) * N_ITEMS / KG.
    auto read_part = [&](int buf, int g, int part, AReg (&a)[T::TM], BReg (&b)[T::TN]) {
        read_items(buf, g, part * N_ITEMS / T::KG, (part + 1) * N_ITEMS / T::KG, a, b);
    };

    auto mfma_steps = [&](const AReg (&a)[T::TM], const BReg (&b)[T::TN], int s0, int s1) {
#pragma unroll
        for (int s = s0; s < s1; ++s)
#pragma unroll
            for (int mi = 0; mi < T::TM; ++mi)
#pragma unroll
                for (int ni = 0; ni < T::TN; ++ni)
                    acc[mi][ni] = Op::mma(a[mi][s], b[ni][s], acc[mi][ni]);
    };

    AReg opa[2][T::TM];
    BReg opb[2][T::TN];

    // One slice held in LDS buffer `buf` (operand group g uses set g & 1):
    // the copy of slice s + STAGES - 1 is started first, into the buffer that
    // slice s - 1 used (every wave finished reading it before the previous
    // barrier); slice s + 1 is complete at this slice's barrier.  The last
    // HOLD k steps of MFMAs run after the barrier, behind the reads of the next
    // slice's first operand group, so the matrix core keeps working while the
    // waves synchronise.
    // Inside a slice (SCHED >= 1) the reads of group g+1 go out in KG parts,
    // one after each k step of group g's MFMAs, fenced by scheduling barriers
    // so the compiler keeps the MFMAs in k-step order (left free, it pairs
    // MFMAs on the same accumulator, which then wait on each other).  Spread
    // out, the waves' reads do not reach the LDS in one burst.  A copy
    // instruction holds its wave while the address unit takes it in: with
    // SCHED = 2 one copy follows each k step, behind MFMAs already issued,
    // which pays on small wave tiles (512 x 4096 x 4096 on 64 x 128 tiles:
    // +7 %); on the 256 x 256 tile, where the other wave of the SIMD covers
    // the burst, one burst at the start of the slice measured faster (as did
    // that burst against issuing the copies right after the barrier, ahead of
    // the held MFMAs).  With SCHED = 0 all reads of group g+1 go out before
    // group g.
    // `more` is a compile-time flag: the last slice is peeled off the loop so
    // that no control-flow join sits in front of the held MFMAs (at a join the
    // compiler's LDS wait would also cover the next slice's fresh reads).
    // `hoisted_tag` (HOIST_SPREAD tiles only): the caller has checked that
    // slice s + STAGES - 1 is a whole direct slice, so its copies go out one
    // per k step through descriptors built once, at the top of the slice.
    auto slice = [&](auto more_tag, auto hoisted_tag, int buf, int s) {
        constexpr bool more = decltype(more_tag)::value;
        constexpr bool HOISTED = decltype(hoisted_tag)::value;
        const int ahead = s + T::STAGES - 1;
        // Copies of a direct slice spread over the k steps (SCHED = 2); a
        // register-staged slice is copied whole at the start.
        const bool spread = T::SPREAD_COPIES && !T::HOIST_SPREAD && more && direct_ok &&
                            ahead < full_slices;
        if (more && ahead < nslices && !HOISTED && !spread) load_slice(ahead);
        __amdgpu_buffer_rsrc_t hs_ra, hs_rb;
        float* hs_dst = smem;
        if constexpr (HOISTED) {
            const int64_t k0 = (int64_t)ahead * T::BK;
            const float* const a_base =
                p.A + uniform_i64(a_org + (T::A_KC ? k0 : k0 * p.lda));
            const float* const b_base =
                p.B + uniform_i64(b_org + (T::B_KC ? k0 : k0 * p.ldb));
            hs_ra = __builtin_amdgcn_make_buffer_rsrc((void*)a_base, (short)0, (int)a_span,
                                                      0x00020000);
            hs_rb = __builtin_amdgcn_make_buffer_rsrc((void*)b_base, (short)0, (int)b_span,
                                                      0x00020000);
            hs_dst = smem + (ahead % T::STAGES) * T::BUF_FLOATS;
        }
#pragma unroll
        for (int g = 0; g < T::NKG; ++g) {
            const int s1 = g + 1 < T::NKG ? T::KG : T::KG - T::HOLD;
            if constexpr (T::ILV) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int st = 0; st < s1; ++st) {
                    if (g & 1)
                        mfma_steps(opa[1], opb[1], st, st + 1);
                    else
                        mfma_steps(opa[0], opb[0], st, st + 1);
                    if (g + 1 < T::NKG) {
                        if (g & 1)
                            read_part(buf, g + 1, st, opa[0], opb[0]);
                        else
                            read_part(buf, g + 1, st, opa[1], opb[1]);
                    }
                    if constexpr (HOISTED) {
                        // Copy j = this k step's index, as load_direct_part
                        // issues it.
                        const int j = g * T::KG + st;
                        if (j < T::A_CHW)
                            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                                hs_ra, (lds_void_t*)(hs_dst + 256 * (wave * T::A_CHW + j)), 16,
                                a_off[j < T::A_CHW ? j : 0], 0, 0, 0);
                        else if (j < T::LPS)
                            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                                hs_rb,
                                (lds_void_t*)(hs_dst + T::A_FLOATS +
                                              256 * (wave * T::B_CHW + j - T::A_CHW)),
                                16, b_off[j >= T::A_CHW && j < T::LPS ? j - T::A_CHW : 0], 0,
                                0, 0);
                    } else if constexpr (T::SPREAD_COPIES) {
                        const int step = g * T::KG + st;
                        if (spread && step < T::LPS)
                            load_direct_part(ahead * T::BK, ahead % T::STAGES, step, step + 1);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                if (g + 1 < T::NKG) {
                    if (g & 1)
                        read_group(buf, g + 1, opa[0], opb[0]);
                    else
                        read_group(buf, g + 1, opa[1], opb[1]);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (g & 1)
                    mfma_steps(opa[1], opb[1], 0, s1);
                else
                    mfma_steps(opa[0], opb[0], 0, s1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (more) {
            // The direct copies count on vmcnt: wait for this wave's, then the
            // barrier makes every wave's part of the slice visible.
            wait_slice(s + 1, ahead < nslices ? ahead : nslices - 1);
            lds_barrier();
            if constexpr (kRaceCheck) {
                // Slice s is consumed: its buffer is refilled only after this.
                poison_lds(smem + buf * T::BUF_FLOATS, T::BUF_FLOATS, tid, T::NT);
                lds_barrier();
            }
            read_group((s + 1) % T::STAGES, 0, opa[0], opb[0]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // The last group, NKG-1, is odd: operand set 1.
        mfma_steps(opa[1], opb[1], T::KG - T::HOLD, T::KG);
        __builtin_amdgcn_sched_barrier(0);
    };

    if constexpr (kRaceCheck) {
        poison_lds(smem, T::STAGES * T::BUF_FLOATS, tid, T::NT);
        lds_barrier();
    }
#pragma unroll
    for (int t = 0; t < T::STAGES - 1; ++t)
        if (t < nslices) load_slice(t);
    wait_slice(0, (T::STAGES - 1 < nslices ? T::STAGES - 1 : nslices) - 1);
    lds_barrier();
    read_group(0, 0, opa[0], opb[0]);
    int s = 0;
    if constexpr (T::HOIST_SPREAD) {
        // Slices whose slice ahead is a whole direct slice: every slice but
        // the last STAGES - 1 when BK divides K and the slices copy directly.
        const int s_end = direct_ok ? min(nslices - 1, full_slices - (T::STAGES - 1)) : 0;
        for (; s < s_end; ++s) slice(std::true_type(), std::true_type(), s % T::STAGES, s);
    }
    for (; s + 1 < nslices; ++s) slice(std::true_type(), std::false_type(), s % T::STAGES, s);
    slice(std::false_type(), std::false_type(), (nslices - 1) % T::STAGES, nslices - 1);

    // k groups 1..KSPLIT-1 hand their partial sums to group 0 through LDS
    // (lane-contiguous 16-byte records, conflict-free); group 0 adds them in
    // group order, so the result does not depend on timing.
    // With four or more k groups the adding and the stores are shared: every
    // group writes its records, and group g sums the accumulator rows r in
    // [g, g + 1) * ACC / KSPLIT over all groups, in the same group order
    // 0, 1, ... (the same FP32 operations, so the same bits), and stores
    // those rows: 1024^3 on the 64 x 64 x 128 tile with four k groups,
    // 19.95 -> 19.69 us (with two groups it measured 0.5 % slower, and stays
    // with group 0).  Split-K shares the partial tile and the join the same
    // way (SK_SHARED, below).
    constexpr bool SHARED_ROWS = T::KSPLIT >= 4 && Op::ACC % (4 * T::KSPLIT) == 0 &&
                                 T::KSPLIT * T::BM * T::BN <= T::STAGES * T::BUF_FLOATS;
    constexpr bool SHARED_EXCHANGE = SHARED_ROWS && !T::SK;
    constexpr bool SK_SHARED = SHARED_ROWS && T::SK;
    constexpr int NACC = T::TM * T::TN * Op::ACC;  // accumulator values per lane
    static_assert(T::KSPLIT == 1 || NACC % 4 == 0, "whole 16-byte records");
    // Record q of a wave holds its accumulator values f = 4q .. 4q + 3,
    // f = (mi * TN + ni) * ACC + r, lane l's at 4 * (q * 64 + l) of `dst`.
    auto write_records = [&](float* const dst) {
#pragma unroll
        for (int q = 0; q < NACC / 4; ++q) {
            f32x4 v;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int f = 4 * q + c;
                v[c] = acc[f / (T::TN * Op::ACC)][(f / Op::ACC) % T::TN][f % Op::ACC];
            }
            *(f32x4*)(dst + 4 * (q * 64 + lane)) = v;
        }
    };
    // Split-K join.  Each workgroup writes its partial tile to the workspace
    // and counts itself in on the tile's counter; the workgroup that arrives
    // last adds every split's partial in split order 0, 1, ... (so the sum
    // does not depend on which split finished last), resets the counter for
    // the next call and stores the tile.  No workgroup waits for another.
    // Ordering rests on how gfx950 (a member of the GFX942 family in LLVM's
    // AMDGPU memory model) performs relaxed device-scope atomics, not on
    // C++ release/acquire: the model maps relaxed agent-scope atomic stores
    // and loads of global memory to global_store / global_load with the sc1
    // bit (performed coherently across the XCDs' L2 caches) and atomic RMWs
    // to global_atomic at the device's coherence point.  Every partial is
    // such a store; s_waitcnt vmcnt(0) holds each wave until its stores are
    // acknowledged, the barrier holds lane 0 until every wave has done so,
    // and only then does lane 0 increment the counter.  The last arriver
    // sees every other increment, so every partial was complete before its
    // own increment returned, and its sc1 loads issue after that return.
    // A device-scope release on the increment and an acquire fence after it
    // would state the same order in the language's model, but on gfx950
    // they write back and invalidate the XCD's whole L2 per workgroup (the
    // operand tiles of every other workgroup on it included): measured at
    // 1024^3 with 4 chunks, 24.6 -> 53.7 us per product; at 512x4096x4096
    // with 8 chunks, 154 -> 172 us.
    // sk_arrive: once every wave's partial stores are acknowledged, lane 0
    // counts the workgroup in on the tile's counter; returns whether it
    // arrived last.  The flag goes in LDS word 0: every wave's reads of the
    // slices and records end before the first barrier here.
    auto sk_arrive = [&](int tile) {
        int* const sk_last = (int*)smem;
        wait_vmcnt<0>();
        __syncthreads();
        if (tid == 0) {
            const uint32_t before = __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
            const int last = before == (uint32_t)p.splits - 1;
            if (last)
                __hip_atomic_store(p.counters + tile, 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            *sk_last = last;
        }
        __syncthreads();
        return *sk_last != 0;
    };
    if constexpr (SHARED_EXCHANGE) {
        constexpr int RQ = Op::ACC / T::KSPLIT;  // accumulator rows per group
        lds_barrier();  // every wave is done reading the slices
        write_records(smem + (kgrp * T::NWMN + wave_mn) * 64 * NACC);
        lds_barrier();
        // Group G's rows, summed in group order.
        auto sum_rows = [&](auto gtag) {
            constexpr int G = decltype(gtag)::value;
#pragma unroll
            for (int mi = 0; mi < T::TM; ++mi)
#pragma unroll
                for (int ni = 0; ni < T::TN; ++ni)
#pragma unroll
                    for (int q4 = 0; q4 < RQ / 4; ++q4) {
                        const int q = ((mi * T::TN + ni) * Op::ACC + G * RQ) / 4 + q4;
                        f32x4 sum;
#pragma unroll
                        for (int j = 0; j < T::KSPLIT; ++j) {
                            f32x4 v;
                            if (j == G) {
#pragma unroll
                                for (int c = 0; c < 4; ++c) v[c] = acc[mi][ni][G * RQ + 4 * q4 + c];
                            } else {
                                v = *(const f32x4*)(smem + (j * T::NWMN + wave_mn) * 64 * NACC +
                                                    4 * (q * 64 + lane));
                            }
                            if (j == 0)
                                sum = v;
                            else
                                sum += v;
                        }
#pragma unroll
                        for (int c = 0; c < 4; ++c) acc[mi][ni][G * RQ + 4 * q4 + c] = sum[c];
                    }
        };
        for_group<0, T::KSPLIT>(kgrp, sum_rows);
    } else if constexpr (SK_SHARED) {
        // Split-K with shared rows: group g sums its rows over the k groups,
        // writes them as its part of the partial tile, and in the workgroup
        // that arrives last adds them over the splits and stores them.
        constexpr int RQ = Op::ACC / T::KSPLIT;  // accumulator rows per group
        constexpr int NQ = T::TM * T::TN * RQ;   // values per lane of a group's rows
        constexpr int TILE = T::BM * T::BN;
        lds_barrier();  // every wave is done reading the slices
        write_records(smem + (kgrp * T::NWMN + wave_mn) * 64 * NACC);
        lds_barrier();
        // All terms are read back from the records (the group's own
        // included), so no accumulator is picked by the run-time group index
        // (which would move the accumulators to scratch memory).
        float part[NQ];
#pragma unroll
        for (int mi = 0; mi < T::TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < T::TN; ++ni)
#pragma unroll
                for (int q4 = 0; q4 < RQ / 4; ++q4) {
                    const int q = ((mi * T::TN + ni) * Op::ACC + kgrp * RQ) / 4 + q4;
                    f32x4 sum = *(const f32x4*)(smem + wave_mn * 64 * NACC + 4 * (q * 64 + lane));
#pragma unroll
                    for (int j = 1; j < T::KSPLIT; ++j)
                        sum += *(const f32x4*)(smem + (j * T::NWMN + wave_mn) * 64 * NACC +
                                               4 * (q * 64 + lane));
#pragma unroll
                    for (int c = 0; c < 4; ++c) part[(mi * T::TN + ni) * RQ + 4 * q4 + c] = sum[c];
                }
        // The partial tile of a split: value j (= (mi * TN + ni) * RQ + r)
        // of lane l of wave (kgrp, wave_mn) at ((kgrp * NWMN + wave_mn) * NQ
        // + j) * 64 + l, so each store or load covers 256 contiguous bytes.
        if (!sk_full) {
            const int tile = sk_tail;
            float* const slot0 = p.ws + (int64_t)tile * p.splits * TILE +
                                 (kgrp * T::NWMN + wave_mn) * 64 * NQ + lane;
            {
                float* const dst = slot0 + (int64_t)tc.b * TILE;
#pragma unroll
                for (int j = 0; j < NQ; ++j)
                    __hip_atomic_store(dst + j * 64, part[j], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            if (!sk_arrive(tile)) return;
            // Sums over the splits in split order; the loads of up to four
            // splits go out together (splits past the last repeat the last one's
            // loads, whose values are not added).
#pragma unroll
            for (int j = 0; j < NQ; ++j) part[j] = 0.0f;
#pragma unroll 1
            for (int sp0 = 0; sp0 < p.splits; sp0 += 4) {
                float v[4][NQ];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float* const src = slot0 + (int64_t)min(sp0 + u, p.splits - 1) * TILE;
#pragma unroll
                    for (int j = 0; j < NQ; ++j)
                        v[u][j] = __hip_atomic_load(src + j * 64, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const bool in = sp0 + u < p.splits;
#pragma unroll
                    for (int j = 0; j < NQ; ++j) part[j] = in ? part[j] + v[u][j] : part[j];
                }
            }
        }
        // The group's rows of C, as in the epilogue below with the rows
        // taken at run time.
        typedef float svec_t __attribute__((ext_vector_type(T::BV), aligned(4)));
#pragma unroll
        for (int mi = 0; mi < T::TM; ++mi)
#pragma unroll
            for (int h = 0; h < NBV; ++h) {
                const int col = wx * T::WTN + T::bcol(h * T::BV, li);
#pragma unroll
                for (int r = 0; r < RQ; ++r) {
                    const int row = wy * T::WTM + T::arow(mi, Op::row(kgrp * RQ + r, lg));
                    float* const c = C + (int64_t)row * p.ldc + col;
                    svec_t v;
#pragma unroll
                    for (int u = 0; u < T::BV; ++u)
                        v[u] = part[(mi * T::TN + h * T::BV + u) * RQ + r];
                    if constexpr (T::EX) {
                        // alpha * sum, plus beta * C when beta != 0.
                        if (p.beta != 0.0f) {
#pragma unroll
                            for (int u = 0; u < T::BV; ++u) {
                                const bool in = full_mn ||
                                                (row < rows_left && col + u < cols_left);
                                const float old = in ? c[u] : 0.0f;
                                v[u] = __builtin_fmaf(p.beta, old, p.alpha * v[u]);
                            }
                        } else {
#pragma unroll
                            for (int u = 0; u < T::BV; ++u) v[u] = p.alpha * v[u];
                        }
                    }
                    if (full_mn) {
                        __builtin_nontemporal_store(v, (svec_t*)c);
                    } else {
#pragma unroll
                        for (int u = 0; u < T::BV; ++u)
                            if (row < rows_left && col + u < cols_left) c[u] = v[u];
                    }
                }
            }
        return;
    } else if constexpr (T::KSPLIT > 1) {
        lds_barrier();  // every wave is done reading the slices
        if (kgrp > 0) write_records(smem + ((kgrp - 1) * T::NWMN + wave_mn) * 64 * NACC);
        lds_barrier();
        // (Split-K: every wave takes part in the join's barriers below.)
        if (kgrp > 0 && !T::SK) return;
#pragma unroll 1
        for (int j = 1; j < T::KSPLIT && kgrp == 0; ++j) {
            const float* const src = smem + ((j - 1) * T::NWMN + wave_mn) * 64 * NACC;
#pragma unroll
            for (int q = 0; q < NACC / 4; ++q) {
                const f32x4 v = *(const f32x4*)(src + 4 * (q * 64 + lane));
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int f = 4 * q + c;
                    acc[f / (T::TN * Op::ACC)][(f / Op::ACC) % T::TN][f % Op::ACC] += v[c];
                }
            }
        }
    }

    // Split-K join with the tile's sums in k group 0 (record layout: value
    // f of lane l at f * 64 + l, so each store or load instruction covers
    // 256 contiguous bytes).
    if constexpr (T::SK && !SK_SHARED) {
        constexpr int TILE = T::BM * T::BN;
        const bool holds = T::KSPLIT == 1 || kgrp == 0;  // waves with the tile's sums
        // A tile that takes all of K has its sums in k group 0 already.
        if (sk_full && !holds) return;
        if (!sk_full) {
            const int tile = sk_tail;
            float* const slot0 =
                p.ws + (int64_t)tile * p.splits * TILE + wave_mn * 64 * NACC + lane;
            if (holds) {
                float* const dst = slot0 + (int64_t)tc.b * TILE;
#pragma unroll
                for (int f = 0; f < NACC; ++f)
                    __hip_atomic_store(
                        dst + f * 64,
                        acc[f / (T::TN * Op::ACC)][(f / Op::ACC) % T::TN][f % Op::ACC],
                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (!sk_arrive(tile) || !holds) return;
            float sum[NACC];
#pragma unroll
            for (int f = 0; f < NACC; ++f) sum[f] = 0.0f;
#pragma unroll 1
            for (int sp = 0; sp < p.splits; ++sp) {
                const float* const src = slot0 + (int64_t)sp * TILE;
#pragma unroll
                for (int f = 0; f < NACC; ++f)
                    sum[f] += __hip_atomic_load(src + f * 64, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int f = 0; f < NACC; ++f)
                acc[f / (T::TN * Op::ACC)][(f / Op::ACC) % T::TN][f % Op::ACC] = sum[f];
        }
    }

    // Epilogue: accumulator r of lane (li, lg) in MFMA tile (mi, ni) is
    // wave-tile row arow(mi, Op::row(r, lg)) and column bcol(ni, li).  The
    // general form stores
    // alpha * acc, plus beta * C when beta != 0 (C is not read otherwise); the
    // choice is made once, outside the store loop.
    // An interior tile reads C ahead of its stores, a fixed number of values
    // ahead (a ring of registers: 32 values per lane, 16 where four waves
    // share a SIMD).  A load placed after a store to C cannot be moved ahead
    // of it (with an unknown ldc the two may overlap), so loads interleaved
    // with the stores waited out one memory latency each (2048^3 with beta =
    // 0.5, the four layouts: 135.3-139.4 TFLOP/s before, 138.0-142.1 after).
    // A whole row tile ahead spilled registers on the widest tiles.
    // With BV > 1 a lane's BV outputs of one row are adjacent columns: an
    // interior tile stores them as one vector (rows with an odd ldc start on
    // any 4-byte boundary, which vector stores accept), an edge tile element
    // by element.
    typedef float cvec_t __attribute__((ext_vector_type(T::BV), aligned(4)));
    // Rows r in [R0, R1) of the accumulators (all of them, or this k group's
    // share after a shared exchange).
    auto store = [&](auto read_c_tag, auto masked_tag, auto r0_tag, auto r1_tag) {
        constexpr bool read_c = decltype(read_c_tag)::value;
        constexpr bool masked = decltype(masked_tag)::value;
        constexpr int R0 = decltype(r0_tag)::value, R1 = decltype(r1_tag)::value;
        constexpr bool ahead = T::EX && read_c && !masked;
        constexpr int NR = R1 - R0, NV = T::TM * NBV * NR;  // vectors per lane
        constexpr int AHEAD = (T::OCC >= 3 ? 16 : 32) / T::BV;
        constexpr int DA = !ahead ? 1 : AHEAD < NV ? AHEAD : NV;
        // Address of vector i = (mi * NBV + h) * NR + r - R0.
        auto c_at = [&](int i) {
            const int mi = i / (NBV * NR), h = (i / NR) % NBV, r = R0 + i % NR;
            const int row = wy * T::WTM + T::arow(mi, Op::row(r, lg));
            const int col = wx * T::WTN + T::bcol(h * T::BV, li);
            return (const cvec_t*)(C + (int64_t)row * p.ldc + col);
        };
        cvec_t ring[DA];
        if constexpr (ahead) {
#pragma unroll
            for (int i = 0; i < DA; ++i) ring[i] = *c_at(i);
        }
#pragma unroll
        for (int mi = 0; mi < T::TM; ++mi) {
#pragma unroll
            for (int h = 0; h < NBV; ++h) {
                const int col = wx * T::WTN + T::bcol(h * T::BV, li);
#pragma unroll
                for (int r = R0; r < R1; ++r) {
                    const int row = wy * T::WTM + T::arow(mi, Op::row(r, lg));
                    float* const c = C + (int64_t)row * p.ldc + col;
                    cvec_t v;
#pragma unroll
                    for (int u = 0; u < T::BV; ++u) v[u] = acc[mi][h * T::BV + u][r];
                    if constexpr (T::EX) {
                        if constexpr (read_c) {
                            if constexpr (ahead) {
                                const int i = (mi * NBV + h) * NR + r - R0;
                                const cvec_t old = ring[i % DA];
                                if (i + DA < NV) ring[i % DA] = *c_at(i + DA);
#pragma unroll
                                for (int u = 0; u < T::BV; ++u)
                                    v[u] = __builtin_fmaf(p.beta, old[u], p.alpha * v[u]);
                            } else {
#pragma unroll
                                for (int u = 0; u < T::BV; ++u)
                                    if (row < rows_left && col + u < cols_left)
                                        v[u] = __builtin_fmaf(p.beta, c[u], p.alpha * v[u]);
                            }
                        } else {
#pragma unroll
                            for (int u = 0; u < T::BV; ++u) v[u] = p.alpha * v[u];
                        }
                    }
                    if (!masked) {
                        // Non-temporal: C is not read again by this kernel,
                        // and the hint keeps it from displacing operands in
                        // the caches (batched 1024 x 128^3: 42.5 -> 41.1 us;
                        // large products unchanged).
                        __builtin_nontemporal_store(v, (cvec_t*)c);
                    } else {
#pragma unroll
                        for (int u = 0; u < T::BV; ++u)
                            if (row < rows_left && col + u < cols_left) c[u] = v[u];
                    }
                }
            }
        }
    };
    auto store_rows = [&](auto read_c_tag, auto r0_tag, auto r1_tag) {
        if (full_mn)
            store(read_c_tag, std::false_type(), r0_tag, r1_tag);
        else
            store(read_c_tag, std::true_type(), r0_tag, r1_tag);
    };
    auto store_tile = [&](auto read_c_tag) {
        if constexpr (SHARED_EXCHANGE) {
            constexpr int RQ = Op::ACC / T::KSPLIT;
            for_group<0, T::KSPLIT>(kgrp, [&](auto gtag) {
                constexpr int G = decltype(gtag)::value;
                store_rows(read_c_tag, std::integral_constant<int, G * RQ>(),
                           std::integral_constant<int, (G + 1) * RQ>());
            });
        } else {
            store_rows(read_c_tag, std::integral_constant<int, 0>(),
                       std::integral_constant<int, Op::ACC>());
        }
    };
    if (T::EX && p.beta != 0.0f)
        store_tile(std::true_type());
    else
        store_tile(std::false_type());
}

template <class T>
__global__ __launch_bounds__(T::NT) __attribute__((amdgpu_waves_per_eu(T::OCC)))
void sgemm_mfma_dl_kernel(GemmArgs p) {
    sgemm_mfma_dl_body<T>(p);
}

}  // namespace sgemm_dev
