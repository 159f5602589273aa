// Shared device pieces of the FP32 GEMM kernels (gfx950, wave64):
//  * the kernel argument block,
//  * the workgroup -> output-tile map (XCD-aware, grouped),
//  * coalesced 16-byte global loads with zero-filled masks for tails.
//
// "CMU DLSys Lecture 12: GPU Acceleration" section 5 splits the work into
// block-owned output tiles and stages operand slabs cooperatively, with
// zero-filled masked loads where the tile runs past the matrix; section 1
// gives the ceil-div launch with a bounds check.  "Tiling Strategies"
// section 2 ("The Tiled Solution") gives the same loop over K in slices.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Race-check build (SGEMM_RACECHECK = 1, a separate test library): every
// LDS buffer is filled with NaN at the start of a workgroup and again as soon
// as the workgroup is done with it (after the barrier that ends its use, with
// a barrier after the fill), and workgroups take their tiles in reverse order.
// A wave that read a slice before its copy had landed, or after its buffer was
// handed on, would read NaN, and NaN reaches the result.  The product library
// is built with SGEMM_RACECHECK = 0, where none of this is compiled in.
#ifndef SGEMM_RACECHECK
#define SGEMM_RACECHECK 0
#endif

namespace sgemm_dev {

constexpr bool kRaceCheck = SGEMM_RACECHECK != 0;

// n floats of LDS from p set to NaN by the nt threads of a workgroup (the
// caller adds the barrier).
__device__ __forceinline__ void poison_lds(float* p, int n, int tid, int nt) {
    for (int i = tid; i < n; i += nt) p[i] = __builtin_nanf("");
}

// Geometry of a 2-D convolution run as an implicit GEMM (NHWC input, KRSC
// filters, NPQK output): GEMM row m = (n * P + p) * Q + q, column = output
// channel, reduction index k = (r * S + s) * C + c.  Unused by plain GEMMs.
struct ConvGeom {
    int H, W, C;          // input image
    int P, Q, S;          // output image, filter width (R = K / (S * C))
    int pad_h, pad_w, stride_h, stride_w, dil_h, dil_w;
};

// Kernel arguments.  Sizes are validated on the host: M, N, K < 2^31, all
// element offsets fit in int64.
struct GemmArgs {
    const float* A;
    const float* B;
    float* C;
    int64_t lda, ldb, ldc;
    int64_t strideA, strideB, strideC;  // batch strides (elements)
    int M, N, K;
    int tiles_m, tiles_n;               // output tiles per matrix
    int batch_base;                     // first batch index of this launch
    int batch_count;                    // batch members in this launch
    float alpha, beta;                  // C = alpha op(A) op(B) + beta C (general form only)
    ConvGeom conv;                      // implicit-GEMM convolution only
    // Split-K kernels only: split b (the batch index) reduces k in
    // [b * kchunk, min(K, (b + 1) * kchunk)); its partial tile goes to ws at
    // [tile][split], and counters[tile] counts the splits that have arrived.
    float* ws;
    uint32_t* counters;
    int kchunk, splits;
    int full_tiles;  // split-K: tiles taking all of K with no join (0: every tile splits)
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// 16-byte vector that only claims 4-byte alignment: rows with an odd leading
// dimension start on any 4-byte boundary and are still read with one
// global_load_dwordx4 (the hardware accepts dword-aligned vector loads).
typedef float f32x4_u __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, one L2 each

// Workgroups are handed to the XCDs round-robin (id % 8), and each XCD has its
// own L2.  Renumber so that each XCD receives a contiguous run of tile ids;
// with the grouped order below, neighbouring tiles that share A rows and B
// columns then run on the same XCD and hit the same L2.
__device__ __forceinline__ uint32_t xcd_contiguous_id(uint32_t bid, uint32_t nblocks) {
    const uint32_t xcd = bid % kNumXcd;
    const uint32_t slot = bid / kNumXcd;
    const uint32_t q = nblocks / kNumXcd;
    const uint32_t r = nblocks % kNumXcd;
    return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// Tile coordinates from a linear tile id: groups of `group_m` tile rows, and
// inside a group the tile row varies fastest, so consecutive ids sweep a
// group_m-tall column of tiles that reuses the same B panel.
__device__ __forceinline__ void grouped_tile(uint32_t pid, int tiles_m, int tiles_n, int group_m,
                                             int& tm, int& tn) {
    const uint32_t per_group = (uint32_t)group_m * (uint32_t)tiles_n;
    const uint32_t group = pid / per_group;
    const int first_m = (int)group * group_m;
    const int gsize = min(tiles_m - first_m, group_m);
    const uint32_t in_group = pid - group * per_group;
    tm = first_m + (int)(in_group % (uint32_t)gsize);
    tn = (int)(in_group / (uint32_t)gsize);
}

// Block -> (batch member, tile row, tile column) for a 1-D grid that covers
// tiles_m * tiles_n * batch_count workgroups.
struct TileCoord {
    int b, tm, tn;
};

__device__ __forceinline__ TileCoord map_block(const GemmArgs& p, int group_m) {
    const uint32_t nblocks = gridDim.x;
    const uint32_t bid = kRaceCheck ? nblocks - 1 - blockIdx.x : blockIdx.x;
    const uint32_t pid = xcd_contiguous_id(bid, nblocks);
    const uint32_t per_matrix = (uint32_t)p.tiles_m * (uint32_t)p.tiles_n;
    TileCoord t;
    t.b = (int)(pid / per_matrix);
    grouped_tile(pid - (uint32_t)t.b * per_matrix, p.tiles_m, p.tiles_n, group_m, t.tm, t.tn);
    t.b += p.batch_base;
    return t;
}

// Split-K block -> (tile, chunk).  With full_tiles = F > 0 the first F tiles
// (in grouped order) take all of K and need no join, and the other R tiles
// are split: each XCD receives F / 8 full tiles and (gridDim - F) / 8
// chunks, the full tiles first.  The host keeps both multiples of 8.
struct SplitCoord {
    TileCoord tc;  // tc.b: the chunk (0 for a full tile)
    int tail;      // join slot of a split tile, in [0, R) (every tile when F = 0)
    bool full;
};

__device__ __forceinline__ SplitCoord map_split_block(const GemmArgs& p, int group_m) {
    const uint32_t nblocks = gridDim.x;
    const uint32_t bid = kRaceCheck ? nblocks - 1 - blockIdx.x : blockIdx.x;
    const uint32_t tiles = (uint32_t)p.tiles_m * (uint32_t)p.tiles_n;
    SplitCoord s;
    uint32_t lin;
    if (p.full_tiles == 0) {
        const uint32_t pid = xcd_contiguous_id(bid, nblocks);
        s.tc.b = (int)(pid / tiles);
        lin = pid - (uint32_t)s.tc.b * tiles;
        s.tail = (int)lin;
        s.full = false;
    } else {
        const uint32_t F = (uint32_t)p.full_tiles, R = tiles - F;
        const uint32_t fx = F / kNumXcd, tx = (nblocks - F) / kNumXcd;
        const uint32_t xcd = bid % kNumXcd, slot = bid / kNumXcd;
        if (slot < fx) {
            lin = xcd * fx + slot;
            s.tc.b = 0;
            s.tail = 0;
            s.full = true;
        } else {
            const uint32_t u = xcd * tx + (slot - fx);
            s.tail = (int)(u % R);
            s.tc.b = (int)(u / R);
            lin = F + (uint32_t)s.tail;
            s.full = false;
        }
    }
    grouped_tile(lin, p.tiles_m, p.tiles_n, group_m, s.tc.tm, s.tc.tn);
    return s;
}

__device__ __forceinline__ f32x4 ldg4(const float* p) {
    return (f32x4)(*(const f32x4_u*)p);
}

// Four consecutive elements p[0..3] of one row, of which only the first
// `valid` (clamped to 0..4) exist; the rest read as zero and are not
// accessed, so padding and memory past the matrix are never touched.
__device__ __forceinline__ f32x4 ldg4_masked(const float* p, int valid) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (valid >= 4) {
        v = ldg4(p);
    } else if (valid > 0) {
        v.x = p[0];
        if (valid > 1) v.y = p[1];
        if (valid > 2) v.z = p[2];
    }
    return v;
}

__device__ __forceinline__ void stg4_masked(float* p, f32x4 v, int valid) {
    if (valid >= 4) {
        *(f32x4_u*)p = (f32x4_u)v;
    } else if (valid > 0) {
        p[0] = v.x;
        if (valid > 1) p[1] = v.y;
        if (valid > 2) p[2] = v.z;
    }
}

}  // namespace sgemm_dev
