// Sliding window sums y[i] = sum_{d<W} x[i+d], 0 <= i < n, with cooperative
// staging ("CMU DLSys Lecture 12: GPU Acceleration", section 3: a block loads
// the union of its outputs' windows -- its T outputs plus the W - 1 halo
// values -- into shared memory once, synchronises, and every thread reads its
// windows there; the input holds n + W - 1 valid values and the load guard is
// against that count, not n).
//
// gfx950 shape of the same idea.  The work is a few additions per value, so
// it is bound by HBM bandwidth (8 bytes per output), not by arithmetic:
//  * A workgroup of 256 lanes owns T = 1024 * QUADS consecutive outputs;
//    lane t owns the quads of outputs 4t + 1024j (j < QUADS), so every
//    16-byte store of a wave covers 1 KB of y contiguously.  Small blocks
//    put more workgroups, and so more copies, in flight at once; large ones
//    make the W - 1 halo a smaller share of each block's inputs.  Measured
//    on 2^28 outputs (TB/s for QUADS = 1 / 2 / 4): W = 5: 6.61 / 6.45 / 6.28;
//    W = 9: 6.42 / 6.45 / 6.18; W = 17: 5.97 / 6.43 / 6.20; W = 24: 5.65 /
//    5.90 / 5.89; W = 33: 4.67 / 4.87 / 4.89.  So QUADS = 1 up to W = 8, 2 up
//    to W = 24, 4 beyond.
//  * The block's T + W - 1 input values are copied straight into LDS with
//    buffer_load_dwordx4 ... lds (1 KB per wave instruction, no VGPR staging).
//    The buffer descriptor's range ends at the last valid input, so the
//    buffer unit returns zeros past it: the lecture's guard against n + W - 1,
//    done by the hardware.
//  * Every input and output is touched once, so the copies carry the
//    non-temporal hint (cache-policy bit 1, `nt`) and the 16-byte stores are
//    non-temporal: the streams do not displace other lines on their way
//    through the caches (W = 5 at QUADS = 4: 5.87 -> 6.2 TB/s).
//  * Each lane sums its four outputs from 16-byte quads of the staged span:
//    quad q holds x[o+4q .. o+4q+3], so the four values of step d come from
//    quads d/4 and d/4 + 1, and (W + 3) / 4 + 1 ds_read_b128 serve all W
//    steps.  The lanes of a pass read consecutive quads (no bank conflicts;
//    one float per step at a 16-byte lane stride conflicted 1.7 times per
//    access).  Each output adds its terms in the order d = 0, 1, ..., W-1,
//    like the definition.
#pragma once

#include "tile_common.hpp"

namespace sgemm_dev {

template <int QUADS_>
struct WindowTile {
    static constexpr int NT = 256;                 // lanes per workgroup
    static constexpr int QUADS = QUADS_;           // output quads per lane
    static constexpr int T = NT * 4 * QUADS;       // outputs per workgroup
    static constexpr int MAX_W = 1024;             // widest window supported
    static constexpr int CHUNK = 256;              // floats per direct-copy wave instruction
    // LDS floats: the T + MAX_W - 1 staged inputs, plus the last quad read
    // past a lane's window (whole quads up to o + 4 * ceil(W / 4) + 3).
    static constexpr int TILE = ((T + MAX_W + 7 + CHUNK - 1) / CHUNK) * CHUNK;
};

typedef __attribute__((address_space(3))) void lds_void_w;

// Widest windows of the 1024- and 2048-output blocks.
constexpr int kWindowQuads1Max = 8;
constexpr int kWindowQuads2Max = 24;
// Cache-policy operand of the copies: bit 1 is the non-temporal hint.
constexpr int kWindowLoadNt = 2;

template <class WT>
__device__ __forceinline__ void window_sum_body(const float* x, float* y, int64_t n, int W) {
    __shared__ __attribute__((aligned(16))) float tile[WT::TILE];

    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int64_t base = (int64_t)blockIdx.x * WT::T;

    // Inputs of this block: [base, base + T + W - 1), clipped to the n + W - 1
    // valid values; everything past the clip reads as zero.
    const int64_t valid = n + W - 1 - base;
    const int64_t span = (int64_t)WT::T + W - 1;
    const int count = (int)(valid < span ? valid : span);
    const int chunks = (WT::T + W - 1 + WT::CHUNK - 1) / WT::CHUNK;
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc((void*)(x + base), (short)0, count * 4, 0x00020000);
    for (int c = wave; c < chunks; c += WT::NT / 64)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_w*)(tile + WT::CHUNK * c), 16,
                                                 (WT::CHUNK * c + 4 * lane) * 4, 0, 0,
                                                 kWindowLoadNt);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

#pragma unroll
    for (int j = 0; j < WT::QUADS; ++j) {
        const int o = 4 * tid + WT::NT * 4 * j;  // first output of this quad, in the block
        if (base + o >= n) break;
        const f32x4* const t = (const f32x4*)(tile + o);  // o is a multiple of 4
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        f32x4 cur = t[0];
        for (int q = 0; 4 * q < W; ++q) {
            const f32x4 nxt = t[q + 1];
            // Steps d = 4q + r: output i adds x[o + i + d], the element
            // r + i of the pair (cur, nxt).
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (4 * q + r < W) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] += r + i < 4 ? cur[r + i] : nxt[r + i - 4];
                }
            }
            cur = nxt;
        }
        const int64_t left = n - (base + o);
        if (left >= 4)
            __builtin_nontemporal_store((f32x4_u)acc, (f32x4_u*)(y + base + o));
        else
            stg4_masked(y + base + o, acc, (int)left);
    }
}

template <int QUADS>
__global__ __launch_bounds__(256) void window_sum_kernel(const float* x, float* y, int64_t n,
                                                         int W) {
    window_sum_body<WindowTile<QUADS>>(x, y, n, W);
}

}  // namespace sgemm_dev
