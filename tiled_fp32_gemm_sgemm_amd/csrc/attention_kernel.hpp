// Blockwise attention on the gfx950 matrix cores: O = softmax(scale Q K^T) V
// per head, FP32, forward only ("Tiling Strategies" section 5, the
// FlashAttention row of the tiling-beyond-GEMM table: Q, K and V are tiled
// along the sequence and each K/V block is reused by every query row of the
// workgroup; the softmax is kept online, so the Sq x Skv score matrix never
// leaves registers).
//
// Work split.  One workgroup per (head, block of BQ = 32 * NW queries); wave w
// owns 32 queries and keeps them for the whole pass.  Keys and values stream
// through LDS in blocks of BKV = 64 rows, two blocks in flight, copied by
// buffer_load_dwordx4 ... lds (no VGPR staging; rows past Skv read as zeros
// because the buffer descriptor's range ends at the last key).
//
// Scores, transposed.  With v_mfma_f32_32x32x2_f32 the accumulator rows are
// spread over a lane's registers and lane groups and the columns over lanes,
// so the product is formed as S^T = K Q^T: lane (j, g) (j = lane % 32,
// g = lane / 32) then holds, for its own query j, the scores of 16 of every
// 32 keys, the other 16 sitting in lane j ^ 32; a row maximum or sum is a
// register loop plus one cross-lane exchange.  The reduction over d is split
// between the lane groups (g takes d = g*D/2 + kk), so each lane's Q values are
// D/2 consecutive floats, loaded once into registers.
//
// Values.  O^T = V^T P^T: the B operand of step (n, r) is the lane's own
// probability register P^T[32n + row(r, g)][j], so the key order of that
// product is the register order (a permutation of the sum); the A operand is
// V[32n + row(r, g)][d] for the lane's d values, with the output rows
// interleaved (d = DT * i + t for tile t, lane row i) so that one ds_read of DT
// floats serves all DT tiles.
//
// Online softmax, in base 2: Q is scaled by scale * log2(e) as it is loaded,
// so the products are base-2 scores; per block, m_new = max(m, block max),
// alpha = 2^(m - m_new), p = 2^(s - m_new), l = alpha l + sum p,
// O = alpha O + P V; at the end O / l.
//
// LDS layouts.  K block [key][d] with quad q of row R stored at q ^ (R % 16):
// the 16 lanes of a ds_read_b128 pass read one logical quad of 16 consecutive
// keys and hit 16 different bank quads.  V block [key][d] as stored: a pass
// reads one key row contiguously.
#pragma once

#include "mfma_dl_kernel.hpp"
#include "tile_common.hpp"

namespace sgemm_dev {

constexpr int kHeadsPerGroup = 8;

struct AttnArgs {
    const float* Q;
    const float* K;
    const float* V;
    float* O;
    int64_t BH;        // heads
    int Sq, Skv;
    int q_blocks;      // ceil(Sq / BQ)
    float scale_log2;  // scale * log2(e)
};

template <int D_, bool CAUSAL_>
struct AttnTile {
    static constexpr int D = D_;
    static constexpr bool CAUSAL = CAUSAL_;  // key j allowed for query i only when j <= i
    static constexpr int NW = 8, NT = 64 * NW;
    static constexpr int BQ = 32 * NW;       // queries per workgroup
    static constexpr int BKV = 64;           // keys per block
    static constexpr int HALF = D / 2;       // d values per lane group in the score product
    static constexpr int DT = D / 32;        // 32-row tiles of O^T
    static constexpr int OP = DT >= 4 ? 1 : 4 / DT;  // partial O accumulators (>= 4 chains)
    static constexpr int QPR = D / 4;        // 16-byte quads per K or V row
    static constexpr int BLK = BKV * D;      // floats per K (or V) block
    static constexpr int STAGE = 2 * BLK;    // K block, then V block
    static constexpr int CHW = BLK / 256 / NW;  // 1 KB copies per wave per block
    static constexpr int LDS_BYTES = 2 * STAGE * 4;
    static_assert(D == 64 || D == 128, "head dimension");
    static_assert(BLK % (256 * NW) == 0, "block copies split over the waves");
    static_assert(QPR % 16 == 0, "K rows span whole 64-bank rows");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <class T>
__device__ __forceinline__ void attention_body(const AttnArgs& a) {
    using Op = MfmaOp<32>;
    typedef float dvec_t __attribute__((ext_vector_type(T::DT)));
    typedef float dvec_u __attribute__((ext_vector_type(T::DT), aligned(4)));
    __shared__ __attribute__((aligned(16))) float smem[2 * T::STAGE];

    // Workgroup -> (head, query block).  Consecutive ids run on one XCD, so a
    // group of up to 8 heads shares that XCD's L2 for its keys and values.
    // Inside a group the query blocks come last-first: with the causal mask a
    // block's work grows with its index, and handing the longest jobs out
    // first (the longest-processing-time rule) keeps the CUs' finishing times
    // together.  Without the mask every block has the same work.
    const uint32_t pid = xcd_contiguous_id(kRaceCheck ? gridDim.x - 1 - blockIdx.x : blockIdx.x,
                                           gridDim.x);
    const uint32_t per_group = (uint32_t)(kHeadsPerGroup * a.q_blocks);
    const uint32_t hg = pid / per_group;
    const uint32_t l = pid - hg * per_group;
    const uint32_t in_group =
        (uint32_t)min((int64_t)kHeadsPerGroup, a.BH - (int64_t)hg * kHeadsPerGroup);
    const int64_t h = (int64_t)hg * kHeadsPerGroup + l % in_group;
    const int qb = a.q_blocks - 1 - (int)(l / in_group);
    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int j = lane % 32;
    const int g = lane / 32;
    // Wave w takes the 32-query row group w for w < NW/2 and NW-1-(w-NW/2)
    // above: waves w and w + NW/2 usually share a SIMD, and under the causal
    // mask each such pair then holds one early and one late row group, so the
    // SIMDs carry equal work on the diagonal blocks.
    const int wrow = wave < T::NW / 2 ? wave : 3 * T::NW / 2 - 1 - wave;
    const int q_first = qb * T::BQ + 32 * wrow;  // the wave's first query
    const int qi = q_first + j;                  // this lane's query
    const int64_t q_org = uniform_i64(h * (int64_t)a.Sq * T::D);
    const int64_t kv_org = uniform_i64(h * (int64_t)a.Skv * T::D);

    // Key blocks this workgroup needs (causal: none past its last query), and
    // the ones this wave computes (causal: none past the wave's last query;
    // it still copies its share of the later ones and meets the barriers).
    const int nkv = (a.Skv + T::BKV - 1) / T::BKV;
    int nb = nkv, nb_wave = nkv;
    if constexpr (T::CAUSAL) {
        const int last_q = min(a.Sq, qb * T::BQ + T::BQ) - 1;
        nb = min(nkv, last_q / T::BKV + 1);
        nb_wave = min(nb, (q_first + 31) / T::BKV + 1);
    }

    // Q in registers: lane (j, g) holds Q[qi][HALF*g + kk] * scale * log2(e),
    // kk < HALF, so the products come out as base-2 scores; zeros past Sq
    // (those rows are computed and never stored).
    float qreg[T::HALF];
    {
        const float* src = a.Q + q_org + (int64_t)qi * T::D + T::HALF * g;
#pragma unroll
        for (int c = 0; c < T::HALF / 4; ++c) {
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (qi < a.Sq) v = ldg4(src + 4 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e) qreg[4 * c + e] = v[e] * a.scale_log2;
        }
    }

    // Per-lane copy offsets (bytes from the block start), fixed for the pass.
    uint32_t k_off[T::CHW], v_off[T::CHW];
#pragma unroll
    for (int c = 0; c < T::CHW; ++c) {
        const int p = 64 * (wave * T::CHW + c) + lane;  // LDS quad this lane fills
        const int row = p / T::QPR;
        const int pq = p % T::QPR;
        k_off[c] = (uint32_t)((row * T::D + 4 * (pq ^ (row & 15))) * 4);
        v_off[c] = (uint32_t)(p * 16);
    }
    auto load_block = [&](int b, int st) {
        const int k0 = b * T::BKV;
        const int rows = min(T::BKV, a.Skv - k0);
        const int range = rows * T::D * 4;  // the descriptor ends at the last key
        const int64_t off = uniform_i64(kv_org + (int64_t)k0 * T::D);
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.K + off), (short)0, range, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.V + off), (short)0, range, 0x00020000);
        float* const dk = smem + st * T::STAGE;
        float* const dv = dk + T::BLK;
#pragma unroll
        for (int c = 0; c < T::CHW; ++c)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rk, (lds_void_t*)(dk + 256 * (wave * T::CHW + c)), 16, k_off[c], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < T::CHW; ++c)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rv, (lds_void_t*)(dv + 256 * (wave * T::CHW + c)), 16, v_off[c], 0, 0, 0);
    };

    f32x16 o_acc[T::DT][T::OP];
#pragma unroll
    for (int t = 0; t < T::DT; ++t)
#pragma unroll
        for (int u = 0; u < T::OP; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) o_acc[t][u][r] = 0.0f;
    float m_run = -__builtin_huge_valf();
    float l_run = 0.0f;

    if constexpr (kRaceCheck) {
        poison_lds(smem, 2 * T::STAGE, tid, T::NT);
        lds_barrier();
    }
    if (nb > 0) load_block(0, 0);
    wait_vmcnt<0>();
    lds_barrier();
    for (int b = 0; b < nb_wave; ++b) {
        const int st = b & 1;
        if (b + 1 < nb) load_block(b + 1, st ^ 1);
        const float* const Ks = smem + st * T::STAGE;
        const float* const Vs = Ks + T::BLK;

        // S^T = K Q^T for two 32-key tiles, each as two partial sums (the
        // four accumulators rotate, so no MFMA waits on the one before).
        f32x16 s_acc[2][2];
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int r = 0; r < 16; ++r) s_acc[n][u][r] = 0.0f;
#pragma unroll
        for (int kq = 0; kq < T::HALF / 4; ++kq) {
            f32x4 ka[2];
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int R = 32 * n + j;
                const int lq = T::HALF / 4 * g + kq;
                ka[n] = *(const f32x4*)(Ks + R * T::D + 4 * (lq ^ (R & 15)));
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    s_acc[n][s & 1] = Op::mma(ka[n][s], qreg[4 * kq + s], s_acc[n][s & 1]);
        }

        // Mask (only blocks that reach past Skv or, causal, past the wave's
        // first query can hold a disallowed key), then the online softmax.
        // Exponentials are v_exp_f32: 2^-inf = 0, and a result below the
        // normal range may come out as 0, which changes O by less than 2^-126
        // of the weighted |V|.
        const int kbase = b * T::BKV;
        const bool edge =
            kbase + T::BKV > a.Skv || (T::CAUSAL && kbase + T::BKV - 1 > q_first);
        float sv[2][16];
        float mloc = -__builtin_huge_valf();
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sv[n][r] = s_acc[n][0][r] + s_acc[n][1][r];
                if (edge) {
                    const int key = kbase + 32 * n + Op::row(r, g);
                    const bool ok = key < a.Skv && (!T::CAUSAL || key <= qi);
                    sv[n][r] = ok ? sv[n][r] : -__builtin_huge_valf();
                }
                mloc = fmaxf(mloc, sv[n][r]);
            }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float m_new = fmaxf(m_run, mloc);
        // No allowed key yet: shift by 0, every weight is 2^-inf = 0.
        const float m_use = m_new == -__builtin_huge_valf() ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float lsum = 0.0f;
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sv[n][r] = __builtin_amdgcn_exp2f(sv[n][r] - m_use);
                lsum += sv[n][r];
            }
        lsum += __shfl_xor(lsum, 32);
        l_run = l_run * alpha + lsum;
        m_run = m_new;
        // alpha is exactly 1 where the maximum did not move; skip the rescale
        // when that holds for the whole wave.
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int t = 0; t < T::DT; ++t)
#pragma unroll
                for (int u = 0; u < T::OP; ++u)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o_acc[t][u][r] *= alpha;
        }

        // O^T += V^T P^T over the block's 64 keys, in register order.
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int R = 32 * n + Op::row(r, g);
                const dvec_t va = *(const dvec_t*)(Vs + R * T::D + T::DT * j);
                const int u = (16 * n + r) % T::OP;
#pragma unroll
                for (int t = 0; t < T::DT; ++t)
                    o_acc[t][u] = Op::mma(va[t], sv[n][r], o_acc[t][u]);
            }

        // Block b + 1 has landed (this wave's copies), and every wave is done
        // with stage st before the next iteration refills it.
        wait_vmcnt<0>();
        lds_barrier();
        if constexpr (kRaceCheck) {
            poison_lds(smem + st * T::STAGE, T::STAGE, tid, T::NT);
            lds_barrier();
        }
    }
    // Causal: the blocks past this wave's queries, copies and barriers only
    // (every wave passes the same barriers as the compute loop's).
    for (int b = nb_wave; b < nb; ++b) {
        if (b + 1 < nb) load_block(b + 1, (b & 1) ^ 1);
        wait_vmcnt<0>();
        lds_barrier();
        if constexpr (kRaceCheck) {
            poison_lds(smem + (b & 1) * T::STAGE, T::STAGE, tid, T::NT);
            lds_barrier();
        }
    }

    // O[qi][DT * row(r, g) + t] = O^T / l.
    if (qi < a.Sq) {
        float* const dst = a.O + q_org + (int64_t)qi * T::D;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dvec_t v;
#pragma unroll
            for (int t = 0; t < T::DT; ++t) {
                float x = o_acc[t][0][r];
#pragma unroll
                for (int u = 1; u < T::OP; ++u) x += o_acc[t][u][r];
                v[t] = l_run > 0.0f ? x / l_run : 0.0f;
            }
            *(dvec_u*)(dst + T::DT * Op::row(r, g)) = v;
        }
    }
}

template <class T>
__global__ __launch_bounds__(T::NT) __attribute__((amdgpu_waves_per_eu(2)))
void attention_kernel(AttnArgs a) {
    attention_body<T>(a);
}

}  // namespace sgemm_dev
