"""The work and traffic models against the numbers the pages print (CPU)."""
from fractions import Fraction

import pytest

import golden_io
from tiled_fp32_gemm_sgemm_amd import model


def test_load_count_table():
    g = golden_io.read("load_counts.txt")
    N, L, V = g["N"], g["L"], g["V"]
    assert model.untiled_input_loads(N, N, N) == g["one_output_per_thread_global"]
    assert model.register_tile_input_loads(N, N, N, V, V) == g["register_tile_only_global"]
    assert model.global_to_shared_loads(N, N, N, L, L) == g["two_level_global"]
    assert model.shared_to_register_loads(N, N, N, V, V) == g["two_level_shared_to_reg"]
    assert 4 * N * N == g["output_write_bytes"]
    num, den = model.flop_per_global_byte(N, L)
    assert Fraction(num, den) == g["flop_per_global_input_byte"]
    num, den = model.flop_per_global_byte(N, L, with_output=True)
    assert Fraction(num, den) == g["flop_per_byte_with_output"]
    # block shape of the same figure: (L/V)^2 threads, 2SL staged floats
    assert model.threads_per_block(L, L, V, V) == g["block_threads"]
    assert 2 * g["S"] * L == g["block_stage_floats"]


def test_stage_depth_cancels():
    # The global count does not depend on the stage depth when tiles are full.
    for BK in (4, 8, 16, 32):
        assert model.global_to_shared_loads(256, 256, 512, 64, 32, BK, padded=True) == \
            model.global_to_shared_loads(256, 256, 512, 64, 32)


def test_register_budget_and_block_threads():
    g = golden_io.read("register_budget.txt")
    for m, n, no_pf, pf in g["tile"]:
        if no_pf is not None:
            assert model.register_budget(m, n, prefetch=False) == no_pf
        assert model.register_budget(m, n, prefetch=True) == pf
    assert model.register_budget(16, 16) > g["limit"]
    for bm, bn, m, n, threads in g["block"]:
        assert model.threads_per_block(bm, bn, m, n) == threads


def test_launch_arithmetic():
    g = golden_io.read("launch.txt")
    blocks = model.ceil_div(g["n"], g["T"])
    assert blocks == g["blocks"]
    assert blocks * g["T"] - g["n"] == g["idle_threads"]


def test_issue_slot_efficiency_trace():
    # "Tiling Hierarchy on GPUs", "Eliminating Idle slots" / "Register
    # prefetching": 16 LDS + 22 idle + 64 FMA slots, then 16 + 0 + 64.
    assert round(model.issue_slot_efficiency(64, 16, 22), 2) == 0.63
    assert model.issue_slot_efficiency(64, 16, 0) == 0.8


def test_flops_and_bytes():
    assert model.flops(4096, 4096, 4096) == 137438953472
    assert model.compulsory_bytes(4096, 4096, 4096) == 3 * 4 * 4096 * 4096
    assert model.flops(128, 128, 128, batch=1024) == 2 * 128 ** 3 * 1024


@pytest.mark.parametrize("MI,kstep", [(32, 2), (16, 4)])
def test_mfma_instruction_closed_form(MI, kstep):
    # Full tiles: one instruction per MI x MI x kstep block of the product.
    M = N = K = 1024
    assert model.mfma_instructions(M, N, K, 256, 128, 16, MI) == M * N * K // (MI * MI * kstep)
    # Ragged: padded tiles are issued too.
    assert model.mfma_instructions(100, 100, 10, 64, 64, 16, MI) == \
        4 * (64 // MI) ** 2 * (16 // kstep)


def test_valu_fma_closed_form():
    assert model.valu_fma_instructions(1024, 1024, 1024) == 1024 ** 3 // 64


def test_per_xcd_panel_bytes_closed_forms():
    """4096^3 on 256 x 256 tiles: 256 tiles, 32 per XCD in one round, which in
    the grouped order (8 tile rows per group) are 8 tile rows x 4 tile columns;
    each XCD fetches 8 A panels and 4 B panels of 256 x 4096 floats."""
    panel = 256 * 4096 * 4
    assert model.per_xcd_operand_bytes(4096, 4096, 4096, 256, 256, resident=32) == \
        8 * (8 + 4) * panel
    # One XCD holding every tile in one round: each panel once (compulsory A + B).
    assert model.per_xcd_operand_bytes(4096, 4096, 4096, 256, 256, xcds=1) == \
        4 * (2 * 4096 * 4096)
    # 16384 x 4096 x 4096: 128 tiles per XCD in 4 rounds of 32; every round
    # re-reads the XCD's 8 A panels and reads 4 new B panels.
    assert model.per_xcd_operand_bytes(16384, 4096, 4096, 256, 256, resident=32) == \
        8 * 4 * (8 + 4) * panel
    # Independent products of a batch share nothing: A and B once each.
    assert model.per_xcd_operand_bytes(128, 128, 128, 128, 128, batch=1024, resident=128) == \
        1024 * 2 * 128 * 128 * 4
    # Ragged edges count only the rows and columns that exist.
    assert model.per_xcd_operand_bytes(100, 70, 10, 64, 64, xcds=1) == 4 * (100 * 10 + 70 * 10)


def test_grouped_order_and_xcd_runs():
    assert model.xcd_of_blocks(20, 8) == [(0, 3), (3, 3), (6, 3), (9, 3), (12, 2), (14, 2),
                                          (16, 2), (18, 2)]
    # group of 8 tile rows: the tile row varies fastest
    assert [model.grouped_tile(p, 16, 16, 8) for p in (0, 1, 7, 8, 127, 128)] == \
        [(0, 0), (1, 0), (7, 0), (0, 1), (7, 15), (8, 0)]
    # a last group shorter than group_m
    assert model.grouped_tile(130, 10, 16, 8) == (8, 1)


def test_convolution_useful_flops_by_brute_force():
    """Taps on the zero padding are left out of the useful count: checked by
    counting, output by output, the input pixels each filter tap lands on."""
    from workloads import ConvWorkload
    for (H, W, R, S, pad, stride, dil) in [(14, 14, 3, 3, (1, 1), (1, 1), (1, 1)),
                                           (9, 7, 3, 2, (2, 0), (2, 1), (1, 2)),
                                           (5, 6, 1, 1, (0, 0), (1, 1), (1, 1))]:
        w = ConvWorkload("t", 2, H, W, 3, 4, R, S, pad, stride, dil, 0)
        P, Q = w.out_hw
        n = 0
        for p in range(P):
            for q in range(Q):
                for r in range(R):
                    for s in range(S):
                        ih = p * stride[0] - pad[0] + r * dil[0]
                        iw = q * stride[1] - pad[1] + s * dil[1]
                        n += 0 <= ih < H and 0 <= iw < W
        assert w.useful_flops == 2 * w.N * w.K * w.C * n
        assert w.useful_flops <= w.flops
    # 14 x 14, 3 x 3, pad 1: 40 of 42 taps per axis land inside, 1600 / 1764.
    w = ConvWorkload("t", 64, 14, 14, 256, 256, 3, 3, (1, 1), (1, 1), (1, 1), 0)
    assert w.useful_flops * 1764 == w.flops * 1600


def test_l2_read_requests_by_enumeration():
    # Whole-line, line-aligned row pieces: the count is the staged bytes / 128.
    for (M, N, K, BM, BN, BK) in ((4096, 4096, 4096, 256, 256, 32), (512, 512, 1024, 64, 64, 128)):
        staged = model.global_to_shared_loads(M, N, K, BM, BN, BK, padded=True)
        assert model.l2_read_requests(M, N, K, BM, BN, BK) * 128 == 4 * staged

    # Brute force: the set of 128-byte lines holding each valid element a
    # tile reads, per tile and slice, A and B separately.
    def enumerate_requests(M, N, K, BM, BN, BK, batch, lda, ldb):
        total = 0
        for tm in range(-(-M // BM)):
            for tn in range(-(-N // BN)):
                for k0 in range(0, K, BK):
                    ks = range(k0, min(k0 + BK, K))
                    for r in range(tm * BM, min(tm * BM + BM, M)):
                        total += len({(4 * (r * lda + k)) // 128 for k in ks})
                    for k in ks:
                        total += len({(4 * (k * ldb + n)) // 128
                                      for n in range(tn * BN, min(tn * BN + BN, N))})
        return total * batch
    for shape in ((128, 128, 128, 128, 128, 16, 3, 128, 128), (70, 90, 50, 32, 64, 16, 1, 53, 97),
                  (65, 33, 40, 64, 32, 32, 2, 43, 35), (40, 64, 200, 32, 32, 64, 1, 203, 67)):
        assert model.l2_read_requests(*shape) == enumerate_requests(*shape), shape
    # The batched 1024 x 128^3 product on 128 x 128 x 16 tiles: 1.5 requests
    # per 128 staged bytes (A rows of 64 bytes).
    staged = model.global_to_shared_loads(128, 128, 128, 128, 128, 16, padded=True) * 1024
    assert Fraction(model.l2_read_requests(128, 128, 128, 128, 128, 16, 1024) * 128,
                    4 * staged) == Fraction(3, 2)
