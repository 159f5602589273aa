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
