"""GPU parity of sgemm_splitk_noalloc, the split-K entry point that takes its
workspace from the library's own per-GPU buffer instead of the caller.

Its output must equal sgemm_splitk's (the entry point with a caller-supplied
workspace) bit for bit for the same tile and chunk count, and the oracle's:
bit for bit on integer-valued inputs, within 2e-4 * (|A||B|)_ij otherwise.
Calls follow each other on one GPU, the second one smaller than the first, so
the buffer is reused with another tile count and chunk count.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import parity
from workloads import operands

import tiled_fp32_gemm_sgemm_amd as sg
from tiled_fp32_gemm_sgemm_amd import _native

pytestmark = pytest.mark.gpu

SENTINEL = -7.25
GUARD = 129
SCRATCH_BYTES = 64 * 1024 * 1024


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _call(entry, M, N, K, A, lda, B, ldb, ldc, config, splits):
    """One call through the C ABI; returns C's M x N window (host)."""
    dev = _dev()
    lib = _native.lib()
    C = torch.full((M * ldc + GUARD,), SENTINEL, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if entry == "noalloc":
        st = lib.sgemm_splitk_noalloc(config, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                                      C.data_ptr(), ldc, splits, stream)
    else:
        nbytes = sg.splitk_plan(M, N, K, splits, None if config < 0 else config)[2]
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
        st = lib.sgemm_splitk(config, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                              C.data_ptr(), ldc, splits, ws.data_ptr(), ws.numel(), stream)
    assert st == 0, "%s: %s" % (entry, sg.status_string(st))
    torch.cuda.synchronize()
    Ch = C.cpu().numpy()
    idx = np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
    written = np.zeros(Ch.size, dtype=bool)
    written[idx] = True
    assert np.all(Ch[~written] == SENTINEL), "%s wrote outside C's window" % entry
    return Ch[idx]


# (M, N, K, lda, ldb, ldc, splits): the first call larger than the second,
# ragged edges and odd leading dimensions; 0 = the time model's chunk count.
CALLS = [(300, 520, 6000, 6003, 523, 525, 0),
         (130, 70, 3001, 3003, 70, 75, 5)]


@pytest.mark.parametrize("dist", ["int4", "uniform"])
def test_noalloc_matches_workspace_entry_point(dist):
    dev = _dev()
    for i, (M, N, K, lda, ldb, ldc, splits) in enumerate(CALLS):
        cfg, used, nbytes = sg.splitk_plan(M, N, K, splits)
        assert used > 1 and nbytes <= SCRATCH_BYTES, (cfg, used, nbytes)
        A_cpu, B_cpu = operands(M, N, K, lda, ldb, seed=700 + i, dist_a=dist)
        A, B = A_cpu.to(dev), B_cpu.to(dev)
        got = _call("noalloc", M, N, K, A, lda, B, ldb, ldc, -1, splits)
        want = _call("workspace", M, N, K, A, lda, B, ldb, ldc, cfg, used)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
            "call %d: the two entry points differ" % i
        ref, mag, _ = oracle.sgemm_f64(M, N, K, A_cpu.numpy(), lda, B_cpu.numpy(), ldb)
        what = "noalloc call %d %s" % (i, (M, N, K, cfg, used))
        if dist == "int4":
            parity.assert_bitwise(got, ref, what)
        else:
            parity.assert_within_tolerance(got, ref, mag, what)


def test_noalloc_every_splitk_tile_in_turn():
    """Each tile with a split-K variant, at 3 chunks, one call after another
    on the shared buffer; integer inputs, bit-exact."""
    dev = _dev()
    M, N, K, lda, ldb, ldc = 257, 129, 1000, 1003, 131, 133
    A_cpu, B_cpu = operands(M, N, K, lda, ldb, seed=71, dist_a="int4")
    A, B = A_cpu.to(dev), B_cpu.to(dev)
    ref, _, _ = oracle.sgemm_f64(M, N, K, A_cpu.numpy(), lda, B_cpu.numpy(), ldb)
    for config in [c for c in range(sg.num_configs()) if sg.config_has_splitk(c)]:
        got = _call("noalloc", M, N, K, A, lda, B, ldb, ldc, config, 3)
        parity.assert_bitwise(got, ref, "noalloc cfg%d" % config)


def test_noalloc_rejects_plans_beyond_the_buffer():
    dev = _dev()
    cfg = [c for c in range(sg.num_configs()) if sg.config_has_splitk(c)][0]
    M = N = 4096
    K = 8192
    assert sg.splitk_plan(M, N, K, 8, cfg)[2] > SCRATCH_BYTES
    C = torch.full((GUARD,), SENTINEL, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    st = _native.lib().sgemm_splitk_noalloc(cfg, M, N, K, C.data_ptr(), K, C.data_ptr(), N,
                                            C.data_ptr(), N, 8, stream)
    assert st == -10, sg.status_string(st)
    torch.cuda.synchronize()
    assert torch.all(C == SENTINEL)


def test_noalloc_in_a_captured_graph():
    """The callers it is for: two split-K products captured in a HIP graph with
    no allocation in the graph, replayed three times with eager calls of the
    same entry point on other shapes in between (one stream, so no overlap);
    every replay equals the eager results bit for bit."""
    dev = _dev()
    gen = torch.Generator(device=dev).manual_seed(23)
    A1 = torch.randn(200, 3000, device=dev, generator=gen)
    B1 = torch.randn(3000, 150, device=dev, generator=gen)
    A2 = torch.randn(64, 5000, device=dev, generator=gen)
    B2 = torch.randn(5000, 96, device=dev, generator=gen)
    A3 = torch.randn(130, 2000, device=dev, generator=gen)
    B3 = torch.randn(2000, 70, device=dev, generator=gen)
    C1 = torch.empty(200, 150, device=dev)
    C2 = torch.empty(64, 96, device=dev)
    C3 = torch.empty(130, 70, device=dev)
    assert sg.splitk_plan(200, 150, 3000, 6)[1] > 1 and sg.splitk_plan(64, 96, 5000, 4)[1] > 1

    def calls():
        sg.sgemm_splitk_noalloc(A1, B1, C1, splits=6)
        sg.sgemm_splitk_noalloc(A2, B2, C2, splits=4)

    calls()  # eager first: the buffer's address is looked up outside capture
    torch.cuda.synchronize()
    ref = [C1.clone(), C2.clone()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for r in range(3):
        C1.fill_(float("nan"))
        C2.fill_(float("nan"))
        sg.sgemm_splitk_noalloc(A3, B3, C3, splits=5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((C1, C2), ref):
            assert torch.equal(got.view(torch.int32), want.view(torch.int32)), "replay %d" % r
