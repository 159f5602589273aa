"""GPU parity of the general form with a split reduction (sgemm_ex_splitk).

C = alpha op(A) op(B) + beta C with the k range cut into chunks whose partial
tiles join inside the launch, in chunk order; the joining workgroup applies
alpha and beta.  Inputs are small integers and the scalars dyadic, so every
partial sum is exact and the result must equal the oracle's general form bit
for bit, for every tile, layout and chunk count.  C's row padding and a guard
after it hold a sentinel that must come back unchanged, A's and B's padding
is NaN, and after every call the workspace's per-tile counters must be zero
again.  The race-check build (NaN-filled LDS, tiles in reverse order) runs
every tile and layout once more.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import parity
from workloads import matrix, stored_operands

import tiled_fp32_gemm_sgemm_amd as sg
from tiled_fp32_gemm_sgemm_amd import _native

pytestmark = pytest.mark.gpu

SENTINEL = -7.25
GUARD = 257
LAYOUTS = [(0, 0), (1, 0), (0, 1), (1, 1)]
LAYOUT_IDS = ["nn", "tn", "nt", "tt"]
GSK_CONFIGS = [c for c in range(sg.num_configs()) if sg.config_has_general_splitk(c)]


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _case(tA, tB, M, N, K, seed, pads=(3, 1, 5)):
    lda = (M if tA else K) + pads[0]
    ldb = (K if tB else N) + pads[1]
    ldc = N + pads[2]
    A, B = stored_operands(bool(tA), bool(tB), M, N, K, lda, ldb, seed, "int4")
    C = matrix(M, N, ldc, seed + 1, "int4")
    return lda, ldb, ldc, A, B, C


def run_ex_splitk(tA, tB, M, N, K, alpha, A_cpu, lda, B_cpu, ldb, beta, C_cpu, ldc, config,
                  splits, ws=None, lib=None, expect=0):
    """One call; returns (C window, workspace, plan).  With expect != 0 the
    call must fail with that status and leave C untouched."""
    dev = _dev()
    lib = lib or _native.lib()
    A, B = A_cpu.to(dev), B_cpu.to(dev)
    Ch0 = torch.full((M * ldc + GUARD,), SENTINEL, dtype=torch.float32)
    Ch0[:C_cpu.numel()] = torch.where(torch.isnan(C_cpu), torch.tensor(SENTINEL), C_cpu)
    C = Ch0.to(dev)
    plan_cfg, plan_splits = ctypes.c_int(), ctypes.c_int64()
    nbytes = lib.sgemm_ex_splitk_plan(config, tA, tB, M, N, K, splits, ctypes.byref(plan_cfg),
                                      ctypes.byref(plan_splits))
    if expect == 0:
        assert nbytes >= 0, sg.status_string(int(nbytes))
    if ws is None:
        ws = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ws_bytes = ws.numel()
    st = lib.sgemm_ex_splitk(config, tA, tB, M, N, K, alpha, A.data_ptr(), lda, B.data_ptr(),
                             ldb, beta, C.data_ptr(), ldc, splits, ws.data_ptr(), ws_bytes,
                             stream)
    torch.cuda.synchronize()
    Ch = C.cpu().numpy()
    if expect != 0:
        assert st == expect, sg.status_string(st)
        assert np.array_equal(Ch, Ch0.numpy()), "a failed call wrote C"
        return None, ws, None
    assert st == 0, sg.status_string(st)
    idx = np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
    written = np.zeros(Ch.size, dtype=bool)
    written[idx] = True
    assert np.all(Ch[~written] == SENTINEL), "C written outside its M x N window"
    if plan_splits.value > 1:
        assert torch.count_nonzero(ws[:sg.SPLITK_HEADER_BYTES]).item() == 0, "counters not reset"
    return Ch[idx], ws, (plan_cfg.value, plan_splits.value)


def _ref(tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    ref, _, _ = oracle.sgemm_ex_f64(bool(tA), bool(tB), M, N, K, alpha, A.numpy(), lda,
                                    B.numpy(), ldb, beta, C.numpy(), ldc)
    return ref


def test_general_splitk_configs_exist():
    assert len(GSK_CONFIGS) >= 4
    for c in GSK_CONFIGS:
        assert sg.config_has_general_form(c) and sg.config_has_splitk(c)


# Ragged edges, partial last slices, chunks that do not divide K evenly.
SHAPES = [(257, 129, 1000), (64, 640, 513), (130, 70, 3001)]


@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("config", GSK_CONFIGS, ids=lambda c: "cfg%d" % c)
def test_ex_splitk_every_tile_bitwise(config, layout):
    tA, tB = layout
    # One workspace, zeroed once, for every call of the test.
    need = max(sg.ex_splitk_plan(M, N, K, tA, tB, splits, config)[2]
               for (M, N, K) in SHAPES for splits in (2, 3, 7))
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=_dev())
    for i, (M, N, K) in enumerate(SHAPES):
        for splits, (alpha, beta) in [(2, (2.0, -1.0)), (3, (1.0, 0.0)), (7, (-0.5, 0.25))]:
            lda, ldb, ldc, A, B, C = _case(tA, tB, M, N, K, 100 * config + 10 * i + splits)
            got, ws, plan = run_ex_splitk(tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                          config, splits, ws)
            assert plan[0] == config
            ref = _ref(tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
            parity.assert_bitwise(got, ref, "ex_splitk cfg%d %s %s S=%d a%g b%g"
                                  % (config, layout, (M, N, K), splits, alpha, beta))


# Thin long-K products and a grid with a partial last layer (hybrid plans),
# with the time model's tile and chunk count.
AUTO_SHAPES = [(512, 512, 8192), (128, 1024, 4096), (1088, 1024, 1024), (256, 4096, 2048)]


@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("shape", AUTO_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ex_splitk_auto_plan_bitwise(shape, layout):
    tA, tB = layout
    M, N, K = shape
    lda, ldb, ldc, A, B, C = _case(tA, tB, M, N, K, M + N + K + tA + 2 * tB, pads=(0, 0, 0))
    got, _, plan = run_ex_splitk(tA, tB, M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, -1, 0)
    ref = _ref(tA, tB, M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc)
    parity.assert_bitwise(got, ref, "ex_splitk auto %s %s plan %s" % (shape, layout, plan))
    if shape[2] >= 4096:
        assert plan[1] > 1, "a thin long-K product should split: plan %s" % (plan,)


def test_ex_splitk_uniform_tolerance_and_repeatable():
    M, N, K = 300, 200, 5000
    lda, ldb, ldc = M, K, N
    A, B = stored_operands(True, True, M, N, K, lda, ldb, 77, "uniform")
    C = matrix(M, N, ldc, 78, "uniform")
    got1, ws, _ = run_ex_splitk(1, 1, M, N, K, 0.75, A, lda, B, ldb, -1.5, C, ldc, -1, 5)
    got2, _, _ = run_ex_splitk(1, 1, M, N, K, 0.75, A, lda, B, ldb, -1.5, C, ldc, -1, 5, ws)
    assert np.array_equal(got1.view(np.uint32), got2.view(np.uint32)), "join order not fixed"
    ref, mag, _ = oracle.sgemm_ex_f64(True, True, M, N, K, 0.75, A.numpy(), lda, B.numpy(), ldb,
                                      -1.5, C.numpy(), ldc)
    parity.assert_within_tolerance(got1, ref, mag, "ex_splitk uniform")


def test_ex_splitk_alpha_zero_and_k_zero_scale_c():
    M, N = 70, 90
    for K, alpha in [(0, 1.0), (50, 0.0)]:
        lda, ldb, ldc, A, B, C = _case(0, 0, M, N, max(K, 1), 5)
        got, _, _ = run_ex_splitk(0, 0, M, N, K, alpha, A, lda, B, ldb, -2.0, C, ldc, -1, 4)
        want = -2.0 * C.view(-1)[: M * ldc].view(M, ldc)[:, :N].numpy()
        assert np.array_equal(got, want)


def test_ex_splitk_errors_enqueue_nothing():
    M, N, K = 64, 64, 512
    lda, ldb, ldc, A, B, C = _case(0, 0, M, N, K, 9)
    no_gsk = [c for c in range(sg.num_configs()) if not sg.config_has_general_splitk(c)][0]
    run_ex_splitk(0, 0, M, N, K, 1.0, A, lda, B, ldb, 1.0, C, ldc, no_gsk, 2,
                  expect=_status("SGEMM_STATUS_INVALID_CONFIG"))
    small = torch.zeros(256, dtype=torch.uint8, device=_dev())
    run_ex_splitk(0, 0, M, N, K, 1.0, A, lda, B, ldb, 1.0, C, ldc, GSK_CONFIGS[0], 4, small,
                  expect=_status("SGEMM_STATUS_INVALID_WORKSPACE"))
    run_ex_splitk(2, 0, M, N, K, 1.0, A, lda, B, ldb, 1.0, C, ldc, -1, 0,
                  expect=_status("SGEMM_STATUS_INVALID_OP"))


def _status(name):
    codes = {"SGEMM_STATUS_INVALID_CONFIG": -7, "SGEMM_STATUS_INVALID_OP": -8,
             "SGEMM_STATUS_INVALID_WORKSPACE": -9}
    return codes[name]


def test_ex_splitk_tensor_api_shares_the_default_workspace():
    dev = _dev()
    g = torch.Generator("cpu").manual_seed(3)
    At = torch.randint(-4, 5, (4096, 300), generator=g).float()   # stored K x M
    B = torch.randint(-4, 5, (4096, 200), generator=g).float()    # stored K x N
    C = torch.randint(-4, 5, (300, 200), generator=g).float()
    out = sg.sgemm_ex_splitk(At.to(dev), B.to(dev), C.to(dev), alpha=2.0, beta=-1.0,
                             transA=True)
    ref = 2.0 * (At.double().T @ B.double()) - C.double()
    assert torch.equal(out.cpu().double(), ref)
    # The plain split-K call on the same stream reuses that workspace.
    A2 = torch.randint(-4, 5, (200, 3000), generator=g).float()
    B2 = torch.randint(-4, 5, (3000, 100), generator=g).float()
    out2 = sg.sgemm_splitk(A2.to(dev), B2.to(dev), splits=6)
    assert torch.equal(out2.cpu().double(), A2.double() @ B2.double())
    out3 = sg.sgemm_ex_splitk(At.to(dev), B.to(dev), C.to(dev), alpha=2.0, beta=-1.0,
                              transA=True, splits=9)
    assert torch.equal(out3.cpu().double(), ref)


@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("config", GSK_CONFIGS, ids=lambda c: "cfg%d" % c)
def test_ex_splitk_racecheck(config, layout):
    tA, tB = layout
    M, N, K = 257, 129, 1000
    lda, ldb, ldc, A, B, C = _case(tA, tB, M, N, K, 7 * config + tA + 2 * tB)
    got, _, _ = run_ex_splitk(tA, tB, M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, config, 3,
                              lib=_native.racecheck_lib())
    ref = _ref(tA, tB, M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc)
    parity.assert_bitwise(got, ref, "racecheck ex_splitk cfg%d %s" % (config, layout))
