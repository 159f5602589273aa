"""Seeded random shapes through the automatic choices (MI355X) against the oracle.

The named workloads and the hand-picked ragged shapes each land on a few tiles;
these shapes, drawn log-uniformly, let the time model pick whatever it picks
(the plain product's tile, the split-K plan, hybrid or not, the general
form's tile and the general form's split plan), with leading dimensions past
the row length.  Inputs are small
integers and the scalars dyadic, so every result is exact and unique, and the
comparison is bit for bit.  Padding in A and B is NaN; C's padding and a guard
past it hold a sentinel that must come back unchanged.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import parity
import tiled_fp32_gemm_sgemm_amd as sg
from tiled_fp32_gemm_sgemm_amd import _native
from workloads import matrix, operands, stored_operands

pytestmark = pytest.mark.gpu

SENTINEL = -7.25
GUARD = 257


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _draw_cases(n, seed):
    r = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M, N = (int(np.exp(r.uniform(np.log(8.0), np.log(2048.0)))) for _ in range(2))
        K = int(np.exp(r.uniform(0.0, np.log(4096.0))))
        pads = r.integers(0, 6, 3)
        layout = (int(r.integers(0, 2)), int(r.integers(0, 2)))
        alpha = float(r.choice([1.0, 2.0, -0.5]))
        beta = float(r.choice([0.0, 1.0, -1.0, 0.25]))
        cases.append((i, M, N, K, int(pads[0]), int(pads[1]), int(pads[2]), layout, alpha, beta))
    return cases


CASES = _draw_cases(96, 20261202)
IDS = ["%dx%dx%d" % (c[1], c[2], c[3]) for c in CASES]


def _c_buffer(M, ldc, dev, init=None):
    C = torch.full((M * ldc + GUARD,), SENTINEL, dtype=torch.float32)
    if init is not None:
        C[: init.numel()] = torch.where(torch.isnan(init), torch.tensor(SENTINEL), init)
    return C.to(dev)


def _window(C, M, N, ldc):
    Ch = C.cpu().numpy()
    idx = np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
    written = np.zeros(Ch.size, dtype=bool)
    written[idx] = True
    assert np.all(Ch[~written] == SENTINEL), "C written outside its M x N window"
    return Ch[idx]


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_random_shape_plain_and_splitk(case):
    i, M, N, K, pa, pb, pc, _, _, _ = case
    dev = _dev()
    lda, ldb, ldc = K + pa, N + pb, N + pc
    A_cpu, B_cpu = operands(M, N, K, lda, ldb, 1000 + i, "int4")
    ref, _, _ = oracle.sgemm_f64(M, N, K, A_cpu.numpy(), lda, B_cpu.numpy(), ldb)
    A, B = A_cpu.to(dev), B_cpu.to(dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    # The plain product, tile chosen by the time model.
    C = _c_buffer(M, ldc, dev)
    st = sg.sgemm_raw(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc, stream)
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    parity.assert_bitwise(_window(C, M, N, ldc), ref, "sgemm %dx%dx%d" % (M, N, K))
    # Split-K with the automatic plan (which may keep the plain kernel, split
    # every tile, or split only the last partial layer).
    lib = _native.lib()
    plan_cfg, plan_splits = ctypes.c_int(), ctypes.c_int64()
    nbytes = lib.sgemm_splitk_plan(-1, M, N, K, 0, ctypes.byref(plan_cfg),
                                   ctypes.byref(plan_splits))
    assert nbytes >= 0, sg.status_string(int(nbytes))
    ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
    C = _c_buffer(M, ldc, dev)
    st = lib.sgemm_splitk(-1, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc,
                          0, ws.data_ptr(), ws.numel(), ctypes.c_void_p(stream))
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    parity.assert_bitwise(_window(C, M, N, ldc), ref,
                          "splitk %dx%dx%d plan %s" % (M, N, K, (plan_cfg.value,
                                                                 plan_splits.value)))
    if plan_splits.value > 1:
        assert torch.count_nonzero(ws[:sg.SPLITK_HEADER_BYTES]).item() == 0, "counters not reset"


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_random_shape_general(case):
    i, M, N, K, pa, pb, pc, (tA, tB), alpha, beta = case
    dev = _dev()
    lda = (M if tA else K) + pa
    ldb = (K if tB else N) + pb
    ldc = N + pc
    A_cpu, B_cpu = stored_operands(bool(tA), bool(tB), M, N, K, lda, ldb, 2000 + i, "int4")
    C_cpu = matrix(M, N, ldc, 3000 + i, "int4")
    ref, _, _ = oracle.sgemm_ex_f64(bool(tA), bool(tB), M, N, K, alpha, A_cpu.numpy(), lda,
                                    B_cpu.numpy(), ldb, beta, C_cpu.numpy(), ldc)
    A, B = A_cpu.to(dev), B_cpu.to(dev)
    C = _c_buffer(M, ldc, dev, C_cpu)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = sg.sgemm_ex_raw(tA, tB, M, N, K, alpha, A.data_ptr(), lda, B.data_ptr(), ldb, beta,
                         C.data_ptr(), ldc, stream)
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    parity.assert_bitwise(_window(C, M, N, ldc), ref,
                          "ex %dx%dx%d t%d%d a%g b%g" % (M, N, K, tA, tB, alpha, beta))


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_random_shape_general_splitk(case):
    """The general form split over k with the automatic plan (which may keep
    the unsplit general form), on the same shapes, layouts and scalars."""
    i, M, N, K, pa, pb, pc, (tA, tB), alpha, beta = case
    dev = _dev()
    lda = (M if tA else K) + pa
    ldb = (K if tB else N) + pb
    ldc = N + pc
    A_cpu, B_cpu = stored_operands(bool(tA), bool(tB), M, N, K, lda, ldb, 4000 + i, "int4")
    C_cpu = matrix(M, N, ldc, 5000 + i, "int4")
    ref, _, _ = oracle.sgemm_ex_f64(bool(tA), bool(tB), M, N, K, alpha, A_cpu.numpy(), lda,
                                    B_cpu.numpy(), ldb, beta, C_cpu.numpy(), ldc)
    A, B = A_cpu.to(dev), B_cpu.to(dev)
    C = _c_buffer(M, ldc, dev, C_cpu)
    cfg, splits, nbytes = sg.ex_splitk_plan(M, N, K, bool(tA), bool(tB))
    ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = sg.sgemm_ex_splitk_raw(tA, tB, M, N, K, alpha, A.data_ptr(), lda, B.data_ptr(), ldb,
                                beta, C.data_ptr(), ldc, ws.data_ptr(), ws.numel(), stream)
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    parity.assert_bitwise(_window(C, M, N, ldc), ref,
                          "ex_splitk %dx%dx%d t%d%d a%g b%g plan %s"
                          % (M, N, K, tA, tB, alpha, beta, (cfg, splits)))
    if splits > 1:
        assert torch.count_nonzero(ws[:sg.SPLITK_HEADER_BYTES]).item() == 0, "counters not reset"
