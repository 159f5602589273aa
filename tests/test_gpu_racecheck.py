"""Race-sensitivity runs: the race-check build of the library against the oracle.

libsgemm_racecheck.so is the same C ABI built with SGEMM_RACECHECK=1: every
LDS buffer of the GEMM, convolution and attention kernels is filled with NaN at
the start of a workgroup and again as soon as the workgroup is done with it
(after the barrier that ends its use), and workgroups take their tiles in
reverse order.  A wave that read a slice before its copy had landed (a wait
that counts too few outstanding copies), or after its buffer had been handed
on to a later slice (a barrier in the wrong place), reads NaN, and NaN reaches
the result; so does a read of LDS that no copy writes (padding, a tail the
loader skipped).  Integer-valued inputs are compared with the oracle bit for
bit, which a NaN anywhere fails.

Every tile configuration runs shapes with several slices, ragged M, N and K
(partial last slices go through the register-staged copy) and strided batches,
plus the general form, the convolution and the attention.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import parity
from workloads import matrix, operands, stored_operands

import tiled_fp32_gemm_sgemm_amd as sg
from tiled_fp32_gemm_sgemm_amd import _native

pytestmark = pytest.mark.gpu

SENTINEL = -7.25
GUARD = 257


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _rc():
    return _native.racecheck_lib()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream(_dev()).cuda_stream)


def _windows(Ch, batch, M, N, ldc, strideC):
    written = np.zeros(Ch.size, dtype=bool)
    out = np.empty((batch, M, N), dtype=np.float32)
    for b in range(batch):
        idx = b * strideC + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
        out[b] = Ch[idx]
        written[idx] = True
    assert np.all(Ch[~written] == SENTINEL), "C written outside its M x N window(s)"
    return out


# (M, N, K, lda, ldb, ldc, batch): several slices for every BK, ragged edges,
# partial last slices, odd leading dimensions, a strided batch.
SHAPES = [(256, 256, 256, 256, 256, 256, 1),
          (257, 129, 300, 303, 131, 133, 1),
          (64, 640, 513, 515, 640, 641, 1),
          (130, 70, 1000, 1003, 70, 75, 1),
          (65, 63, 150, 151, 65, 66, 3)]
PATHS = ["valu"] + ["cfg%d" % i for i in range(34)]


def test_every_config_is_covered():
    assert sg.num_configs() == len(PATHS) - 1
    assert _rc().sgemm_num_configs() == sg.num_configs()


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_racecheck_gemm_bitwise(shape, path):
    M, N, K, lda, ldb, ldc, batch = shape
    dev = _dev()
    sa, sb, sc = M * lda + 5, K * ldb + 3, M * ldc + 7
    A_cpu, B_cpu = operands(M, N, K, lda, ldb, seed=M + 3 * N + 5 * K + batch, dist_a="int4",
                            batch=batch, strideA=sa, strideB=sb)
    A, B = A_cpu.to(dev), B_cpu.to(dev)
    c_len = (batch - 1) * sc + M * ldc
    C = torch.full((c_len + GUARD,), SENTINEL, dtype=torch.float32, device=dev)
    lib = _rc()
    if path == "valu":
        st = lib.sgemm_valu_strided_batched(M, N, K, A.data_ptr(), lda, sa, B.data_ptr(), ldb, sb,
                                            C.data_ptr(), ldc, sc, batch, _stream())
    else:
        st = lib.sgemm_with_config(int(path[3:]), M, N, K, A.data_ptr(), lda, sa, B.data_ptr(),
                                   ldb, sb, C.data_ptr(), ldc, sc, batch, _stream())
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    got = _windows(C.cpu().numpy(), batch, M, N, ldc, sc)
    for b in range(batch):
        ref, _, _ = oracle.sgemm_f64(M, N, K, A_cpu[b * sa:].numpy(), lda, B_cpu[b * sb:].numpy(),
                                     ldb)
        parity.assert_bitwise(got[b], ref, "racecheck %s %s member %d" % (path, shape, b))


GENERAL = [c for c in range(sg.num_configs()) if sg.config_has_general_form(c)]
LAYOUTS = [(0, 0), (1, 0), (0, 1), (1, 1)]


@pytest.mark.parametrize("layout", LAYOUTS, ids=["NN", "TN", "NT", "TT"])
@pytest.mark.parametrize("config", GENERAL)
def test_racecheck_general_bitwise(config, layout):
    tA, tB = layout
    M, N, K = 200, 260, 333
    lda = (M if tA else K) + 3
    ldb = (K if tB else N) + 1
    ldc = N + 2
    dev = _dev()
    seed = 17 * config + tA + 2 * tB
    A_cpu, B_cpu = stored_operands(bool(tA), bool(tB), M, N, K, lda, ldb, seed, "int4")
    C0 = matrix(M, N, ldc, seed + 1, "int4")
    alpha, beta = 2.0, -1.0
    # C's window from C0; its row padding and a guard after it hold the sentinel.
    Ch = np.full(M * ldc + GUARD, SENTINEL, dtype=np.float32)
    win = (np.arange(M)[:, None] * ldc + np.arange(N)[None, :]).ravel()
    Ch[win] = C0.numpy()[win]
    C = torch.from_numpy(Ch).to(dev)
    A, B = A_cpu.to(dev), B_cpu.to(dev)
    st = _rc().sgemm_ex_with_config(config, tA, tB, M, N, K, alpha, A.data_ptr(), lda, 0,
                                    B.data_ptr(), ldb, 0, beta, C.data_ptr(), ldc, 0, 1,
                                    _stream())
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    got = _windows(C.cpu().numpy(), 1, M, N, ldc, M * ldc)[0]
    ref, _, _ = oracle.sgemm_ex_f64(bool(tA), bool(tB), M, N, K, alpha, A_cpu.numpy(), lda,
                                    B_cpu.numpy(), ldb, beta, C0.numpy(), ldc)
    parity.assert_bitwise(got, ref, "racecheck ex cfg%d %s" % (config, layout))


CONV = [c for c in range(sg.num_configs()) if sg.conv2d_config_available(c)]
# N, H, W, C, K, R, S, pad, stride: C = 64 stages directly on every tile, C = 24
# gathers through registers.
CONV_SHAPES = [(2, 9, 11, 64, 40, 3, 3, 1, 1), (1, 10, 7, 24, 33, 3, 3, 1, 2)]


@pytest.mark.parametrize("shape", CONV_SHAPES, ids=lambda s: "N%dH%dW%dC%dK%d" % s[:5])
@pytest.mark.parametrize("config", CONV)
def test_racecheck_conv_bitwise(config, shape):
    N, H, W, C, K, R, S, pad, stride = shape
    dev = _dev()
    gen = torch.Generator("cpu").manual_seed(N + H + C + K + config)
    x = torch.randint(-4, 5, (N, H, W, C), generator=gen).float()
    wt = torch.randint(-4, 5, (K, R, S, C), generator=gen).float()
    P, Q = sg.conv2d_output_size(H, W, R, S, (pad, pad), (stride, stride), (1, 1))
    n_out = N * P * Q * K
    y = torch.full((n_out + GUARD,), SENTINEL, dtype=torch.float32, device=dev)
    xd, wd = x.reshape(-1).to(dev), wt.reshape(-1).to(dev)
    st = _rc().conv2d_nhwc_with_config(config, N, H, W, C, K, R, S, pad, pad, stride, stride, 1,
                                       1, xd.data_ptr(), wd.data_ptr(), y.data_ptr(), _stream())
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert np.all(yh[n_out:] == SENTINEL), "y written past its end"
    ref, _ = oracle.conv2d_nhwc_f64(x.numpy(), wt.numpy(), N, H, W, C, K, R, S, (pad, pad),
                                    (stride, stride), (1, 1))
    parity.assert_bitwise(yh[:n_out].reshape(N, P, Q, K), ref,
                          "racecheck conv cfg%d %s" % (config, shape))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 300, 513, 64), (3, 129, 200, 128)],
                         ids=lambda s: "BH%d_Sq%d_Skv%d_D%d" % s)
def test_racecheck_attention(shape, causal):
    """Every K/V block goes through the two-stage ring; O against the oracle
    to the attention bound of the parity tests (a NaN fails it)."""
    BH, Sq, Skv, D = shape
    dev = _dev()
    gen = torch.Generator("cpu").manual_seed(BH + Sq + Skv + D + causal)
    q = torch.randn(BH, Sq, D, generator=gen)
    k = torch.randn(BH, Skv, D, generator=gen)
    v = torch.randn(BH, Skv, D, generator=gen)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    o = torch.full((BH * Sq * D + GUARD,), SENTINEL, device=dev)
    qd, kd, vd = q.reshape(-1).to(dev), k.reshape(-1).to(dev), v.reshape(-1).to(dev)
    st = _rc().attention_fwd(BH, Sq, Skv, D, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                             o.data_ptr(), scale, int(causal), _stream())
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    oh = o.cpu().numpy()
    assert np.all(oh[BH * Sq * D:] == SENTINEL), "O written past its end"
    got = oh[:BH * Sq * D].reshape(BH, Sq, D).astype(np.float64)
    ref, mag, smax = oracle.attention_f64(q.numpy(), k.numpy(), v.numpy(), BH, Sq, Skv, D, scale,
                                          causal)
    tol = (2e-4 + 4.0 * D * 2.0 ** -24 * smax)[..., None] * mag
    err = np.abs(got - ref)
    assert np.all(err <= tol), "racecheck attention %s causal=%d: %d outside the bound" % (
        shape, causal, int((~(err <= tol)).sum()))
