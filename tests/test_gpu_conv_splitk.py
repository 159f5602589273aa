"""GPU parity of the split-K convolution (conv2d_nhwc_splitk in
include/conv2d.h) against the oracle.

The convolution is that of "Tiling Strategies" section 5 (the convolution row
of the tiling-beyond-GEMM table), run as an implicit GEMM whose reduction over
R*S*C is cut into chunks joined through a workspace; the chunks of a tile are
added in chunk order, so results are reproducible bit for bit.  Integer-valued
inputs are compared bit for bit with the oracle, real ones within
|y - y_ref| <= 2e-4 * sum |x||wt|.  Every call checks that nothing past the
output was written and that the workspace's counter header is back at zero.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
from workloads import CONV_WORKLOADS, conv_operands

import tiled_fp32_gemm_sgemm_amd as sg
from tiled_fp32_gemm_sgemm_amd import _native

pytestmark = pytest.mark.gpu

SENTINEL = -7.25
GUARD = 97


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _workspace(nbytes):
    return torch.zeros(max(nbytes, sg.SPLITK_HEADER_BYTES) + 256, dtype=torch.uint8,
                       device=_dev())


def conv_splitk_gpu(x, wt, N, H, W, C, K, R, S, pad=(0, 0), stride=(1, 1), dil=(1, 1),
                    splits=0, config=None, ws=None, lib=None):
    """One call on CPU float32 buffers; returns y (N, P, Q, K) after checking
    the output's guard region and the workspace header."""
    dev = _dev()
    P, Q = sg.conv2d_output_size(H, W, R, S, pad, stride, dil)
    _, _, nbytes, _ = sg.conv2d_splitk_plan(N, H, W, C, K, R, S, pad, stride, dil, splits,
                                            config)
    if ws is None:
        ws = _workspace(nbytes)
    xd = torch.cat([x.reshape(-1), torch.full((GUARD,), float("nan"))]).to(dev)
    wd = torch.cat([wt.reshape(-1), torch.full((GUARD,), float("nan"))]).to(dev)
    n_out = N * P * Q * K
    yd = torch.full((n_out + GUARD,), SENTINEL, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (-1 if config is None else config, N, H, W, C, K, R, S, pad[0], pad[1], stride[0],
            stride[1], dil[0], dil[1], xd.data_ptr(), wd.data_ptr(), yd.data_ptr(), splits,
            ws.data_ptr(), ws.numel(), stream)
    st = (lib or _native.lib()).conv2d_nhwc_splitk(*args)
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    yh = yd.cpu().numpy()
    assert np.all(yh[n_out:] == SENTINEL), "y written past its end"
    assert int(ws[:sg.SPLITK_HEADER_BYTES].view(torch.int32).abs().sum()) == 0, \
        "counter header not back at zero"
    return yh[:n_out].reshape(N, P, Q, K)


def _inputs(N, H, W, C, K, R, S, seed, dist):
    gen = torch.Generator("cpu").manual_seed(seed)
    if dist == "int4":
        x = torch.randint(-4, 5, (N, H, W, C), generator=gen).float()
        wt = torch.randint(-4, 5, (K, R, S, C), generator=gen).float()
    else:
        x = torch.rand((N, H, W, C), generator=gen) * 2 - 1
        wt = torch.rand((K, R, S, C), generator=gen) * 2 - 1
    return x, wt


SK_CONFIGS = [c for c in range(sg.num_configs()) if sg.conv2d_config_has_splitk(c)]

# N, H, W, C, K, R, S, pad, stride, dil -- C = 64 and 96 stage directly (a
# chunk of an odd number of 32-wide slices starts inside a filter tap), C = 32
# on the BK = 32 tiles only, C = 3, 12 and 48 gather through registers; row
# counts N*P*Q and K cross tile edges.
SHAPES = [
    (2, 9, 11, 64, 40, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 17, 13, 32, 70, 3, 3, (1, 1), (2, 2), (1, 1)),
    (2, 12, 10, 96, 33, 5, 3, (2, 1), (1, 2), (2, 1)),
    (1, 20, 7, 128, 130, 3, 3, (0, 2), (1, 1), (1, 3)),
    (2, 6, 6, 3, 17, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 9, 9, 12, 20, 7, 7, (3, 3), (2, 2), (1, 1)),
    (4, 5, 5, 48, 9, 3, 2, (1, 0), (1, 1), (1, 1)),
]


def _ids(s):
    return "N%dH%dW%dC%dK%dR%dS%d_p%d%d_s%d%d_d%d%d" % (s[:7] + s[7] + s[8] + s[9])


@pytest.mark.parametrize("splits", [2, 3, 5])
@pytest.mark.parametrize("config", SK_CONFIGS)
@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_conv_splitk_integer_bitwise(shape, config, splits):
    N, H, W, C, K, R, S, pad, stride, dil = shape
    x, wt = _inputs(N, H, W, C, K, R, S, seed=N + H + C + K, dist="int4")
    y = conv_splitk_gpu(x, wt, N, H, W, C, K, R, S, pad, stride, dil, splits, config)
    ref, _ = oracle.conv2d_nhwc_f64(x.numpy(), wt.numpy(), N, H, W, C, K, R, S, pad, stride, dil)
    parity.assert_bitwise(y, ref, "conv split-K cfg%d S%d %s" % (config, splits, _ids(shape)))


@pytest.mark.parametrize("config", SK_CONFIGS)
@pytest.mark.parametrize("shape", SHAPES[:4], ids=_ids)
def test_conv_splitk_uniform_tolerance_and_repeatable(shape, config):
    N, H, W, C, K, R, S, pad, stride, dil = shape
    x, wt = _inputs(N, H, W, C, K, R, S, seed=3 * N + W + K, dist="uniform")
    y = conv_splitk_gpu(x, wt, N, H, W, C, K, R, S, pad, stride, dil, 4, config)
    ref, mag = oracle.conv2d_nhwc_f64(x.numpy(), wt.numpy(), N, H, W, C, K, R, S, pad, stride,
                                      dil)
    parity.assert_within_tolerance(y, ref, mag, "conv split-K cfg%d %s" % (config, _ids(shape)))
    y2 = conv_splitk_gpu(x, wt, N, H, W, C, K, R, S, pad, stride, dil, 4, config)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "not reproducible"


# Shapes whose automatic plan is hybrid: 256 tiles take all of R*S*C, the rest
# are split (chunks of 7 slices of 32, so most start inside a filter tap).
HYBRID = [(40, 15, 15, 96, 96, 3, 3, (1, 1), (1, 1), (1, 1)),
          (32, 17, 17, 96, 96, 3, 3, (1, 1), (1, 1), (1, 1))]


@pytest.mark.parametrize("shape", HYBRID, ids=_ids)
def test_conv_splitk_hybrid_plan_bitwise(shape):
    N, H, W, C, K, R, S, pad, stride, dil = shape
    cfg, splits, nbytes, full = sg.conv2d_splitk_plan(N, H, W, C, K, R, S, pad, stride, dil)
    assert splits > 1 and full > 0, "expected a hybrid plan"
    info = sg.config_info(cfg)
    P, Q = sg.conv2d_output_size(H, W, R, S, pad, stride, dil)
    tiles = -(-N * P * Q // info["bm"]) * -(-K // info["bn"])
    assert nbytes == sg.SPLITK_HEADER_BYTES + (tiles - full) * splits * info["bm"] * info["bn"] * 4
    x, wt = _inputs(N, H, W, C, K, R, S, seed=N * C + K, dist="int4")
    ref, _ = oracle.conv2d_nhwc_f64(x.numpy(), wt.numpy(), N, H, W, C, K, R, S, pad, stride, dil)
    ws = _workspace(nbytes)
    y = conv_splitk_gpu(x, wt, N, H, W, C, K, R, S, pad, stride, dil, ws=ws)
    parity.assert_bitwise(y, ref, "conv hybrid %s" % _ids(shape))
    y = conv_splitk_gpu(x, wt, N, H, W, C, K, R, S, pad, stride, dil, ws=ws,
                        lib=_native.racecheck_lib())
    parity.assert_bitwise(y, ref, "conv hybrid race-check %s" % _ids(shape))


@pytest.mark.parametrize("config", SK_CONFIGS)
def test_conv_splitk_racecheck_bitwise(config):
    """Race-check build (slices poisoned with NaN once consumed, workgroups in
    reverse order): the join must still see only complete partials."""
    N, H, W, C, K, R, S, pad, stride, dil = SHAPES[2]
    x, wt = _inputs(N, H, W, C, K, R, S, seed=11, dist="int4")
    y = conv_splitk_gpu(x, wt, N, H, W, C, K, R, S, pad, stride, dil, 3, config,
                        lib=_native.racecheck_lib())
    ref, _ = oracle.conv2d_nhwc_f64(x.numpy(), wt.numpy(), N, H, W, C, K, R, S, pad, stride, dil)
    parity.assert_bitwise(y, ref, "conv split-K race-check cfg%d" % config)


def test_conv_splitk_shares_workspace_with_sgemm_splitk():
    """Calls of both kinds, of different tile counts, in turn on one
    workspace: each leaves the counter header at zero for the next."""
    dev = _dev()
    shape = HYBRID[0]
    N, H, W, C, K, R, S, pad, stride, dil = shape
    x, wt = _inputs(N, H, W, C, K, R, S, seed=5, dist="int4")
    ref, _ = oracle.conv2d_nhwc_f64(x.numpy(), wt.numpy(), N, H, W, C, K, R, S, pad, stride, dil)
    gen = torch.Generator("cpu").manual_seed(6)
    A = torch.randint(-4, 5, (700, 3000), generator=gen).float()
    B = torch.randint(-4, 5, (3000, 300), generator=gen).float()
    gref, _ = oracle.matmul_f64(A.numpy(), B.numpy())
    ws = _workspace(64 << 20)
    for _ in range(2):
        y = conv_splitk_gpu(x, wt, N, H, W, C, K, R, S, pad, stride, dil, ws=ws)
        parity.assert_bitwise(y, ref, "conv on a shared workspace")
        C_ = sg.sgemm_splitk(A.to(dev), B.to(dev), splits=7, workspace=ws)
        torch.cuda.synchronize()
        parity.assert_bitwise(C_.cpu().numpy(), gref, "sgemm_splitk on a shared workspace")
        y = conv_splitk_gpu(x[:3], wt, 3, H, W, C, K, R, S, pad, stride, dil, splits=9, config=28,
                            ws=ws)
        parity.assert_bitwise(y, ref[:3], "small conv on a shared workspace")


@pytest.mark.parametrize("name", sorted(CONV_WORKLOADS))
def test_conv_splitk_workload_sampled(name):
    """The benchmark layers with the automatic plan, on sampled outputs
    (every edge of the output image, all channels of one position, random
    positions); a second call must give the same bits."""
    w = CONV_WORKLOADS[name]
    x, wt = conv_operands(w)
    dev = _dev()
    P, Q = sg.conv2d_output_size(w.H, w.W, w.R, w.S, w.pad, w.stride, w.dil)
    xd = x.to(dev).view(w.N, w.H, w.W, w.C)
    wd = wt.to(dev).view(w.K, w.R, w.S, w.C)
    y = sg.conv2d_nhwc_splitk(xd, wd, w.pad, w.stride, w.dil)
    y2 = sg.conv2d_nhwc_splitk(xd, wd, w.pad, w.stride, w.dil)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32)), "not reproducible"
    yh = y.cpu().numpy().reshape(-1)
    rng = np.random.default_rng(13)
    n_out = w.N * P * Q * w.K
    pos = [(n, p, q) for n in (0, w.N - 1) for p in (0, P - 1) for q in range(Q)]
    pos += [(n, p, q) for n in (0, w.N - 1) for p in range(P) for q in (0, Q - 1)]
    idx = [((n * P + p) * Q + q) * w.K + k for (n, p, q) in pos for k in (0, w.K - 1)]
    idx += [((w.N // 2 * P + P // 2) * Q + Q // 2) * w.K + k for k in range(w.K)]
    idx += list(range(n_out - 64 * w.K, n_out, 7))  # the last row tiles (split ones)
    idx = np.concatenate([np.asarray(idx, np.int64), rng.integers(0, n_out, 20000)])
    ref, mag = oracle.conv2d_nhwc_entries_f64(x.numpy(), wt.numpy(), w.N, w.H, w.W, w.C, w.K,
                                              w.R, w.S, idx, w.pad, w.stride, w.dil)
    parity.assert_within_tolerance(yh[idx], ref, mag, "conv split-K workload %s" % name)


def test_conv_splitk_tensor_api_matches_conv2d_nhwc():
    """The tensor entry with its default workspace, against the plain
    convolution on integer inputs (both exact)."""
    dev = _dev()
    gen = torch.Generator("cpu").manual_seed(4)
    x = torch.randint(-3, 4, (40, 15, 15, 96), generator=gen).float().to(dev)
    wt = torch.randint(-3, 4, (96, 3, 3, 96), generator=gen).float().to(dev)
    y = sg.conv2d_nhwc_splitk(x, wt, pad=1)
    ref = sg.conv2d_nhwc(x, wt, pad=1)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)


def test_conv_splitk_degenerate_sizes():
    # filter wider than the padded image: no outputs, nothing written
    x, wt = _inputs(1, 2, 2, 4, 3, 5, 5, seed=1, dist="int4")
    y = conv_splitk_gpu(x, wt, 1, 2, 2, 4, 3, 5, 5, splits=3, config=28)
    assert y.size == 0
    # no channels: every output is the empty sum, +0
    y = conv_splitk_gpu(torch.zeros(0), torch.zeros(0), 2, 4, 4, 0, 3, 3, 3, (1, 1), splits=2,
                        config=28)
    assert y.shape == (2, 4, 4, 3)
    assert np.all(y == 0.0) and not np.any(np.signbit(y))
    # more chunks requested than slices: the plan caps them
    x, wt = _inputs(1, 4, 4, 32, 8, 1, 1, seed=2, dist="int4")
    _, sp, _, _ = sg.conv2d_splitk_plan(1, 4, 4, 32, 8, 1, 1, 0, 1, 1, 16, 28)
    assert sp == 1
    y = conv_splitk_gpu(x, wt, 1, 4, 4, 32, 8, 1, 1, splits=16, config=28)
    ref, _ = oracle.conv2d_nhwc_f64(x.numpy(), wt.numpy(), 1, 4, 4, 32, 8, 1, 1)
    parity.assert_bitwise(y, ref, "conv split-K, one slice")


def test_conv_splitk_invalid_arguments_enqueue_nothing():
    dev = _dev()
    y = torch.full((64,), SENTINEL, device=dev)
    # x and the filters are large enough for every call below (C up to 64),
    # should one be enqueued after all.
    x = torch.zeros(4096, device=dev)
    ws = _workspace(0)
    lib = _native.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream

    def call(config=-1, C=4, splits=0, xp=None, ws_bytes=None, stride=1):
        return lib.conv2d_nhwc_splitk(config, 1, 4, 4, C, 4, 3, 3, 1, 1, stride, 1, 1, 1,
                                      x.data_ptr() if xp is None else xp, x.data_ptr(),
                                      y.data_ptr(), splits, ws.data_ptr(),
                                      ws.numel() if ws_bytes is None else ws_bytes, stream)
    assert call(stride=0) == -1
    assert call(C=-1) == -1
    assert call(splits=65) == -1
    assert call(splits=-1) == -1
    assert call(config=0) == -7  # no convolution split-K kernel
    assert call(config=sg.num_configs()) == -7
    assert call(xp=0) == -3
    # a split plan with too small a workspace
    assert call(config=28, C=64, splits=4, ws_bytes=1024) == -9
    torch.cuda.synchronize()
    assert torch.all(y == SENTINEL)
