"""GPU parity of the 2-D convolution (implicit GEMM on the matrix cores)
against the oracle, through the C ABI of include/conv2d.h.

y[n][p][q][k] = sum_{r,s,c} x[n][p*sh - ph + r*dh][q*sw - pw + s*dw][c] *
wt[k][r][s][c] ("Tiling Strategies" section 5, the convolution row of the
tiling-beyond-GEMM table).  Integer-valued inputs are compared bit for bit,
real ones within |y - y_ref| <= 2e-4 * sum |x||wt|.  The output buffer carries
a guard region filled with a sentinel that must come back unchanged; the input
and filter buffers are followed by NaNs that must never be read.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
from workloads import CONV_WORKLOADS, conv_operands

import tiled_fp32_gemm_sgemm_amd as sg

pytestmark = pytest.mark.gpu

SENTINEL = -7.25
GUARD = 97


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def conv_gpu(x, wt, N, H, W, C, K, R, S, pad=(0, 0), stride=(1, 1), dil=(1, 1), config=None):
    """Runs one call on CPU float32 buffers; returns y (N, P, Q, K) after
    checking that nothing past it was written."""
    dev = _dev()
    P, Q = sg.conv2d_output_size(H, W, R, S, pad, stride, dil)
    xd = torch.cat([x.reshape(-1), torch.full((GUARD,), float("nan"))]).to(dev)
    wd = torch.cat([wt.reshape(-1), torch.full((GUARD,), float("nan"))]).to(dev)
    n_out = N * P * Q * K
    yd = torch.full((n_out + GUARD,), SENTINEL, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = sg.conv2d_nhwc_raw(N, H, W, C, K, R, S, xd.data_ptr(), wd.data_ptr(), yd.data_ptr(),
                            pad, stride, dil, stream, config)
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    yh = yd.cpu().numpy()
    assert np.all(yh[n_out:] == SENTINEL), "y written past its end"
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


CONV_CONFIGS = [c for c in range(sg.num_configs()) if sg.conv2d_config_available(c)]

# N, H, W, C, K, R, S, pad, stride, dil -- C multiples of 64 stage directly on
# every tile, multiples of 32 on the BK = 32 tiles, the rest gather through
# registers; row counts N*P*Q and K cross tile edges.
SHAPES = [
    (2, 9, 11, 64, 40, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 17, 13, 32, 70, 3, 3, (1, 1), (2, 2), (1, 1)),
    (3, 8, 8, 64, 64, 1, 1, (0, 0), (1, 1), (1, 1)),
    (2, 12, 10, 32, 33, 5, 3, (2, 1), (1, 2), (2, 1)),
    (1, 20, 7, 128, 130, 3, 3, (0, 2), (1, 1), (1, 3)),
    (2, 6, 6, 3, 17, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 9, 9, 12, 20, 7, 7, (3, 3), (2, 2), (1, 1)),
    (4, 5, 5, 48, 9, 3, 2, (1, 0), (1, 1), (1, 1)),
]


def _ids(s):
    return "N%dH%dW%dC%dK%dR%dS%d_p%d%d_s%d%d_d%d%d" % (s[:7] + s[7] + s[8] + s[9])


@pytest.mark.parametrize("config", CONV_CONFIGS)
@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_conv_integer_bitwise(shape, config):
    N, H, W, C, K, R, S, pad, stride, dil = shape
    assert sg.conv2d_config_available(config)
    x, wt = _inputs(N, H, W, C, K, R, S, seed=N + H + C + K, dist="int4")
    y = conv_gpu(x, wt, N, H, W, C, K, R, S, pad, stride, dil, config)
    ref, _ = oracle.conv2d_nhwc_f64(x.numpy(), wt.numpy(), N, H, W, C, K, R, S, pad, stride, dil)
    parity.assert_bitwise(y, ref, "conv cfg%d %s" % (config, _ids(shape)))


@pytest.mark.parametrize("config", CONV_CONFIGS)
@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_conv_uniform_tolerance(shape, config):
    N, H, W, C, K, R, S, pad, stride, dil = shape
    x, wt = _inputs(N, H, W, C, K, R, S, seed=3 * N + W + K, dist="uniform")
    y = conv_gpu(x, wt, N, H, W, C, K, R, S, pad, stride, dil, config)
    ref, mag = oracle.conv2d_nhwc_f64(x.numpy(), wt.numpy(), N, H, W, C, K, R, S, pad, stride,
                                      dil)
    parity.assert_within_tolerance(y, ref, mag, "conv cfg%d %s" % (config, _ids(shape)))


def test_conv_worked_example():
    # The lecture's sliding window as a convolution: inputs 1..8, width 5.
    x = torch.arange(1, 9, dtype=torch.float32)
    y = conv_gpu(x, torch.ones(5), 1, 1, 8, 1, 1, 1, 5)
    assert y.ravel().tolist() == [15.0, 20.0, 25.0, 30.0]


def test_conv_degenerate_sizes():
    # filter wider than the padded image: no outputs, nothing written
    x, wt = _inputs(1, 2, 2, 4, 3, 5, 5, seed=1, dist="int4")
    y = conv_gpu(x, wt, 1, 2, 2, 4, 3, 5, 5)
    assert y.size == 0
    # no channels: every output is the empty sum, +0
    y = conv_gpu(torch.zeros(0), torch.zeros(0), 2, 4, 4, 0, 3, 3, 3, (1, 1))
    assert y.shape == (2, 4, 4, 3)
    assert np.all(y == 0.0) and not np.any(np.signbit(y))


def test_conv_invalid_arguments_enqueue_nothing():
    dev = _dev()
    y = torch.full((64,), SENTINEL, device=dev)
    x = torch.zeros(64, device=dev)
    lib_call = sg.conv2d_nhwc_raw
    base = dict(N=1, H=4, W=4, C=4, K=4, R=3, S=3)
    bad = [dict(stride=(0, 1)), dict(dil=(1, 0)), dict(pad=(-1, 0))]
    for kw in bad:
        st = lib_call(*base.values(), x.data_ptr(), x.data_ptr(), y.data_ptr(), **kw)
        assert st == -1
    st = lib_call(1, 4, 4, -1, 4, 3, 3, x.data_ptr(), x.data_ptr(), y.data_ptr())
    assert st == -1
    st = lib_call(1, 4, 4, 4, 4, 3, 3, 0, x.data_ptr(), y.data_ptr(), pad=1)
    assert st == -3
    st = lib_call(1, 4, 4, 4, 4, 3, 3, x.data_ptr(), x.data_ptr(), y.data_ptr(), pad=1, config=0)
    assert st == -7
    torch.cuda.synchronize()
    assert torch.all(y == SENTINEL)


@pytest.mark.parametrize("name", sorted(CONV_WORKLOADS))
def test_conv_workload_sampled(name):
    """The benchmark shapes in the launch configuration the benchmark times
    (automatic tile choice), on sampled outputs: every edge of the output
    image and random positions, all channels of a few positions."""
    w = CONV_WORKLOADS[name]
    x, wt = conv_operands(w)
    dev = _dev()
    P, Q = sg.conv2d_output_size(w.H, w.W, w.R, w.S, w.pad, w.stride, w.dil)
    y = sg.conv2d_nhwc(x.to(dev).view(w.N, w.H, w.W, w.C), wt.to(dev).view(w.K, w.R, w.S, w.C),
                       w.pad, w.stride, w.dil)
    torch.cuda.synchronize()
    yh = y.cpu().numpy().reshape(-1)
    rng = np.random.default_rng(12)
    n_out = w.N * P * Q * w.K
    pos = [(n, p, q) for n in (0, w.N - 1) for p in (0, P - 1) for q in range(Q)]
    pos += [(n, p, q) for n in (0, w.N - 1) for p in range(P) for q in (0, Q - 1)]
    idx = [((n * P + p) * Q + q) * w.K + k for (n, p, q) in pos for k in (0, w.K - 1)]
    idx += [((w.N // 2 * P + P // 2) * Q + Q // 2) * w.K + k for k in range(w.K)]
    idx = np.concatenate([np.asarray(idx, np.int64), rng.integers(0, n_out, 20000)])
    ref, mag = oracle.conv2d_nhwc_entries_f64(x.numpy(), wt.numpy(), w.N, w.H, w.W, w.C, w.K,
                                              w.R, w.S, idx, w.pad, w.stride, w.dil)
    parity.assert_within_tolerance(yh[idx], ref, mag, "conv workload %s" % name)


def test_conv_tensor_api_matches_torch_conv():
    dev = _dev()
    gen = torch.Generator("cpu").manual_seed(4)
    x = torch.randint(-3, 4, (2, 10, 12, 32), generator=gen).float()
    wt = torch.randint(-3, 4, (24, 3, 3, 32), generator=gen).float()
    y = sg.conv2d_nhwc(x.to(dev), wt.to(dev), pad=1, stride=(2, 1))
    ref = torch.nn.functional.conv2d(x.permute(0, 3, 1, 2).double(),
                                     wt.permute(0, 3, 1, 2).double(), stride=(2, 1), padding=1)
    assert torch.equal(y.cpu().double(), ref.permute(0, 2, 3, 1))
