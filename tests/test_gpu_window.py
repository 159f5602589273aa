"""GPU parity of the sliding window sum (MI355X) against the oracle.

y[i] = sum_{d<W} x[i+d] for i < n ("CMU DLSys Lecture 12: GPU Acceleration",
section 3).  Integer inputs give exact sums in any order, so those cases are
compared bit for bit; real inputs within |y - y_ref| <= 2e-4 * sum_d |x[i+d]|.
The n + W - 1 valid inputs are followed by NaN (never read), y's tail past n
holds a sentinel (never written), and pointers are also tried off 16-byte
alignment.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
import tiled_fp32_gemm_sgemm_amd as sg
from workloads import draw

pytestmark = pytest.mark.gpu

SENTINEL = -7.25
GUARD = 64


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_window(n, W, vals, x_off=0, y_off=0):
    """vals: the n + W - 1 inputs (CPU float32).  Returns y (n values)."""
    dev = _dev()
    x = torch.full((x_off + n + W - 1 + GUARD,), float("nan"), dtype=torch.float32)
    x[x_off:x_off + n + W - 1] = vals
    y = torch.full((y_off + n + GUARD,), SENTINEL, dtype=torch.float32)
    xd, yd = x.to(dev), y.to(dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = sg.window_sum_raw(n, W, xd.data_ptr() + 4 * x_off, yd.data_ptr() + 4 * y_off, stream)
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    yh = yd.cpu().numpy()
    assert np.all(yh[:y_off] == SENTINEL) and np.all(yh[y_off + n:] == SENTINEL)
    return yh[y_off:y_off + n]


def _vals(n, W, seed, dist):
    gen = torch.Generator("cpu").manual_seed(seed)
    return draw(gen, n + W - 1, dist)


# Widths on both sides of 8 and 24 (the widest windows of the blocks of 1024
# and 2048 outputs; wider ones take 4096), and lengths around the block sizes.
@pytest.mark.parametrize("W", [1, 2, 3, 5, 8, 9, 16, 24, 25, 64, 255, 1023, 1024])
@pytest.mark.parametrize("n", [1, 3, 4, 5, 1023, 1024, 1025, 2047, 2049, 4095, 4096, 4097, 12289,
                               100003])
def test_window_integer_bitwise(n, W):
    v = _vals(n, W, n + 7 * W, "int4")
    got = run_window(n, W, v)
    ref, _ = oracle.window_sum_f64(n, W, v.numpy())
    parity.assert_bitwise(got, ref, "window n=%d W=%d" % (n, W))


@pytest.mark.parametrize("W", [1, 5, 31, 1024])
@pytest.mark.parametrize("n", [7, 4097, 65537])
def test_window_uniform_tolerance(n, W):
    v = _vals(n, W, 3 * n + W, "uniform")
    got = run_window(n, W, v)
    ref, mag = oracle.window_sum_f64(n, W, v.numpy())
    parity.assert_within_tolerance(got, ref, mag, "window uniform n=%d W=%d" % (n, W))


@pytest.mark.parametrize("W", [5, 17, 33])
@pytest.mark.parametrize("x_off,y_off", [(1, 0), (2, 3), (3, 1)])
def test_window_unaligned_pointers(x_off, y_off, W):
    n = 9001
    v = _vals(n, W, 17, "int4")
    got = run_window(n, W, v, x_off, y_off)
    ref, _ = oracle.window_sum_f64(n, W, v.numpy())
    parity.assert_bitwise(got, ref, "window offsets %d %d W=%d" % (x_off, y_off, W))


def test_window_worked_example():
    # The lecture's figure: inputs 1..8, W = 5 -> 15, 20, 25, 30.
    got = run_window(4, 5, torch.arange(1, 9, dtype=torch.float32))
    assert got.tolist() == [15.0, 20.0, 25.0, 30.0]


def test_window_large_full():
    n, W = (1 << 24) + 3, 5
    v = _vals(n, W, 5, "uniform")
    got = run_window(n, W, v)
    ref, mag = oracle.window_sum_f64(n, W, v.numpy())
    parity.assert_within_tolerance(got, ref, mag, "window large")


def test_window_tensor_api():
    dev = _dev()
    x = torch.randint(-4, 5, (50000,), dtype=torch.float32, device=dev)
    y = sg.window_sum(x, 7)
    ref = torch.nn.functional.conv1d(x.double().view(1, 1, -1),
                                     torch.ones(1, 1, 7, dtype=torch.float64, device=dev))
    assert torch.equal(y.double(), ref.view(-1))
