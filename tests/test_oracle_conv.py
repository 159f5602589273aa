"""Pins for the oracle's 2-D convolution (CPU).

The convolution is the "Convolution" row of the tiled-kernel table in "Tiling
Strategies", section 5: NHWC input x[n][h][w][c], KRSC filters wt[k][r][s][c],
y[n][p][q][k] = sum_{r,s,c} x[n][p*sh - ph + r*dh][q*sw - pw + s*dw][c] *
wt[k][r][s][c], zero outside the image.  The oracle is tied to things other
than itself:
  * the lecture's sliding-window example (inputs 1..8, width 5 -> 15, 20, 25,
    30) as a one-channel, one-row convolution with a ones filter;
  * a library routine: torch's float64 conv2d on the CPU (NCHW / KCRS views of
    the same values), with padding, stride and dilation;
  * special cases: a 1x1 convolution is a matrix product (numpy), a centred
    delta filter with "same" padding returns the input exactly;
  * an invariant: moving the image one pixel inside a zero border moves the
    output one pixel (stride 1);
  * exact rational sums on tiny inputs, and exact integer results.
Planted mistakes in a copy of oracle.c must each fail one of these checks.
"""
import ctypes
import os
import random
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import torch

import golden_io
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PAD = 4096  # NaNs after every buffer: a planted index slip reads NaN, inside the buffer


def _buf(a):
    a = np.asarray(a, dtype=np.float32).ravel()
    return np.concatenate([a, np.full(PAD, np.nan, np.float32)])


def _real(x, wt, N, H, W, C, K, R, S, pad=(0, 0), stride=(1, 1), dil=(1, 1)):
    return oracle.conv2d_nhwc_f64(x, wt, N, H, W, C, K, R, S, pad, stride, dil)


def _rand(shape, rng, dist="normal"):
    if dist == "int":
        return rng.integers(-4, 5, size=shape).astype(np.float32)
    return rng.standard_normal(shape).astype(np.float32)


def _torch_conv(x, wt, pad, stride, dil):
    """torch float64 conv2d of NHWC x and KRSC wt; returns NPQK."""
    xt = torch.from_numpy(np.ascontiguousarray(x.transpose(0, 3, 1, 2))).double()
    wtt = torch.from_numpy(np.ascontiguousarray(wt.transpose(0, 3, 1, 2))).double()
    y = torch.nn.functional.conv2d(xt, wtt, stride=stride, padding=pad, dilation=dil)
    return y.permute(0, 2, 3, 1).numpy()


# ------------------------------------------------------------------ checks
# Each takes conv(x, wt, N, H, W, C, K, R, S, pad, stride, dil) -> (y, yabs).

def check_worked_example(conv):
    g = golden_io.read("window5_sums.txt")
    x = np.asarray(g["x"], np.float32)
    W, w = len(x), g["width"]
    y, yabs = conv(_buf(x), _buf(np.ones(w)), 1, 1, W, 1, 1, 1, w, (0, 0), (1, 1), (1, 1))
    assert y.ravel().tolist() == [float(v) for v in g["y"]]
    assert yabs.ravel().tolist() == [float(v) for v in g["y"]]


CASES = [
    # N, H, W, C, K, R, S, pad, stride, dil
    (2, 7, 9, 3, 4, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 8, 6, 5, 2, 3, 2, (0, 1), (2, 1), (1, 1)),
    (3, 10, 11, 4, 3, 3, 3, (2, 2), (1, 2), (2, 2)),
    (1, 5, 5, 8, 8, 5, 5, (2, 2), (1, 1), (1, 1)),
    (2, 9, 4, 2, 5, 1, 3, (0, 3), (3, 1), (1, 2)),
    (1, 4, 4, 16, 7, 4, 4, (1, 2), (2, 2), (1, 1)),
]


def check_torch_conv2d(conv):
    rng = np.random.default_rng(11)
    for (N, H, W, C, K, R, S, pad, stride, dil) in CASES:
        x = _rand((N, H, W, C), rng)
        wt = _rand((K, R, S, C), rng)
        y, yabs = conv(_buf(x), _buf(wt), N, H, W, C, K, R, S, pad, stride, dil)
        ref = _torch_conv(x.astype(np.float64), wt.astype(np.float64), pad, stride, dil)
        refabs = _torch_conv(np.abs(x).astype(np.float64), np.abs(wt).astype(np.float64), pad,
                             stride, dil)
        assert y.shape == ref.shape
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * max(1.0, np.abs(refabs).max()))
        assert np.allclose(yabs, refabs, rtol=1e-12, atol=1e-12)


def check_1x1_is_matmul(conv):
    rng = np.random.default_rng(5)
    N, H, W, C, K = 2, 5, 3, 7, 6
    x = _rand((N, H, W, C), rng)
    wt = _rand((K, 1, 1, C), rng)
    y, _ = conv(_buf(x), _buf(wt), N, H, W, C, K, 1, 1, (0, 0), (1, 1), (1, 1))
    ref = x.reshape(-1, C).astype(np.float64) @ wt.reshape(K, C).T.astype(np.float64)
    assert np.allclose(y.reshape(-1, K), ref, rtol=1e-13, atol=1e-13)


def check_delta_filter_identity(conv):
    rng = np.random.default_rng(7)
    N, H, W, C, R, S = 2, 6, 7, 5, 3, 5
    x = _rand((N, H, W, C), rng)
    wt = np.zeros((C, R, S, C), np.float32)
    for c in range(C):
        wt[c, R // 2, S // 2, c] = 1.0
    y, _ = conv(_buf(x), _buf(wt), N, H, W, C, C, R, S, (R // 2, S // 2), (1, 1), (1, 1))
    assert np.array_equal(y, x.astype(np.float64))


def check_translation(conv):
    rng = np.random.default_rng(9)
    N, H, W, C, K, R, S = 1, 9, 10, 3, 2, 3, 2
    img = _rand((N, 5, 5, C), rng)
    wt = _rand((K, R, S, C), rng)
    x0 = np.zeros((N, H, W, C), np.float32)
    x1 = np.zeros((N, H, W, C), np.float32)
    x0[:, 2:7, 2:7] = img
    x1[:, 3:8, 3:8] = img          # one pixel down and right
    y0, _ = conv(_buf(x0), _buf(wt), N, H, W, C, K, R, S, (1, 1), (1, 1), (1, 1))
    y1, _ = conv(_buf(x1), _buf(wt), N, H, W, C, K, R, S, (1, 1), (1, 1), (1, 1))
    assert np.array_equal(y1[:, 1:, 1:], y0[:, :-1, :-1])
    assert np.any(y0 != 0.0)


def check_fraction_bruteforce(conv):
    rng = random.Random(3)
    for (N, H, W, C, K, R, S, pad, stride, dil) in [(1, 3, 4, 2, 2, 2, 3, (1, 1), (1, 2), (1, 1)),
                                                    (2, 4, 3, 1, 3, 2, 2, (1, 0), (2, 1), (2, 1))]:
        x = np.array([rng.choice([-1, 1]) * rng.random() * 2.0 ** rng.randint(-20, 20)
                      for _ in range(N * H * W * C)], np.float32).reshape(N, H, W, C)
        wt = np.array([rng.choice([-1, 1]) * rng.random() * 2.0 ** rng.randint(-20, 20)
                       for _ in range(K * R * S * C)], np.float32).reshape(K, R, S, C)
        y, _ = conv(_buf(x), _buf(wt), N, H, W, C, K, R, S, pad, stride, dil)
        assert np.all(np.isfinite(y))
        P, Q = y.shape[1], y.shape[2]
        assert P == oracle.conv_out_size(H, pad[0], R, stride[0], dil[0])
        for n in range(N):
            for p in range(P):
                for q in range(Q):
                    for k in range(K):
                        exact = Fraction(0)
                        mag = Fraction(0)
                        for r in range(R):
                            for s in range(S):
                                h = p * stride[0] - pad[0] + r * dil[0]
                                w = q * stride[1] - pad[1] + s * dil[1]
                                if 0 <= h < H and 0 <= w < W:
                                    for c in range(C):
                                        t = Fraction(float(x[n, h, w, c])) * \
                                            Fraction(float(wt[k, r, s, c]))
                                        exact += t
                                        mag += abs(t)
                        err = abs(Fraction(float(y[n, p, q, k])) - exact)
                        assert err <= mag * Fraction(1, 2 ** 50)


def check_integer_exact(conv):
    rng = np.random.default_rng(13)
    N, H, W, C, K, R, S = 2, 11, 9, 6, 5, 3, 3
    x = _rand((N, H, W, C), rng, "int")
    wt = _rand((K, R, S, C), rng, "int")
    y, _ = conv(_buf(x), _buf(wt), N, H, W, C, K, R, S, (1, 1), (2, 1), (1, 1))
    ref = _torch_conv(x.astype(np.float64), wt.astype(np.float64), (1, 1), (2, 1), (1, 1))
    assert np.array_equal(y, ref)


PIN_CHECKS = [check_worked_example, check_torch_conv2d, check_1x1_is_matmul,
              check_delta_filter_identity, check_translation, check_fraction_bruteforce,
              check_integer_exact]


@pytest.mark.parametrize("chk", PIN_CHECKS, ids=lambda c: c.__name__)
def test_conv_oracle_pin(chk):
    chk(_real)


def test_conv_output_sizes_and_empty():
    assert oracle.conv_out_size(56, 1, 3, 1, 1) == 56
    assert oracle.conv_out_size(56, 1, 3, 2, 1) == 28
    assert oracle.conv_out_size(7, 0, 3, 1, 3) == 1
    assert oracle.conv_out_size(2, 0, 3, 1, 1) == 0
    # window larger than the padded input: empty output
    y, yabs = _real(np.zeros(8, np.float32), np.zeros(18, np.float32), 1, 2, 2, 2, 1, 3, 3)
    assert y.shape == (1, 0, 0, 1)
    # no channels: every output is the empty sum
    y, _ = _real(np.zeros(0, np.float32), np.zeros(0, np.float32), 1, 3, 3, 0, 2, 3, 3, (1, 1))
    assert y.shape == (1, 3, 3, 2) and np.all(y == 0.0)
    with pytest.raises(ValueError):
        _real(np.zeros(9, np.float32), np.zeros(9, np.float32), 1, 3, 3, 1, 1, 3, 3, (0, 0),
              (0, 1))


def test_conv_entries_match_full():
    rng = np.random.default_rng(21)
    N, H, W, C, K, R, S = 2, 9, 8, 4, 6, 3, 3
    x = _rand((N, H, W, C), rng)
    wt = _rand((K, R, S, C), rng)
    args = (N, H, W, C, K, R, S)
    y, yabs = oracle.conv2d_nhwc_f64(x, wt, *args, pad=(1, 0), stride=(1, 2), dil=(2, 1))
    idx = rng.integers(0, y.size, size=50)
    e, eabs = oracle.conv2d_nhwc_entries_f64(x, wt, *args, idx, pad=(1, 0), stride=(1, 2),
                                             dil=(2, 1))
    assert np.array_equal(e, y.ravel()[idx]) and np.array_equal(eabs, yabs.ravel()[idx])


# ------------------------------------------------------------- planted mistakes

CONV_MUTATIONS = {
    "pad_sign": ("const int64_t h = p * g->stride_h - g->pad_h + r * g->dil_h;",
                 "const int64_t h = p * g->stride_h + g->pad_h + r * g->dil_h;"),
    "stride_ignored": ("const int64_t w = q * g->stride_w - g->pad_w + s * g->dil_w;",
                       "const int64_t w = q - g->pad_w + s * g->dil_w;"),
    "dilation_ignored": ("const int64_t h = p * g->stride_h - g->pad_h + r * g->dil_h;",
                         "const int64_t h = p * g->stride_h - g->pad_h + r;"),
    "filter_r_s_swapped": ("const float *const wp = wt + ((k * g->R + r) * g->S + s) * g->C;",
                           "const float *const wp = wt + ((k * g->R + s) * g->S + r) * g->C;"),
    "row_bound_off_by_one": ("if (h < 0 || h >= g->H) continue;",
                             "if (h < 0 || h > g->H) continue;"),
    "first_channel_dropped": ("for (int64_t c = 0; c < g->C; ++c) {\n                const double prod",
                              "for (int64_t c = 1; c < g->C; ++c) {\n                const double prod"),
    "abs_dropped": ("accabs += fabs(prod);", "accabs += prod;"),
    "fp32_accumulation": ("acc += prod;", "acc = (float)(acc + prod);"),
    "output_q_k_swapped": ("const int64_t k = t % K;\n        t /= K;\n        const int64_t q = t % g.Q;\n"
                           "        t /= g.Q;",
                           "const int64_t q = t % g.Q;\n        t /= g.Q;\n        const int64_t k = t % K;\n"
                           "        t /= K;"),
}


def _build_mutant(tmp_path, name):
    old, new = CONV_MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation anchor missing: %s" % name
    src = tmp_path / ("oracle_c_%s.c" % name)
    src.write_text(text.replace(old, new))
    so = tmp_path / ("liboracle_c_%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", str(src), "-o", str(so), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_conv2d_nhwc_f64.argtypes = [i64] * 13 + [p, p, p, p]
    lib.oracle_conv2d_nhwc_f64.restype = ctypes.c_int

    def conv(x, wt, N, H, W, C, K, R, S, pad=(0, 0), stride=(1, 1), dil=(1, 1)):
        xx = np.ascontiguousarray(np.asarray(x, np.float32).ravel())
        ww = np.ascontiguousarray(np.asarray(wt, np.float32).ravel())
        P = oracle.conv_out_size(H, pad[0], R, stride[0], dil[0])
        Q = oracle.conv_out_size(W, pad[1], S, stride[1], dil[1])
        y = np.empty((N, P, Q, K), np.float64)
        ya = np.empty((N, P, Q, K), np.float64)
        st = lib.oracle_conv2d_nhwc_f64(N, H, W, C, K, R, S, pad[0], pad[1], stride[0],
                                        stride[1], dil[0], dil[1], xx.ctypes.data,
                                        ww.ctypes.data, y.ctypes.data, ya.ctypes.data)
        assert st == 0
        return y, ya

    return conv


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(CONV_MUTATIONS))
def test_planted_mistake_in_conv_fails_a_pin(tmp_path, name):
    conv = _build_mutant(tmp_path, name)
    failed = []
    for chk in PIN_CHECKS:
        try:
            chk(conv)
        except AssertionError:
            failed.append(chk.__name__)
    assert failed, "mutation %s passed every pin" % name


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_unmutated_conv_copy_passes(tmp_path):
    CONV_MUTATIONS["_noop"] = ("acc += prod;", "acc += prod;")
    try:
        conv = _build_mutant(tmp_path, "_noop")
        for chk in PIN_CHECKS:
            chk(conv)
    finally:
        del CONV_MUTATIONS["_noop"]
