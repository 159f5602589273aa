"""Pins for the oracle's sliding window sum and the window load model (CPU).

y[i] = sum_{d<W} x[i+d] for i < n ("CMU DLSys Lecture 12: GPU Acceleration",
section 3).  The oracle is tied to: the lecture's worked example (inputs 1..8,
W = 5 -> 15, 20, 25, 30), closed forms for arithmetic sequences and constant
inputs, exact rational sums on small cases, and numpy's convolution (a
library routine).  Planted mistakes in a copy of oracle.c must fail one of
them.  The load model is tied to the section's printed counts.
"""
import ctypes
import os
import random
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import golden_io
import oracle
from tiled_fp32_gemm_sgemm_amd import model

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PAD = 8  # every buffer below carries PAD extra NaNs, so planted index slips stay inside


def _real(n, W, x):
    return oracle.window_sum_f64(n, W, x)


def _buf(vals):
    v = np.asarray(vals, dtype=np.float32)
    return np.concatenate([v, np.full(PAD, np.nan, np.float32)])


def check_window_worked_example(win):
    g = golden_io.read("window5_sums.txt")
    x = _buf(g["x"])
    y, _ = win(len(g["y"]), g["width"], x)
    assert y.tolist() == [float(v) for v in g["y"]]


def check_window_closed_forms(win):
    for n, W in [(1, 1), (7, 3), (100, 5), (33, 17), (5, 64)]:
        x = _buf(np.arange(1, n + W, dtype=np.float32))          # x_j = j + 1
        y, yabs = win(n, W, x)
        i = np.arange(n)
        want = W * (i + 1) + W * (W - 1) // 2
        assert np.all(np.isfinite(y)) and np.array_equal(y, want.astype(np.float64))
        assert np.array_equal(yabs, want.astype(np.float64))
        ones = _buf(-np.ones(n + W - 1, np.float32))
        y, yabs = win(n, W, ones)
        assert np.all(y == -W) and np.all(yabs == W)


def check_window_fraction_bruteforce(win, seed=6):
    rng = random.Random(seed)
    for n, W in [(1, 1), (3, 2), (6, 5), (9, 4), (4, 9)]:
        vals = [np.float32(rng.uniform(-1, 1) * 2.0 ** rng.randint(-20, 20)) for _ in range(n + W - 1)]
        x = _buf(vals)
        y, yabs = win(n, W, x)
        assert np.all(np.isfinite(y))
        for i in range(n):
            exact = sum(Fraction(float(vals[i + d])) for d in range(W))
            mag = sum(abs(Fraction(float(vals[i + d]))) for d in range(W))
            bound = Fraction(W) * Fraction(2.0 ** -53) * mag
            assert abs(Fraction(float(y[i])) - exact) <= bound, (n, W, i)
            assert abs(Fraction(float(yabs[i])) - mag) <= bound, (n, W, i)


def check_window_numpy_convolve(win, seed=2):
    rng = np.random.default_rng(seed)
    for n, W in [(1000, 5), (257, 31), (64, 1)]:
        vals = rng.standard_normal(n + W - 1).astype(np.float32)
        y, _ = win(n, W, _buf(vals))
        ref = np.convolve(vals.astype(np.float64), np.ones(W), mode="valid")
        assert np.all(np.abs(y - ref) <= 1e-12 * np.maximum(1.0, np.abs(ref)))


WINDOW_PIN_CHECKS = [check_window_worked_example, check_window_closed_forms,
                     check_window_fraction_bruteforce, check_window_numpy_convolve]


@pytest.mark.parametrize("chk", WINDOW_PIN_CHECKS, ids=lambda f: f.__name__)
def test_window_oracle_pin(chk):
    chk(_real)


def test_window_empty_and_argument_checks():
    y, yabs = oracle.window_sum_f64(0, 5, np.zeros(0, np.float32))
    assert y.size == 0 and yabs.size == 0
    with pytest.raises(ValueError):
        oracle.window_sum_f64(4, 5, np.zeros(7, np.float32))   # needs n + W - 1 = 8
    with pytest.raises(ValueError):
        oracle.window_sum_f64(4, 0, np.zeros(8, np.float32))


def test_window_load_model():
    g = golden_io.read("window_loads.txt")
    T, W = g["T"], g["W"]
    assert model.window_independent_loads(T, W) == g["independent"]
    assert model.window_staged_loads(T, W, T) == g["staged"]
    assert Fraction(model.window_staged_loads(T, W, T),
                    model.window_independent_loads(T, W)) == g["staged_fraction"]
    # the section's general ratio T(2R+1) / (T + 2R) for full blocks
    for T, R in [(256, 2), (4096, 2), (64, 7)]:
        W = 2 * R + 1
        assert Fraction(model.window_independent_loads(T, W), model.window_staged_loads(T, W, T)) \
            == Fraction(T * (2 * R + 1), T + 2 * R)
    # a partial last block stages its own outputs plus the halo
    assert model.window_staged_loads(10, 5, 4) == 2 * 8 + (2 + 4)
    assert model.window_bytes(4, 5) == 4 * (8 + 4)


WINDOW_MUTATIONS = {
    "last_term_dropped": ("for (int64_t d = 0; d < W; ++d) {\n            const double v = (double)x[i + d];",
                          "for (int64_t d = 0; d < W - 1; ++d) {\n            const double v = (double)x[i + d];"),
    "window_shifted": ("const double v = (double)x[i + d];", "const double v = (double)x[i + d + 1];"),
    "abs_dropped": ("sa += fabs(v);", "sa += v;"),
    "fp32_sum": ("            s += v;\n            sa += fabs(v);",
                 "            s = (float)(s + v);\n            sa += fabs(v);"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(WINDOW_MUTATIONS))
def test_planted_mistake_in_window_fails_a_pin(tmp_path, name):
    old, new = WINDOW_MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation anchor missing: %s" % name
    src = tmp_path / ("oracle_w_%s.c" % name)
    src.write_text(text.replace(old, new))
    so = tmp_path / ("liboracle_w_%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", str(src), "-o", str(so), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_window_sum_f64.argtypes = [i64, i64, p, p, p]
    lib.oracle_window_sum_f64.restype = None

    def win(n, W, x):
        xx = np.ascontiguousarray(np.asarray(x, np.float32))
        y = np.empty(n, np.float64)
        ya = np.empty(n, np.float64)
        lib.oracle_window_sum_f64(n, W, xx.ctypes.data, y.ctypes.data, ya.ctypes.data)
        return y, ya

    failed = []
    for chk in WINDOW_PIN_CHECKS:
        try:
            chk(win)
        except AssertionError:
            failed.append(chk.__name__)
    assert failed, "mutation %s passed every pin" % name
