"""Pins for the oracle's general form C = alpha op(A) op(B) + beta C (no GPU).

The general form reads transposed operands ("CMU DLSys Lecture 12: GPU
Acceleration", section 4 writes the product as C = A^T B with A stored K x M)
and applies the BLAS-style scalar update.  Each check ties it to something
other than itself: exact rational arithmetic on tiny shapes for all four
operand layouts, the lecture's worked example through the transposed form,
the transpose identity (A B)^T = B^T A^T bit for bit, closed forms for the
scalars (alpha = 0, beta = 0 with NaN in C, all-ones operands).  Planted
mistakes in a copy of oracle.c must each fail at least one of them.

Every operand buffer built here is square-padded (at least
max(M, N, K) rows of at least max(M, N, K) + 1 floats), so that a planted
index mistake still reads inside the buffer.
"""
import ctypes
import random
import shutil
import subprocess
import os
from fractions import Fraction

import numpy as np
import pytest

import golden_io
import oracle

U64 = 2.0 ** -53
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
LAYOUTS = [(False, False), (True, False), (False, True), (True, True)]


def _stored(trans, rows, cols):
    return (cols, rows) if trans else (rows, cols)


def _padded(rng_or_fill, rows, cols, ld, side):
    """A side x (ld) buffer (side >= rows) holding a rows x cols matrix; the
    rest is NaN unless rng_or_fill is a number."""
    buf = np.full(side * ld, np.nan, dtype=np.float32)
    for r in range(rows):
        for c in range(cols):
            v = rng_or_fill() if callable(rng_or_fill) else rng_or_fill
            buf[r * ld + c] = np.float32(v)
    return buf


def _real_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    out, out_abs, _ = oracle.sgemm_ex_f64(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta,
                                          C, ldc)
    return out, out_abs


# ---------------------------------------------------------------- pin checks
# Each takes ``ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
# -> (out, out_abs)`` on flat float32 buffers.

def check_ex_fraction_bruteforce(ex, seed=3):
    rng = random.Random(seed)
    val = lambda: rng.uniform(-1, 1) * 2.0 ** rng.randint(-10, 10)
    scalars = [(1.0, 0.0), (-1.5, 0.25), (0.75, -2.0), (2.0, 1.0)]
    for (M, N, K) in [(1, 1, 1), (2, 3, 5), (3, 2, 4), (5, 4, 6), (4, 6, 3), (1, 5, 2)]:
        side = max(M, N, K)
        ld = side + 1
        for (tA, tB) in LAYOUTS:
            alpha, beta = scalars[(M + 2 * N + tA + 2 * tB) % len(scalars)]
            ra, ca = _stored(tA, M, K)
            rb, cb = _stored(tB, K, N)
            A = _padded(val, ra, ca, ld, side)
            B = _padded(val, rb, cb, ld, side)
            C = _padded(val, M, N, ld, side)
            out, out_abs = ex(tA, tB, M, N, K, alpha, A, ld, B, ld, beta, C, ld)
            assert np.all(np.isfinite(out)) and np.all(np.isfinite(out_abs)), (tA, tB)
            for i in range(M):
                for j in range(N):
                    terms = []
                    for k in range(K):
                        a = A[k * ld + i] if tA else A[i * ld + k]
                        b = B[j * ld + k] if tB else B[k * ld + j]
                        terms.append(Fraction(float(a)) * Fraction(float(b)))
                    c = Fraction(float(C[i * ld + j]))
                    exact = Fraction(alpha) * sum(terms) + Fraction(beta) * c
                    mag = abs(Fraction(alpha)) * sum(abs(t) for t in terms) + \
                        abs(Fraction(beta)) * abs(c)
                    bound = Fraction(K + 2) * Fraction(U64) * mag
                    assert abs(Fraction(float(out[i, j])) - exact) <= bound, (tA, tB, i, j)
                    assert abs(Fraction(float(out_abs[i, j])) - mag) <= bound, (tA, tB, i, j)


def check_ex_worked_example(ex):
    """The lecture's outer product [2, 3]^T [5, 7] in its own form, C = A^T B
    with A stored as the 1 x 2 strip, and with B transposed as well."""
    g = golden_io.read("outer_product_v2.txt")
    M, N, K = g["M"], g["N"], g["K"]
    ld = 4
    A = np.full(4 * ld, np.nan, dtype=np.float32)
    A[:M] = g["A"]                      # stored K x M = one row
    B_row = np.full(4 * ld, np.nan, dtype=np.float32)
    B_row[:N] = g["B"]                  # stored K x N
    B_col = np.full(4 * ld, np.nan, dtype=np.float32)
    B_col[0], B_col[ld] = g["B"]        # stored N x K = one column
    want = [float(v) for v in g["C"]]
    out, _ = ex(True, False, M, N, K, 1.0, A, ld, B_row, ld, 0.0, None, ld)
    assert out.ravel().tolist() == want
    out, _ = ex(True, True, M, N, K, 1.0, A, ld, B_col, ld, 0.0, None, ld)
    assert out.ravel().tolist() == want


def check_ex_transpose_identity(ex, seed=8):
    """(A B)^T = B^T A^T: the same k-ordered sums, so bit for bit."""
    rng = np.random.default_rng(seed)
    M, N, K = 5, 7, 6
    side = 8
    ld = 9
    A = np.full(side * ld, np.nan, np.float32)
    B = np.full(side * ld, np.nan, np.float32)
    for i in range(M):
        A[i * ld:i * ld + K] = rng.standard_normal(K).astype(np.float32)
    for k in range(K):
        B[k * ld:k * ld + N] = rng.standard_normal(N).astype(np.float32)
    C1, _ = ex(False, False, M, N, K, 1.0, A, ld, B, ld, 0.0, None, ld)
    C2, _ = ex(True, True, N, M, K, 1.0, B, ld, A, ld, 0.0, None, ld)
    assert np.array_equal(C1, C2.T)
    C3, _ = ex(False, True, M, M, K, 1.0, A, ld, A, ld, 0.0, None, ld)   # A A^T is symmetric
    assert np.array_equal(C3, C3.T)


def check_ex_scalar_closed_forms(ex):
    M, N, K = 3, 4, 5
    side, ld = 6, 7
    ones_a = _padded(1.0, M, K, ld, side)
    ones_b = _padded(1.0, K, N, ld, side)
    ones_c = _padded(1.0, M, N, ld, side)
    out, _ = ex(False, False, M, N, K, 2.0, ones_a, ld, ones_b, ld, 3.0, ones_c, ld)
    assert np.all(out == 2 * K + 3)
    # beta = 0: C is not read, NaN there does not matter
    nan_c = np.full(side * ld, np.nan, np.float32)
    out, _ = ex(False, False, M, N, K, -1.0, ones_a, ld, ones_b, ld, 0.0, nan_c, ld)
    assert np.all(out == -K)
    # alpha = 0: A and B are not read
    nan_ab = np.full(side * ld, np.nan, np.float32)
    c = _padded(1.5, M, N, ld, side)
    out, out_abs = ex(True, True, M, N, K, 0.0, nan_ab, ld, nan_ab, ld, -2.0, c, ld)
    assert np.all(out == -3.0) and np.all(out_abs == 3.0)
    # K = 0: the empty sum, so only beta C remains
    out, _ = ex(False, False, M, N, 0, 5.0, nan_ab, ld, nan_ab, ld, 0.5, c, ld)
    assert np.all(out == 0.75)
    # no product term at all (BLAS): signed zeros come from beta C alone
    out, _ = ex(False, False, M, N, 0, -1.0, nan_ab, ld, nan_ab, ld, 0.0, None, ld)
    assert np.all(out == 0.0) and not np.any(np.signbit(out))
    zero_c = _padded(0.0, M, N, ld, side)
    out, _ = ex(False, False, M, N, K, 0.0, nan_ab, ld, nan_ab, ld, -1.0, zero_c, ld)
    assert np.all(np.signbit(out))


EX_PIN_CHECKS = [check_ex_fraction_bruteforce, check_ex_worked_example,
                 check_ex_transpose_identity, check_ex_scalar_closed_forms]


@pytest.mark.parametrize("chk", EX_PIN_CHECKS, ids=lambda f: f.__name__)
def test_oracle_ex_pin(chk):
    chk(_real_ex)


def test_ex_matches_plain_form_bitwise():
    # alpha = 1, beta = 0, no transposes: the same sums as oracle_sgemm_f64.
    rng = np.random.default_rng(2)
    M, N, K, lda, ldb = 17, 13, 29, 31, 15
    A = rng.standard_normal(M * lda).astype(np.float32)
    B = rng.standard_normal(K * ldb).astype(np.float32)
    C1, A1, _ = oracle.sgemm_f64(M, N, K, A, lda, B, ldb)
    C2, A2, _ = oracle.sgemm_ex_f64(False, False, M, N, K, 1.0, A, lda, B, ldb, 0.0)
    assert np.array_equal(C1, C2) and np.array_equal(A1, A2)


def test_ex_entries_match_full_bitwise():
    rng = np.random.default_rng(4)
    M, N, K = 23, 19, 31
    for tA, tB in LAYOUTS:
        ra, ca = _stored(tA, M, K)
        rb, cb = _stored(tB, K, N)
        lda, ldb, ldc = ca + 2, cb + 3, N + 1
        A = rng.standard_normal(ra * lda).astype(np.float32)
        B = rng.standard_normal(rb * ldb).astype(np.float32)
        C = rng.standard_normal(M * ldc).astype(np.float32)
        full, full_abs, _ = oracle.sgemm_ex_f64(tA, tB, M, N, K, -0.5, A, lda, B, ldb, 1.25,
                                                C, ldc)
        r = rng.integers(0, M, 50)
        c = rng.integers(0, N, 50)
        e, e_abs = oracle.ex_entries_f64(tA, tB, K, -0.5, A, lda, B, ldb, 1.25, C, ldc, r, c)
        assert np.array_equal(e, full[r, c]) and np.array_equal(e_abs, full_abs[r, c])


# ------------------------------------------------------------ planted mistakes
EX_MUTATIONS = {
    "transA_ignored": ("(transA ? A[k * lda + i] : A[i * lda + k])", "(A[i * lda + k])"),
    "transB_ignored": ("(transB ? B[j * ldb + k] : B[k * ldb + j])", "(B[k * ldb + j])"),
    "transA_index_swapped": ("(transA ? A[k * lda + i] : A[i * lda + k])",
                             "(transA ? A[i * lda + k] : A[i * lda + k])"),
    "alpha_ignored": ("v = alpha * acc;", "v = acc;"),
    "beta_ignored": ("v = has_product ? v + beta * c : beta * c;",
                     "v = has_product ? v + c : c;"),
    "abs_of_beta_term_dropped": ("vabs += fabs(beta) * fabs(c);", "vabs += beta * c;"),
    "alpha_zero_still_reads": ("const int has_product = alpha != 0.0 && K > 0;",
                               "const int has_product = 1;"),
}


def _build_ex_mutant(tmp_path, name):
    old, new = EX_MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation anchor missing: %s" % name
    src = tmp_path / ("oracle_ex_%s.c" % name)
    src.write_text(text.replace(old, new))
    so = tmp_path / ("liboracle_ex_%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", str(src), "-o", str(so), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_sgemm_ex_f64.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                        ctypes.c_float, p, i64, p, i64, ctypes.c_float, p, i64,
                                        p, p, i64, ctypes.c_int]
    lib.oracle_sgemm_ex_f64.restype = ctypes.c_int

    def ex(tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
        a = np.ascontiguousarray(np.asarray(A, np.float32).ravel())
        b = np.ascontiguousarray(np.asarray(B, np.float32).ravel())
        c = np.ascontiguousarray(np.asarray(C if C is not None else np.zeros(1), np.float32)
                                 .ravel())
        out = np.empty((M, N), np.float64)
        out_abs = np.empty((M, N), np.float64)
        lib.oracle_sgemm_ex_f64(int(tA), int(tB), M, N, K, alpha, a.ctypes.data, lda,
                                b.ctypes.data, ldb, beta, c.ctypes.data, ldc, out.ctypes.data,
                                out_abs.ctypes.data, N, 1)
        return out, out_abs

    return ex


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(EX_MUTATIONS))
def test_planted_mistake_in_general_form_fails_a_pin(tmp_path, name):
    ex = _build_ex_mutant(tmp_path, name)
    failed = []
    for chk in EX_PIN_CHECKS:
        try:
            chk(ex)
        except AssertionError:
            failed.append(chk.__name__)
    assert failed, "mutation %s passed every pin" % name
