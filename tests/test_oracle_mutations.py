"""Planted mistakes in the oracle must fail its pins (CPU only).

Each case copies oracle/oracle.c to a temporary directory, plants one
plausible mistake by text substitution (a dropped term, a wrong sign, a wrong
index, a transposed operand, an ignored leading dimension, a missing absolute
value, FP32 instead of FP64 accumulation), builds it with gcc and runs the pin
checks of test_oracle against it.  Every mutant has to fail at least one pin.
All planted reads stay inside the operand buffers.
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

import test_oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTATIONS = {
    "dropped_first_term": ("for (int64_t k = 0; k < K; ++k) {\n        const double a = (double)Arow[k];",
                           "for (int64_t k = 1; k < K; ++k) {\n        const double a = (double)Arow[k];"),
    "wrong_sign": ("acc[j] += a * b;", "acc[j] -= a * b;"),
    "reversed_column_index": ("const double b = (double)Bk[j];",
                              "const double b = (double)Bk[N - 1 - j];"),
    "transposed_b": ("const double b = (double)Bk[j];",
                     "const double b = (double)B[(j % K) * ldb + (k % N)];"),
    "lda_ignored": ("A + i * lda, B, ldb", "A + i * K, B, ldb"),
    "abs_dropped": ("accabs[j] += aa * fabs(b);", "accabs[j] += aa * b;"),
    "fp32_accumulation": ("acc[j] += a * b;", "acc[j] = (float)(acc[j] + a * b);"),
}


def _build_mutant(tmp_path, name):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation anchor missing: %s" % name
    text = text.replace(old, new, 1)
    src = tmp_path / ("oracle_%s.c" % name)
    src.write_text(text)
    so = tmp_path / ("liboracle_%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", str(src), "-o", str(so), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_sgemm_f64.argtypes = [i64, i64, i64, p, i64, p, i64, p, p, i64, ctypes.c_int]
    lib.oracle_sgemm_f64.restype = ctypes.c_int

    def product(M, N, K, A, lda, B, ldb):
        a = np.ascontiguousarray(np.asarray(A, np.float32).ravel())
        b = np.ascontiguousarray(np.asarray(B, np.float32).ravel())
        C = np.empty((M, N), np.float64)
        Cabs = np.empty((M, N), np.float64)
        lib.oracle_sgemm_f64(M, N, K, a.ctypes.data, lda, b.ctypes.data, ldb,
                             C.ctypes.data, Cabs.ctypes.data, N, 1)
        return C, Cabs

    return product


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(tmp_path, name):
    product = _build_mutant(tmp_path, name)
    failed = []
    for chk in test_oracle.PIN_CHECKS:
        try:
            chk(product)
        except AssertionError:
            failed.append(chk.__name__)
    assert failed, "mutation %s passed every pin" % name


def test_unmutated_copy_passes(tmp_path):
    # The harness itself must not be what fails: a no-op "mutation" passes.
    MUTATIONS["_noop"] = ("acc[j] += a * b;", "acc[j] += a * b;")
    try:
        product = _build_mutant(tmp_path, "_noop")
        test_oracle.pin_checks(product)
    finally:
        del MUTATIONS["_noop"]
