"""Pins for the CPU oracle (no GPU).

The oracle must be right before it can judge the GPU library, so each check
here ties it to something other than itself: exact rational arithmetic on tiny
shapes, a library routine (torch float64 matmul on the CPU, numpy integer
matmul), identities that fix the result bit for bit, and the worked examples
the pages print (fixtures under tests/golden/).  ``pin_checks`` bundles them
so that test_oracle_mutations can show that planted mistakes fail them.
"""
import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import golden_io
from workloads import operands

U64 = 2.0 ** -53


def _real_product(M, N, K, A, lda, B, ldb):
    C, Cabs, _ = oracle.sgemm_f64(M, N, K, A, lda, B, ldb)
    return C, Cabs


# ---------------------------------------------------------------- pin checks
# Each takes ``product(M, N, K, A, lda, B, ldb) -> (C, Cabs)`` on flat float32
# numpy buffers and raises AssertionError when the pin does not hold.

def check_fraction_bruteforce(product, seed=11):
    """Exact rational sums of the FP32 inputs on tiny shapes."""
    rng = random.Random(seed)
    shapes = [(1, 1, 1), (2, 3, 5), (3, 2, 4), (6, 5, 6), (4, 6, 3), (5, 1, 6), (1, 4, 2)]
    for (M, N, K) in shapes:
        lda, ldb = K + rng.randint(0, 2), N + rng.randint(0, 2)
        A = np.full(M * lda, np.nan, dtype=np.float32)
        B = np.full(K * ldb, np.nan, dtype=np.float32)
        for i in range(M):
            for k in range(K):
                A[i * lda + k] = np.float32(rng.uniform(-1, 1) * 2.0 ** rng.randint(-12, 12))
        for k in range(K):
            for j in range(N):
                B[k * ldb + j] = np.float32(rng.uniform(-1, 1) * 2.0 ** rng.randint(-12, 12))
        C, Cabs = product(M, N, K, A, lda, B, ldb)
        assert C.shape == (M, N)
        assert np.all(np.isfinite(C)) and np.all(np.isfinite(Cabs))
        for i in range(M):
            for j in range(N):
                exact = sum(Fraction(float(A[i * lda + k])) * Fraction(float(B[k * ldb + j]))
                            for k in range(K))
                mag = sum(abs(Fraction(float(A[i * lda + k])) * Fraction(float(B[k * ldb + j])))
                          for k in range(K))
                err = abs(Fraction(float(C[i, j])) - exact)
                assert err <= Fraction(K) * Fraction(U64) * mag, (M, N, K, i, j)
                assert abs(Fraction(float(Cabs[i, j])) - mag) <= Fraction(K) * Fraction(U64) * mag


def check_identity_permutation(product, seed=5):
    """A.I = A and I.B = B bit for bit; permutation matrices permute exactly."""
    g = np.random.default_rng(seed)
    M, K = 37, 29
    A = g.uniform(-1, 1, (M, K)).astype(np.float32)
    I = np.eye(K, dtype=np.float32)
    C, _ = product(M, K, K, A.ravel(), K, I.ravel(), K)
    assert np.array_equal(C.astype(np.float32), A)
    Bm = g.uniform(-1, 1, (K, M)).astype(np.float32)
    C, _ = product(K, M, K, I.ravel(), K, Bm.ravel(), M)
    assert np.array_equal(C.astype(np.float32), Bm)
    perm = g.permutation(M)
    P = np.zeros((M, M), dtype=np.float32)
    P[np.arange(M), perm] = 1.0          # (P A)[i] = A[perm[i]]
    C, _ = product(M, K, M, P.ravel(), M, A.ravel(), K)
    assert np.array_equal(C.astype(np.float32), A[perm])
    permk = g.permutation(K)
    Q = np.zeros((K, K), dtype=np.float32)
    Q[permk, np.arange(K)] = 1.0         # (A Q)[:, j] = A[:, permk[j]]
    C, _ = product(M, K, K, A.ravel(), K, Q.ravel(), K)
    assert np.array_equal(C.astype(np.float32), A[:, permk])


def check_small_integers(product, seed=0):
    """Integer inputs in {-4..4}: partial sums stay far below 2^24, so the
    result is exact and unique; compare with numpy's int64 matmul."""
    M, N, K = 40, 33, 1024
    A, B = operands(M, N, K, K + 3, N + 1, seed, "int4")
    A, B = A.numpy(), B.numpy()
    C, Cabs = product(M, N, K, A, K + 3, B, N + 1)
    Ai = A.reshape(M, K + 3)[:, :K].astype(np.int64)
    Bi = B.reshape(K, N + 1)[:, :N].astype(np.int64)
    ref = Ai @ Bi
    assert np.array_equal(C, ref.astype(np.float64))
    assert np.array_equal(Cabs, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64))


def check_torch_float64(product, seed=7):
    """A library routine: torch.matmul in float64 on the CPU, padded operands."""
    M, N, K = 67, 45, 129
    lda, ldb = K + 2, N + 5
    A, B = operands(M, N, K, lda, ldb, seed, "uniform")
    C, Cabs = product(M, N, K, A.numpy(), lda, B.numpy(), ldb)
    At = A.view(M, lda)[:, :K].double()
    Bt = B.view(K, ldb)[:, :N].double()
    ref = (At @ Bt).numpy()
    refabs = (At.abs() @ Bt.abs()).numpy()
    assert np.all(np.abs(C - ref) <= 1e-12 * refabs)
    assert np.all(np.abs(Cabs - refabs) <= 1e-12 * refabs)


def check_worked_examples(product):
    """The pages' worked examples, read as products (tests/golden/)."""
    g = golden_io.read("outer_product_v2.txt")
    M, N, K = g["M"], g["N"], g["K"]
    A = np.array(g["A"], dtype=np.float32)
    B = np.array(g["B"], dtype=np.float32)
    C, _ = product(M, N, K, A, K, B, N)
    assert C.ravel().tolist() == [float(v) for v in g["C"]]
    w = golden_io.read("window5_sums.txt")
    x = np.array(w["x"], dtype=np.float32)
    width, y = w["width"], w["y"]
    M, K = len(y), len(x)
    band = np.zeros((M, K), dtype=np.float32)
    for i in range(M):
        band[i, i:i + width] = 1.0
    C, _ = product(M, 1, K, band.ravel(), K, x, 1)
    assert C.ravel().tolist() == [float(v) for v in y]


PIN_CHECKS = [check_fraction_bruteforce, check_identity_permutation, check_small_integers,
              check_torch_float64, check_worked_examples]


def pin_checks(product):
    for chk in PIN_CHECKS:
        chk(product)


# ------------------------------------------------------------------- tests

@pytest.mark.parametrize("chk", PIN_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(chk):
    chk(_real_product)


def test_all_ones_gives_k():
    M, N, K = 9, 7, 300
    C, Cabs, _ = oracle.sgemm_f64(M, N, K, np.ones(M * K, np.float32), K,
                                  np.ones(K * N, np.float32), N)
    assert np.all(C == K) and np.all(Cabs == K)


def test_padding_never_read():
    M, N, K = 31, 17, 45
    A, B = operands(M, N, K, K + 7, N + 3, 3, "uniform", pad=float("nan"))
    C, Cabs, _ = oracle.sgemm_f64(M, N, K, A.numpy(), K + 7, B.numpy(), N + 3)
    A2, B2 = operands(M, N, K, K, N, 3, "uniform", pad=0.0)
    C2, Cabs2, _ = oracle.sgemm_f64(M, N, K, A2.numpy(), K, B2.numpy(), N)
    assert np.all(np.isfinite(C))
    assert np.array_equal(C, C2) and np.array_equal(Cabs, Cabs2)


def test_k_zero_is_positive_zero():
    C, Cabs, _ = oracle.sgemm_f64(3, 4, 0, np.zeros(1, np.float32), 1,
                                  np.zeros(1, np.float32), 4)
    assert np.all(C == 0) and not np.any(np.signbit(C)) and np.all(Cabs == 0)


def test_empty_m_or_n():
    C, _, _ = oracle.sgemm_f64(0, 5, 3, np.zeros(1, np.float32), 3,
                               np.zeros(15, np.float32), 5)
    assert C.shape == (0, 5)
    C, _, _ = oracle.sgemm_f64(4, 0, 3, np.zeros(12, np.float32), 3,
                               np.zeros(1, np.float32), 1)
    assert C.shape == (4, 0)


def test_exact_cancellation_gives_positive_zero():
    # x + (-x) rounds to +0 under round-to-nearest: the pinned signed-zero rule.
    A = np.array([1.5, -1.5], np.float32)
    B = np.array([2.0, 2.0], np.float32)
    C, _, _ = oracle.sgemm_f64(1, 1, 2, A, 2, B, 1)
    assert C[0, 0] == 0 and not np.signbit(C[0, 0])


def test_thread_count_does_not_change_bits():
    M, N, K = 53, 61, 257
    A, B = operands(M, N, K, K, N, 9, "normal")
    C1, A1, used1 = oracle.sgemm_f64(M, N, K, A.numpy(), K, B.numpy(), N, nthreads=1)
    Cn, An, _ = oracle.sgemm_f64(M, N, K, A.numpy(), K, B.numpy(), N, nthreads=0)
    assert used1 == 1
    assert np.array_equal(C1, Cn) and np.array_equal(A1, An)


def test_entries_match_full_bitwise():
    M, N, K = 45, 39, 211
    lda, ldb = K + 1, N + 2
    A, B = operands(M, N, K, lda, ldb, 4, "uniform")
    C, Cabs, _ = oracle.sgemm_f64(M, N, K, A.numpy(), lda, B.numpy(), ldb)
    g = np.random.default_rng(0)
    rows, cols = g.integers(0, M, 100), g.integers(0, N, 100)
    e, eabs = oracle.entries_f64(K, A.numpy(), lda, B.numpy(), ldb, rows, cols)
    assert np.array_equal(e, C[rows, cols]) and np.array_equal(eabs, Cabs[rows, cols])


def test_batched_matches_torch_bmm():
    M, N, K, batch = 13, 11, 17, 5
    sa, sb = M * K + 3, K * N + 1
    A, B = operands(M, N, K, K, N, 8, "uniform", batch=batch, strideA=sa, strideB=sb, pad=0.0)
    C, Cabs = oracle.sgemm_strided_batched_f64(M, N, K, A.numpy(), K, sa, B.numpy(), N, sb, batch)
    At = torch.stack([A[b * sa: b * sa + M * K].view(M, K) for b in range(batch)]).double()
    Bt = torch.stack([B[b * sb: b * sb + K * N].view(K, N) for b in range(batch)]).double()
    ref = torch.bmm(At, Bt).numpy()
    refabs = torch.bmm(At.abs(), Bt.abs()).numpy()
    assert np.all(np.abs(C - ref) <= 1e-12 * refabs)
    assert np.allclose(Cabs, refabs, rtol=1e-12, atol=0)
    # batch members differ, so a wrong stride would not go unnoticed
    assert not np.allclose(C[0], C[1])
