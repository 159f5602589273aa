"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Inputs come from workloads.py (seeded, built on the CPU) and are handed to both
sides bit for bit.  Padding inside A and B (past each row, up to the leading
dimension) is NaN, so a kernel that reads it produces NaN and fails; C's
padding and a guard region after C are pre-filled with a sentinel that must
come back unchanged.  Integer-valued inputs are compared bit for bit,
real-valued ones to |C - C_ref| <= 2e-4 * (|A||B|)_ij (tests/parity.py).
"""
import random

import numpy as np
import pytest
import torch

import oracle
import parity
from workloads import WORKLOADS, operands, workload_operands

import tiled_fp32_gemm_sgemm_amd as sg

pytestmark = pytest.mark.gpu

SENTINEL = -7.25
GUARD = 257


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def run_gpu(M, N, K, A_cpu, lda, B_cpu, ldb, ldc, path="mfma", config=None, batch=1,
            strideA=0, strideB=0, strideC=None):
    """Runs one call; returns the C windows (batch, M, N) after checking that
    nothing outside them was written."""
    dev = _dev()
    A = A_cpu.to(dev)
    B = B_cpu.to(dev)
    one_c = M * ldc
    if strideC is None:
        strideC = one_c
    c_len = (batch - 1) * strideC + one_c if batch > 0 else 0
    C = torch.full((c_len + GUARD,), SENTINEL, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    if batch == 1 and strideA == 0 and strideB == 0 and config is None:
        st = sg.sgemm_raw(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc,
                          stream, path)
    else:
        st = sg.sgemm_strided_batched_raw(M, N, K, A.data_ptr(), lda, strideA, B.data_ptr(),
                                          ldb, strideB, C.data_ptr(), ldc, strideC, batch,
                                          stream, path, config)
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    Ch = C.cpu().numpy()
    written = np.zeros(c_len + GUARD, dtype=bool)
    out = np.empty((batch, M, N), dtype=np.float32)
    for b in range(batch):
        base = b * strideC
        idx = base + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
        out[b] = Ch[idx]
        written[idx] = True
    outside = Ch[~written]
    assert np.all(outside == SENTINEL), "C written outside its M x N window(s)"
    return out


def oracle_full(M, N, K, A_cpu, lda, B_cpu, ldb):
    C, Cabs, _ = oracle.sgemm_f64(M, N, K, A_cpu.numpy(), lda, B_cpu.numpy(), ldb)
    return C, Cabs


# ------------------------------------------------------------ small ragged shapes

_rng = random.Random(1234)
RAGGED = [(1, 1, 1), (2, 2, 1), (1, 300, 7), (300, 1, 5), (33, 65, 17), (64, 64, 16),
          (65, 63, 15), (127, 129, 31), (128, 128, 16), (255, 257, 33), (256, 128, 16),
          (257, 129, 300), (100, 200, 3), (3, 5, 299), (31, 47, 64), (200, 280, 250),
          (513, 260, 18), (200, 192, 1000), (130, 260, 515)]
RAGGED = [(M, N, K, K + _rng.randint(0, 3), N + _rng.randint(0, 5), N + _rng.randint(0, 7))
          for (M, N, K) in RAGGED]


def _call(path, *args, **kw):
    if path.startswith("cfg"):
        return run_gpu(*args, config=int(path[3:]), **kw)
    return run_gpu(*args, path=path, **kw)


ALL_PATHS = ["valu"] + ["cfg%d" % i for i in range(34)]


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_ragged_integer_bitwise(shape, path):
    M, N, K, lda, ldb, ldc = shape
    A, B = operands(M, N, K, lda, ldb, seed=M * 7 + N * 3 + K, dist_a="int4")
    C = _call(path, M, N, K, A, lda, B, ldb, ldc)[0]
    ref, _ = oracle_full(M, N, K, A, lda, B, ldb)
    parity.assert_bitwise(C, ref, "%s %s" % (path, shape))


def test_every_config_is_covered():
    assert sg.num_configs() == len(ALL_PATHS) - 1


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_ragged_uniform_tolerance(shape, path):
    M, N, K, lda, ldb, ldc = shape
    A, B = operands(M, N, K, lda, ldb, seed=M + N + K, dist_a="uniform")
    C = _call(path, M, N, K, A, lda, B, ldb, ldc)[0]
    ref, mag = oracle_full(M, N, K, A, lda, B, ldb)
    parity.assert_within_tolerance(C, ref, mag, "%s %s" % (path, shape))


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_worked_examples_on_gpu(path):
    import golden_io
    g = golden_io.read("outer_product_v2.txt")
    A = torch.tensor(g["A"], dtype=torch.float32)
    B = torch.tensor(g["B"], dtype=torch.float32)
    C = run_gpu(g["M"], g["N"], g["K"], A, g["K"], B, g["N"], g["N"], path=path)[0]
    assert C.ravel().tolist() == [float(v) for v in g["C"]]
    w = golden_io.read("window5_sums.txt")
    x = torch.tensor(w["x"], dtype=torch.float32)
    M, K = len(w["y"]), len(w["x"])
    band = torch.zeros(M, K)
    for i in range(M):
        band[i, i:i + w["width"]] = 1.0
    C = run_gpu(M, 1, K, band.reshape(-1), K, x, 1, 1, path=path)[0]
    assert C.ravel().tolist() == [float(v) for v in w["y"]]


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_identity_and_zero_rows(path):
    M, K = 300, 200
    A, _ = operands(M, K, K, K, K, seed=3, dist_a="uniform")
    A = A.view(M, K).clone()
    A[7] = 0.0                                # an all-zero row gives exact +0
    A[8, 2:] = -A[8, 2:]                      # mixed signs: -x * 0 terms must not matter
    eye = torch.eye(K)
    C = run_gpu(M, K, K, A.reshape(-1), K, eye.reshape(-1), K, K, path=path)[0]
    parity.assert_bitwise(C, A.numpy().astype(np.float64), "A.I")


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_k_zero_writes_positive_zero(path):
    M, N, ldc = 70, 50, 53
    dummy = torch.zeros(1)
    C = run_gpu(M, N, 0, dummy, 1, dummy, N, ldc, path=path)[0]
    assert np.all(C == 0) and not np.any(np.signbit(C))


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_empty_m_n_batch_write_nothing(path):
    dev = _dev()
    C = torch.full((64,), SENTINEL, device=dev)
    A = torch.ones(64, device=dev)
    for (M, N, K, batch) in [(0, 5, 3, 1), (5, 0, 3, 1), (4, 4, 4, 0)]:
        st = sg.sgemm_strided_batched_raw(M, N, K, A.data_ptr(), 8, 16, A.data_ptr(), 8, 16,
                                          C.data_ptr(), 8, 64, batch, 0, path)
        assert st == 0
    torch.cuda.synchronize()
    assert torch.all(C == SENTINEL)


def test_invalid_arguments_enqueue_nothing():
    dev = _dev()
    C = torch.full((64,), SENTINEL, device=dev)
    A = torch.ones(64, device=dev)
    st = sg.sgemm_raw(4, 4, 4, A.data_ptr(), 3, A.data_ptr(), 4, C.data_ptr(), 4)  # lda < K
    assert st == -2
    st = sg.sgemm_raw(4, 4, 4, A.data_ptr(), 4, 0, 4, C.data_ptr(), 4)  # NULL B
    assert st == -3
    torch.cuda.synchronize()
    assert torch.all(C == SENTINEL)


# ------------------------------------------------------------------ batched

@pytest.mark.parametrize("path", ["mfma", "valu", "cfg1", "cfg2", "cfg5", "cfg6", "cfg7", "cfg11", "cfg13", "cfg32",
                                  "cfg15", "cfg16", "cfg17", "cfg23", "cfg25"])
def test_batched_ragged_members_differ(path):
    M, N, K, lda, ldb, ldc, batch = 45, 77, 33, 36, 80, 79, 6
    sA, sB, sC = M * lda + 5, K * ldb + 3, M * ldc + 11
    A, B = operands(M, N, K, lda, ldb, seed=21, dist_a="int4", batch=batch, strideA=sA,
                    strideB=sB)
    C = _call(path, M, N, K, A, lda, B, ldb, ldc, batch=batch, strideA=sA, strideB=sB,
              strideC=sC)
    ref, _ = oracle.sgemm_strided_batched_f64(M, N, K, A.numpy(), lda, sA, B.numpy(), ldb, sB,
                                              batch)
    parity.assert_bitwise(C, ref, "batched " + path)
    assert not np.array_equal(C[0], C[1])


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_batched_shared_operand_stride_zero(path):
    M, N, K, batch = 64, 96, 40, 5
    A1, _ = operands(M, N, K, K, N, seed=5, dist_a="int4")
    _, Bb = operands(M, N, K, K, N, seed=6, dist_a="int4", batch=batch)
    C = run_gpu(M, N, K, A1[:M * K], K, Bb, N, N, path=path, batch=batch, strideA=0,
                strideB=K * N)
    ref, _ = oracle.sgemm_strided_batched_f64(M, N, K, A1.numpy(), K, 0, Bb.numpy(), N, K * N,
                                              batch)
    parity.assert_bitwise(C, ref, "shared A")


def test_side_stream():
    dev = _dev()
    M, N, K = 200, 300, 100
    A, B = operands(M, N, K, K, N, seed=9, dist_a="int4")
    Ad, Bd = A.to(dev), B.to(dev)
    s = torch.cuda.Stream(dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        C = sg.sgemm(Ad.view(M, K), Bd.view(K, N))
    s.synchronize()
    ref, _ = oracle_full(M, N, K, A, K, B, N)
    parity.assert_bitwise(C.cpu().numpy(), ref, "side stream")


# -------------------------------------------------------- the named workloads

def _sample_indices(M, N, seed, n_random=3000):
    g = np.random.default_rng(seed)
    edges_m = sorted({0, 1, 31, 32, 63, 64, 127, 128, 255, 256, M // 2, M - 2, M - 1} &
                     set(range(M)))
    edges_n = sorted({0, 1, 31, 32, 63, 64, 127, 128, 255, 256, N // 2, N - 2, N - 1} &
                     set(range(N)))
    rows = list(edges_m) + g.integers(0, M, 12).tolist()
    cols = list(edges_n) + g.integers(0, N, 12).tolist()
    rr, cc = np.meshgrid(rows, cols, indexing="ij")
    r = np.concatenate([rr.ravel(), g.integers(0, M, n_random)])
    c = np.concatenate([cc.ravel(), g.integers(0, N, n_random)])
    return r, c


def _check_sampled(w, C, A, B, exact=False):
    r, c = _sample_indices(w.M, w.N, w.seed)
    ref, mag = oracle.entries_f64(w.K, A.numpy(), w.lda, B.numpy(), w.ldb, r, c)
    got = C[r, c]
    if exact:
        parity.assert_bitwise(got, ref, w.name)
    else:
        ratio = parity.assert_within_tolerance(got, ref, mag, w.name)
        print("%s: max |err|/(|A||B|) over %d sampled entries = %.3e" % (w.name, r.size, ratio))


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_square1024_full(path):
    w = WORKLOADS["square1024"]
    A, B = workload_operands(w)
    C = run_gpu(w.M, w.N, w.K, A, w.lda, B, w.ldb, w.ldc, path=path)[0]
    ref, mag = oracle_full(w.M, w.N, w.K, A, w.lda, B, w.ldb)
    ratio = parity.assert_within_tolerance(C, ref, mag, w.name)
    print("square1024 %s: max ratio %.3e" % (path, ratio))


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_square1024_integer_full_bitwise(path):
    w = WORKLOADS["square1024_int"]
    A, B = workload_operands(w)
    C = run_gpu(w.M, w.N, w.K, A, w.lda, B, w.ldb, w.ldc, path=path)[0]
    ref, _ = oracle_full(w.M, w.N, w.K, A, w.lda, B, w.ldb)
    parity.assert_bitwise(C, ref, w.name)


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_square4096_sampled(path):
    w = WORKLOADS["square4096"]
    A, B = workload_operands(w)
    C = run_gpu(w.M, w.N, w.K, A, w.lda, B, w.ldb, w.ldc, path=path)[0]
    _check_sampled(w, C, A, B)


def test_square4096_integer_sampled_bitwise():
    # |partial sums| <= 16 * 4096 < 2^24: exact and unique at the headline size.
    w = WORKLOADS["square4096"]
    A, B = operands(w.M, w.N, w.K, w.lda, w.ldb, seed=11, dist_a="int4")
    C = run_gpu(w.M, w.N, w.K, A, w.lda, B, w.ldb, w.ldc)[0]
    r, c = _sample_indices(w.M, w.N, 11, n_random=20000)
    ref, _ = oracle.entries_f64(w.K, A.numpy(), w.lda, B.numpy(), w.ldb, r, c)
    parity.assert_bitwise(C[r, c], ref, "square4096 int")


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_ragged_workload_sampled(path):
    w = WORKLOADS["ragged"]
    A, B = workload_operands(w)  # NaN padding in A and B
    C = run_gpu(w.M, w.N, w.K, A, w.lda, B, w.ldb, w.ldc, path=path)[0]
    assert np.all(np.isfinite(C))
    _check_sampled(w, C, A, B)


def test_tall_workload_sampled():
    w = WORKLOADS["tall"]
    A, B = workload_operands(w)
    C = run_gpu(w.M, w.N, w.K, A, w.lda, B, w.ldb, w.ldc)[0]
    _check_sampled(w, C, A, B)


def test_shard512_workload_sampled():
    w = WORKLOADS["shard512"]
    A, B = workload_operands(w)
    C = run_gpu(w.M, w.N, w.K, A, w.lda, B, w.ldb, w.ldc)[0]
    _check_sampled(w, C, A, B)


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_batched128_full(path):
    w = WORKLOADS["batched128"]
    A, B = workload_operands(w)
    C = run_gpu(w.M, w.N, w.K, A, w.lda, B, w.ldb, w.ldc, path=path, batch=w.batch,
                strideA=w.strideA, strideB=w.strideB, strideC=w.strideC)
    ref, mag = oracle.sgemm_strided_batched_f64(w.M, w.N, w.K, A.numpy(), w.lda, w.strideA,
                                                B.numpy(), w.ldb, w.strideB, w.batch)
    ratio = parity.assert_within_tolerance(C, ref, mag, w.name)
    print("batched128 %s: max ratio %.3e" % (path, ratio))


# ---------------------------------------------------------------- autotuner
@pytest.mark.parametrize("shape", [(300, 260, 150, 151, 262, 263), (64, 64, 1024, 1024, 64, 64)],
                         ids=lambda s: "x".join(map(str, s[:3])))
def test_autotune_leaves_the_product_in_c(shape):
    M, N, K, lda, ldb, ldc = shape
    A_cpu, B_cpu = operands(M, N, K, lda, ldb, seed=M + 3 * K, dist_a="int4")
    dev = _dev()
    A, B = A_cpu.to(dev), B_cpu.to(dev)
    C = torch.full((M * ldc + GUARD,), SENTINEL, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st, cfg, ms = sg.autotune_raw(M, N, K, A.data_ptr(), lda, 0, B.data_ptr(), ldb, 0,
                                  C.data_ptr(), ldc, 0, 1, stream, reps=2)
    assert st == 0, sg.status_string(st)
    assert sg.config_selectable(cfg) and ms > 0
    torch.cuda.synchronize()
    Ch = C.cpu().numpy()
    got = Ch[np.arange(M)[:, None] * ldc + np.arange(N)[None, :]]
    ref, _ = oracle_full(M, N, K, A_cpu, lda, B_cpu, ldb)
    parity.assert_bitwise(got, ref, "autotune %s" % (shape,))
    assert np.all(Ch[M * ldc:] == SENTINEL)


def test_autotune_tensor_api_batched():
    A_cpu, B_cpu = operands(96, 80, 40, 40, 80, seed=5, dist_a="int4")
    dev = _dev()
    A = torch.stack([A_cpu[: 96 * 40].view(96, 40)] * 3).to(dev) + \
        torch.arange(3, dtype=torch.float32, device=dev).view(3, 1, 1)
    B = torch.stack([B_cpu[: 40 * 80].view(40, 80)] * 3).to(dev)
    cfg, ms, out = sg.autotune(A, B, reps=1)
    assert sg.config_selectable(cfg)
    ref = torch.bmm(A.double().cpu(), B.double().cpu())
    assert torch.equal(out.cpu().double(), ref)
