"""GPU parity of the general form C = alpha op(A) op(B) + beta C (MI355X).

Every case runs through the C ABI (sgemm_ex / sgemm_ex_strided_batched /
sgemm_ex_with_config) and is compared with the oracle's general form, element
by element: bit for bit where the inputs are small integers and the scalars
are dyadic (every partial sum is exact, so the result is unique), within
|C - C_ref| <= 2e-4 * (|alpha| |A||B| + |beta| |C|) otherwise.  C's padding
past each row's N entries and the memory past the last row hold a sentinel
that must survive.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
import tiled_fp32_gemm_sgemm_amd as sg
from workloads import matrix, stored_operands

pytestmark = pytest.mark.gpu

SENTINEL = -7.25
GUARD = 257
LAYOUTS = [(0, 0), (1, 0), (0, 1), (1, 1)]
LAYOUT_IDS = ["nn", "tn", "nt", "tt"]

_rng = np.random.default_rng(1234)
SHAPES = [(1, 1, 1), (33, 65, 17), (65, 63, 15), (127, 129, 31), (128, 128, 16),
          (255, 257, 33), (257, 129, 300), (100, 200, 3), (3, 5, 299), (200, 192, 1000),
          (130, 260, 515), (64, 64, 64)]


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _lds(tA, tB, M, N, K, seed):
    r = np.random.default_rng(seed)
    lda = (M if tA else K) + int(r.integers(0, 4))
    ldb = (K if tB else N) + int(r.integers(0, 4))
    ldc = N + int(r.integers(0, 6))
    return lda, ldb, ldc


def run_ex(tA, tB, M, N, K, alpha, A_cpu, lda, B_cpu, ldb, beta, C_cpu, ldc, config=None,
           batch=1, strideA=0, strideB=0, strideC=None):
    """One call; returns the C windows (batch, M, N) after checking that
    nothing outside them changed."""
    dev = _dev()
    one_c = M * ldc
    if strideC is None:
        strideC = one_c
    c_len = (batch - 1) * strideC + one_c
    C0 = torch.full((c_len + GUARD,), SENTINEL, dtype=torch.float32)
    win = np.zeros(c_len + GUARD, dtype=bool)
    for b in range(batch):
        idx = b * strideC + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
        win[idx] = True
        idx_t = torch.from_numpy(idx.ravel())
        if C_cpu is not None:
            C0[idx_t] = C_cpu[idx_t]
        else:
            C0[idx_t] = float("nan")  # never read when beta == 0
    A = A_cpu.to(dev) if A_cpu is not None else None
    B = B_cpu.to(dev) if B_cpu is not None else None
    C = C0.to(dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = sg.sgemm_ex_raw(tA, tB, M, N, K, alpha, A.data_ptr() if A is not None else 0, lda,
                         B.data_ptr() if B is not None else 0, ldb, beta, C.data_ptr(), ldc,
                         stream, config, batch, strideA, strideB, strideC)
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    Ch = C.cpu().numpy()
    assert np.all(Ch[~win] == SENTINEL), "C written outside its M x N window(s)"
    out = np.empty((batch, M, N), np.float32)
    for b in range(batch):
        out[b] = Ch[b * strideC + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]]
    return out


def ref_ex(tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    out, mag, _ = oracle.sgemm_ex_f64(bool(tA), bool(tB), M, N, K, alpha,
                                      A.numpy() if A is not None else None, lda,
                                      B.numpy() if B is not None else None, ldb, beta,
                                      C.numpy() if C is not None else None, ldc)
    return out, mag


def _case(tA, tB, shape, seed, dist):
    M, N, K = shape
    lda, ldb, ldc = _lds(tA, tB, M, N, K, seed)
    A, B = stored_operands(bool(tA), bool(tB), M, N, K, lda, ldb, seed, dist)
    C = matrix(M, N, ldc, seed + 1, dist)
    return lda, ldb, ldc, A, B, C


# ---------------------------------------------------------------- every layout, auto tile
@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("scalars", [(1.0, 0.0), (2.0, -1.0), (-0.5, 0.25)],
                         ids=["a1b0", "a2bm1", "am05b025"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_general_integer_bitwise(shape, scalars, layout):
    tA, tB = layout
    alpha, beta = scalars
    M, N, K = shape
    lda, ldb, ldc, A, B, C = _case(tA, tB, shape, M * 5 + N + 7 * K + tA + 2 * tB, "int4")
    got = run_ex(tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C if beta else None, ldc)[0]
    ref, _ = ref_ex(tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
    parity.assert_bitwise(got, ref, "ex %s %s %s" % (layout, scalars, shape))


@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_general_uniform_tolerance(shape, layout):
    tA, tB = layout
    M, N, K = shape
    lda, ldb, ldc, A, B, C = _case(tA, tB, shape, M + N + K + 11, "uniform")
    got = run_ex(tA, tB, M, N, K, 0.75, A, lda, B, ldb, -1.5, C, ldc)[0]
    ref, mag = ref_ex(tA, tB, M, N, K, 0.75, A, lda, B, ldb, -1.5, C, ldc)
    parity.assert_within_tolerance(got, ref, mag, "ex uniform %s %s" % (layout, shape))


# ---------------------------------------------------------------- every general tile
GENERAL_CONFIGS = [c for c in range(sg.num_configs()) if sg.config_has_general_form(c)]


def test_general_configs_exist():
    assert len(GENERAL_CONFIGS) >= 4
    assert sg.select_general_config(4096, 4096, 4096) in GENERAL_CONFIGS


@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("config", GENERAL_CONFIGS, ids=lambda c: "cfg%d" % c)
# 520 x 530 holds whole interior tiles of every size (up to 256 x 256) beside
# ragged edge tiles: interior tiles read C ahead of their stores, edge tiles
# element by element.
@pytest.mark.parametrize("shape", [(33, 65, 17), (257, 129, 300), (200, 192, 1000),
                                   (130, 260, 515), (3, 5, 299), (520, 530, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_general_every_tile_bitwise(shape, config, layout):
    tA, tB = layout
    M, N, K = shape
    lda, ldb, ldc, A, B, C = _case(tA, tB, shape, 3 * M + N + K + config, "int4")
    got = run_ex(tA, tB, M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, config=config)[0]
    ref, _ = ref_ex(tA, tB, M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc)
    parity.assert_bitwise(got, ref, "ex cfg%d %s %s" % (config, layout, shape))


# ---------------------------------------------------------------- scalars and degenerate cases
@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
def test_beta_zero_never_reads_c(layout):
    # C's window holds NaN (run_ex fills it so when no C is given): it must not leak.
    tA, tB = layout
    M, N, K = 77, 91, 45
    lda, ldb, ldc, A, B, _ = _case(tA, tB, (M, N, K), 5, "int4")
    got = run_ex(tA, tB, M, N, K, -3.0, A, lda, B, ldb, 0.0, None, ldc)[0]
    assert np.all(np.isfinite(got))
    ref, _ = ref_ex(tA, tB, M, N, K, -3.0, A, lda, B, ldb, 0.0, None, ldc)
    parity.assert_bitwise(got, ref, "beta 0")


@pytest.mark.parametrize("beta", [0.0, 1.0, -2.0])
def test_alpha_zero_scales_c_without_reading_a_b(beta):
    M, N, K, ldc = 70, 50, 33, 53
    C = matrix(M, N, ldc, 3, "int4")
    # A and B are NULL: alpha == 0 means they are not read.
    got = run_ex(1, 0, M, N, K, 0.0, None, M, None, N, beta, C if beta else None, ldc)[0]
    ref, _ = ref_ex(1, 0, M, N, K, 0.0, None, M, None, N, beta, C, ldc)
    parity.assert_bitwise(got, ref, "alpha 0 beta %g" % beta)


@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_k_zero(beta):
    M, N, ldc = 40, 30, 31
    C = matrix(M, N, ldc, 4, "int4")
    A = torch.zeros(4)
    B = torch.zeros(4)
    got = run_ex(0, 1, M, N, 0, 3.0, A, 1, B, 1, beta, C if beta else None, ldc)[0]
    ref, _ = ref_ex(0, 1, M, N, 0, 3.0, A, 1, B, 1, beta, C, ldc)
    parity.assert_bitwise(got, ref, "K 0")
    if beta == 0.0:
        assert not np.any(np.signbit(got))


def test_worked_example_as_a_transpose_b():
    # "CMU DLSys Lecture 12", section 4: [2, 3]^T [5, 7] in the lecture's own
    # C = A^T B form, A stored as the 1 x 2 strip.
    A = torch.tensor([2.0, 3.0])
    B = torch.tensor([5.0, 7.0])
    got = run_ex(1, 0, 2, 2, 1, 1.0, A, 2, B, 2, 0.0, None, 2)[0]
    assert got.ravel().tolist() == [10.0, 14.0, 15.0, 21.0]


@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
def test_general_batched(layout):
    tA, tB = layout
    M, N, K, batch = 96, 80, 72, 5
    lda, ldb, ldc = (M if tA else K) + 1, (K if tB else N) + 3, N + 2
    ra, rb = (K if tA else M), (N if tB else K)
    sA, sB, sC = ra * lda + 7, rb * ldb + 5, M * ldc + 9
    A = torch.cat([stored_operands(bool(tA), bool(tB), M, N, K, lda, ldb, 40 + b, "int4")[0]
                   for b in range(batch)])
    B = torch.cat([stored_operands(bool(tA), bool(tB), M, N, K, lda, ldb, 80 + b, "int4")[1]
                   for b in range(batch)])
    # re-lay with the chosen strides (NaN in the gaps)
    A_s = torch.full(((batch - 1) * sA + ra * lda,), float("nan"))
    B_s = torch.full(((batch - 1) * sB + rb * ldb,), float("nan"))
    for b in range(batch):
        A_s[b * sA:b * sA + ra * lda] = A[b * ra * lda:(b + 1) * ra * lda]
        B_s[b * sB:b * sB + rb * ldb] = B[b * rb * ldb:(b + 1) * rb * ldb]
    C_s = torch.full(((batch - 1) * sC + M * ldc,), float("nan"))
    for b in range(batch):
        C_s[b * sC:b * sC + M * ldc] = matrix(M, N, ldc, 120 + b, "int4")
    got = run_ex(tA, tB, M, N, K, -1.0, A_s, lda, B_s, ldb, 2.0, C_s, ldc, batch=batch,
                 strideA=sA, strideB=sB, strideC=sC)
    for b in range(batch):
        ref, _ = ref_ex(tA, tB, M, N, K, -1.0, A_s[b * sA:], lda, B_s[b * sB:], ldb, 2.0,
                        C_s[b * sC:], ldc)
        parity.assert_bitwise(got[b], ref, "batched %s member %d" % (layout, b))


def test_tensor_api_matches_torch():
    dev = _dev()
    g = torch.Generator("cpu").manual_seed(9)
    At = torch.randint(-4, 5, (300, 200), generator=g).float()   # stored K x M
    Bt = torch.randint(-4, 5, (250, 300), generator=g).float()   # stored N x K
    C = torch.randint(-4, 5, (200, 250), generator=g).float()
    out = sg.sgemm_ex(At.to(dev), Bt.to(dev), C.to(dev), alpha=2.0, beta=-1.0, transA=True,
                      transB=True)
    ref = 2.0 * (At.double().T @ Bt.double().T) - C.double()
    assert torch.equal(out.cpu().double(), ref)


# ---------------------------------------------------------------- full size, sampled
@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
def test_general_4096_sampled(layout):
    tA, tB = layout
    M = N = K = 4096
    A, B = stored_operands(bool(tA), bool(tB), M, N, K, 4096, 4096, 21, "normal")
    C = matrix(M, N, N, 22, "normal")
    got = run_ex(tA, tB, M, N, K, 1.0 / 64, A, 4096, B, 4096, 0.5, C, N)[0]
    r = np.concatenate([np.arange(0, M, 97), _rng.integers(0, M, 3000)])
    c = np.concatenate([np.arange(0, N, 89)[: len(np.arange(0, M, 97))], _rng.integers(0, N, 3000)])
    ref, mag = oracle.ex_entries_f64(bool(tA), bool(tB), K, 1.0 / 64, A.numpy(), 4096,
                                     B.numpy(), 4096, 0.5, C.numpy(), N, r, c)
    parity.assert_within_tolerance(got[r, c], ref, mag, "4096 %s" % (layout,))
