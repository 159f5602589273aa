"""GPU parity at the size limits, through the C ABI of include/sgemm.h.

* An operand of more than 2^31 elements: row offsets past 32 bits.
* Leading dimensions so large that one tile's rows span more than 2^31 bytes:
  the direct copies' 32-bit buffer offsets cannot reach, so every slice goes
  through the register-staged loads, on every tile configuration; C's rows are
  as far apart, so the stores' offsets pass 32 bits too.
* Batch strides past 2^31 elements.
* A strided batch with more workgroups than one launch holds (2^32 - 1
  work-items): the library splits it over several launches.

Operands are drawn on the device (workloads.device_operand, integers -4..4,
NaN padding) and only the rows the oracle needs are copied back, so the
products are exact: every checked entry must match the oracle bit for bit.
Everything outside C's windows starts as a sentinel and must come back
unchanged.  These need tens of GB of device memory (a 288 GB MI355X holds them).
"""
import numpy as np
import pytest
import torch

import oracle
import parity
from workloads import device_operand

import tiled_fp32_gemm_sgemm_amd as sg

pytestmark = pytest.mark.gpu

SENTINEL = -7.25  # not an integer: no exact product of integer inputs equals it


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _call(M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, batch, path="mfma", config=None):
    stream = torch.cuda.current_stream().cuda_stream
    st = sg.sgemm_strided_batched_raw(M, N, K, A.data_ptr(), lda, sA, B.data_ptr(), ldb, sB,
                                      C.data_ptr(), ldc, sC, batch, stream, path, config)
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()


def _untouched_outside(C, M, N, ldc, stride, batch):
    """Every float of C outside the batch's M x N windows still holds the
    sentinel (counted on the device)."""
    inside = batch * M * N
    return int((C != SENTINEL).sum().item()) == inside and bool(
        torch.all(torch.stack([(C[b * stride: b * stride + M * ldc].view(M, ldc)[:, :N]
                                != SENTINEL).all() for b in range(batch)])).item())


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_operand_beyond_2_31_elements(path):
    dev = _dev()
    M, N, K = 131075, 40, 16411  # A holds 2,151,071,825 > 2^31 elements
    assert M * K > 2 ** 31
    A = device_operand(1, M, K, K, 0, seed=21, device=dev)
    B = device_operand(1, K, N, N, 0, seed=22, device=dev)
    C = torch.full((M * N + 64,), SENTINEL, device=dev)
    _call(M, N, K, A, K, 0, B, N, 0, C, N, 0, 1, path)
    assert bool((C[M * N:] == SENTINEL).all().item())
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, M // 2, M - 3, M - 2, M - 1],
                                     rng.integers(0, M, 60)]))
    A_rows = A.view(M, K)[torch.as_tensor(rows, device=dev)].cpu().numpy()
    B_h = B.cpu().numpy()
    ref, _, _ = oracle.sgemm_f64(len(rows), N, K, A_rows, K, B_h, N)
    got = C[: M * N].view(M, N)[torch.as_tensor(rows, device=dev)].cpu().numpy()
    parity.assert_bitwise(got, ref, "%s M*K > 2^31 rows %s" % (path, rows[:6]))


PATHS = [("mfma", c) for c in range(sg.num_configs())] + [("valu", None)]


@pytest.fixture(scope="module")
def wide_operands():
    """A (70 x 100, lda = 2^25 + 3), B (100 x 50, ldb = 2^26 + 5), C (70 x 50,
    ldc = 2^25 + 1): a 64-row tile of A spans 8.5 GB, a 16-row slice of B
    4.0 GB, more than a 32-bit buffer offset reaches, so no tile can use the
    direct copies."""
    dev = _dev()
    M, N, K = 70, 50, 100
    lda, ldb, ldc = 2 ** 25 + 3, 2 ** 26 + 5, 2 ** 25 + 1
    A = device_operand(1, M, K, lda, 0, seed=23, device=dev)
    B = device_operand(1, K, N, ldb, 0, seed=24, device=dev)
    A_h = A.view(M, lda)[:, :K].cpu().numpy()
    B_h = B.view(K, ldb)[:, :N].cpu().numpy()
    ref, _, _ = oracle.sgemm_f64(M, N, K, np.ascontiguousarray(A_h), K,
                                 np.ascontiguousarray(B_h), N)
    C = torch.empty((M * ldc,), dtype=torch.float32, device=dev)
    yield M, N, K, A, lda, B, ldb, C, ldc, ref
    del A, B, C


@pytest.mark.parametrize("path,config", PATHS,
                         ids=["%s%s" % (p, "" if c is None else c) for p, c in PATHS])
def test_leading_dimensions_beyond_32_bit_offsets(wide_operands, path, config):
    M, N, K, A, lda, B, ldb, C, ldc, ref = wide_operands
    C.fill_(SENTINEL)
    _call(M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, 1, path, config)
    got = C.view(M, ldc)[:, :N].cpu().numpy()
    parity.assert_bitwise(got, ref,
                          "%s cfg %s lda %d ldb %d ldc %d" % (path, config, lda, ldb, ldc))
    assert _untouched_outside(C, M, N, ldc, 0, 1)


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_batch_strides_beyond_2_31_elements(path):
    dev = _dev()
    M, N, K, batch = 50, 60, 70, 3
    sA, sB, sC = 2 ** 31 + 5, 2 ** 31 + 7, 2 ** 31 + 9
    A = device_operand(batch, M, K, K, sA, seed=25, device=dev)
    B = device_operand(batch, K, N, N, sB, seed=26, device=dev)
    C = torch.full(((batch - 1) * sC + M * N,), SENTINEL, device=dev)
    _call(M, N, K, A, K, sA, B, N, sB, C, N, sC, batch, path)
    for b in range(batch):
        A_h = A[b * sA: b * sA + M * K].cpu().numpy()
        B_h = B[b * sB: b * sB + K * N].cpu().numpy()
        ref, _, _ = oracle.sgemm_f64(M, N, K, A_h, K, B_h, N)
        got = C[b * sC: b * sC + M * N].view(M, N).cpu().numpy()
        parity.assert_bitwise(got, ref, "%s batch member %d" % (path, b))
    assert _untouched_outside(C, M, N, N, sC, batch)


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_batch_split_over_launches(path):
    """2^24 + 3 products of 1 x 1 x 2 (one workgroup each): more than
    (2^32 - 1) / 256 workgroups, so at least two launches."""
    dev = _dev()
    M, N, K, batch = 1, 1, 2, 2 ** 24 + 3
    A = device_operand(1, batch, K, K, 0, seed=27, device=dev)  # member b = row b
    B = device_operand(1, batch, K, K, 0, seed=28, device=dev)  # stored K x 1, stride K
    C = torch.full((batch + 16,), SENTINEL, device=dev)
    _call(M, N, K, A, K, K, B, N, K, C, N, 1, batch, path)
    ref, _ = oracle.sgemm_strided_batched_f64(M, N, K, A.cpu().numpy(), K, K, B.cpu().numpy(),
                                              N, K, batch)
    parity.assert_bitwise(C[:batch].cpu().numpy(), ref.reshape(batch),
                          "%s batch %d" % (path, batch))
    assert bool((C[batch:] == SENTINEL).all().item())


@pytest.mark.parametrize("W", [5, 17, 33])
def test_window_sum_beyond_2_31_elements(W):
    """n = 2^31 + 4101 window sums of integers: exact.  Output ranges at the
    start, across element 2^31 and at the end, against the oracle on the same
    stretch of x; one window width per block size."""
    dev = _dev()
    n = 2 ** 31 + 4101
    x = device_operand(1, 1, n + W - 1, n + W - 1, 0, seed=29, device=dev)
    y = torch.full((n + 64,), SENTINEL, device=dev)
    st = sg.window_sum_raw(n, W, x.data_ptr(), y.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    assert bool((y[n:] == SENTINEL).all().item())
    for a, b in ((0, 5000), (2 ** 31 - 3000, 2 ** 31 + 3000), (n - 5000, n)):
        ref, _ = oracle.window_sum_f64(b - a, W, x[a:b + W - 1].cpu().numpy())
        parity.assert_bitwise(y[a:b].cpu().numpy(), ref, "window outputs %d..%d" % (a, b))


def _attention_heads(q, k, v, o, heads, Sq, Skv, D, scale, what):
    from test_gpu_attention import assert_attention_close
    for h in heads:
        qs = q[h * Sq * D:(h + 1) * Sq * D].cpu().numpy()
        ks = k[h * Skv * D:(h + 1) * Skv * D].cpu().numpy()
        vs = v[h * Skv * D:(h + 1) * Skv * D].cpu().numpy()
        ref, mag, smax = oracle.attention_f64(qs, ks, vs, 1, Sq, Skv, D, scale, False)
        got = o[h * Sq * D:(h + 1) * Sq * D].cpu().numpy().reshape(1, Sq, D)
        assert_attention_close(got, ref, mag, smax, D, "%s head %d" % (what, h))


@pytest.mark.parametrize("BH,Sq,Skv,D", [
    (65600, 256, 64, 128),   # Q and O hold 2,149,580,800 > 2^31 elements
    (2 ** 23 + 24, 1, 3, 64),  # more workgroups than one launch holds: two launches
], ids=["q_beyond_2_31", "heads_over_two_launches"])
def test_attention_at_the_size_limits(BH, Sq, Skv, D):
    dev = _dev()
    scale = float(np.float32(1.0 / np.sqrt(D)))
    q = device_operand(1, BH * Sq, D, D, 0, seed=30, device=dev, dist="uniform")
    k = device_operand(1, BH * Skv, D, D, 0, seed=31, device=dev, dist="uniform")
    v = device_operand(1, BH * Skv, D, D, 0, seed=32, device=dev, dist="uniform")
    o = torch.full((BH * Sq * D + 64,), SENTINEL, device=dev)
    st = sg.attention_raw(BH, Sq, Skv, D, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                          scale, False, torch.cuda.current_stream().cuda_stream)
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    assert bool((o[BH * Sq * D:] == SENTINEL).all().item())
    assert not bool((o[:BH * Sq * D] == SENTINEL).any().item())
    per_launch = (2 ** 32 - 1) // 512 // ((Sq + 255) // 256)
    heads = sorted({0, 1, BH // 2, BH - 2, BH - 1} |
                   ({per_launch - 1, per_launch, per_launch + 1} if per_launch < BH else set()))
    _attention_heads(q, k, v, o, heads, Sq, Skv, D, scale, "BH %d Sq %d" % (BH, Sq))


def _conv_images_check(x, wt, y, H, W, C, K, R, S, pad, images, what, n_samples=3000):
    """Sampled outputs of the given images (every border position, all
    channels at the centre, random ones) against the oracle run on that image
    alone."""
    P, Q = sg.conv2d_output_size(H, W, R, S, pad, (1, 1), (1, 1))
    wt_h = wt.cpu().numpy()
    rng = np.random.default_rng(13)
    per_img = P * Q * K
    for n in images:
        x_h = x[n * H * W * C:(n + 1) * H * W * C].cpu().numpy()
        pos = [(p, q) for p in (0, P - 1) for q in range(Q)] + \
              [(p, q) for p in range(P) for q in (0, Q - 1)]
        idx = [(p * Q + q) * K + k for (p, q) in pos for k in (0, K - 1)]
        idx += [((P // 2) * Q + Q // 2) * K + k for k in range(K)]
        idx = np.concatenate([np.asarray(idx, np.int64), rng.integers(0, per_img, n_samples)])
        ref, _ = oracle.conv2d_nhwc_entries_f64(x_h, wt_h, 1, H, W, C, K, R, S, idx, pad)
        got = y[n * per_img:(n + 1) * per_img].cpu().numpy()[idx]
        parity.assert_bitwise(got, ref, "%s image %d" % (what, n))


@pytest.fixture(scope="module")
def conv_large_input():
    """180 images of 112 x 112 x 1024 (2,311,061,504 elements, 9.2 GB),
    3 x 3 filters to 64 channels, padding 1."""
    dev = _dev()
    N, H, W, C, K, R, S = 180, 112, 112, 1024, 64, 3, 3
    x = device_operand(1, N * H * W, C, C, 0, seed=33, device=dev)
    wt = device_operand(1, K * R * S, C, C, 0, seed=34, device=dev)
    y = torch.empty((N * H * W * K + 64,), dtype=torch.float32, device=dev)
    yield N, H, W, C, K, R, S, x, wt, y
    del x, wt, y


CONV_LIMIT_CONFIGS = [None] + [c for c in range(sg.num_configs())
                               if sg.conv2d_config_available(c)]


@pytest.mark.parametrize("config", CONV_LIMIT_CONFIGS,
                         ids=["auto" if c is None else "cfg%d" % c for c in CONV_LIMIT_CONFIGS])
def test_conv_input_beyond_2_31_elements(conv_large_input, config):
    """Each tile addresses its images from the first one, so the direct copies
    serve an input of any total size."""
    N, H, W, C, K, R, S, x, wt, y = conv_large_input
    assert N * H * W * C > 2 ** 31
    y.fill_(SENTINEL)
    st = sg.conv2d_nhwc_raw(N, H, W, C, K, R, S, x.data_ptr(), wt.data_ptr(), y.data_ptr(),
                            (1, 1), (1, 1), (1, 1), torch.cuda.current_stream().cuda_stream,
                            config)
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    n_out = N * H * W * K
    assert bool((y[n_out:] == SENTINEL).all().item())
    assert not bool((y[:n_out] == SENTINEL).any().item())
    _conv_images_check(x, wt, y, H, W, C, K, R, S, (1, 1), (0, N // 2, N - 1),
                       "conv cfg %s" % config, n_samples=1000)


def test_conv_image_beyond_31_bit_offsets():
    """Two images of 1040 x 1040 x 1024 (4.4 GB each): one image is more than
    31-bit offsets reach, so the input is gathered through registers, with
    offsets past 2^31 elements in the second image."""
    dev = _dev()
    N, H, W, C, K, R, S = 2, 1040, 1040, 1024, 8, 1, 1
    x = device_operand(1, N * H * W, C, C, 0, seed=35, device=dev)
    wt = device_operand(1, K * R * S, C, C, 0, seed=36, device=dev)
    n_out = N * H * W * K
    y = torch.full((n_out + 64,), SENTINEL, device=dev)
    st = sg.conv2d_nhwc_raw(N, H, W, C, K, R, S, x.data_ptr(), wt.data_ptr(), y.data_ptr(),
                            (0, 0), (1, 1), (1, 1), torch.cuda.current_stream().cuda_stream)
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    assert bool((y[n_out:] == SENTINEL).all().item())
    _conv_images_check(x, wt, y, H, W, C, K, R, S, (0, 0), (0, 1), "conv 1040x1040x1024")


GENERAL_CONFIGS = [None] + [c for c in range(sg.num_configs()) if sg.config_has_general_form(c)]


@pytest.fixture(scope="module")
def wide_general():
    """Stored A (70 x 100, or 100 x 70 transposed) with lda = 2^25 + 3, stored
    B (100 x 50, or 50 x 100) with ldb = 2^26 + 5, C (70 x 50) with ldc =
    2^25 + 1, all integers; one buffer per operand, as large as either layout
    needs."""
    dev = _dev()
    M, N, K = 70, 50, 100
    lda, ldb, ldc = 2 ** 25 + 3, 2 ** 26 + 5, 2 ** 25 + 1
    A = device_operand(1, max(M, K), max(M, K), lda, 0, seed=37, device=dev)
    B = device_operand(1, max(K, N), max(K, N), ldb, 0, seed=38, device=dev)
    C0 = device_operand(1, M, N, ldc, 0, seed=39, device=dev, pad=SENTINEL)
    C = torch.empty_like(C0)
    yield M, N, K, A, lda, B, ldb, C0, C, ldc
    del A, B, C0, C


@pytest.mark.parametrize("config", GENERAL_CONFIGS,
                         ids=["auto" if c is None else "cfg%d" % c for c in GENERAL_CONFIGS])
@pytest.mark.parametrize("transA,transB", [(0, 0), (1, 0), (0, 1), (1, 1)],
                         ids=["NN", "TN", "NT", "TT"])
def test_general_form_beyond_32_bit_offsets(wide_general, transA, transB, config):
    """C = 2 op(A) op(B) + 0.5 C with every leading dimension past 32-bit
    offsets: staged loads in all four layouts and an epilogue that reads C."""
    M, N, K, A, lda, B, ldb, C0, C, ldc = wide_general
    ra, ca = (K, M) if transA else (M, K)
    rb, cb = (N, K) if transB else (K, N)
    C.copy_(C0)
    st = sg.sgemm_ex_raw(transA, transB, M, N, K, 2.0, A.data_ptr(), lda, B.data_ptr(), ldb,
                         0.5, C.data_ptr(), ldc, torch.cuda.current_stream().cuda_stream, config)
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    A_h = np.ascontiguousarray(A[: ra * lda].view(ra, lda)[:, :ca].cpu().numpy())
    B_h = np.ascontiguousarray(B[: rb * ldb].view(rb, ldb)[:, :cb].cpu().numpy())
    C_h = np.ascontiguousarray(C0[: M * ldc].view(M, ldc)[:, :N].cpu().numpy())
    ref, _, _ = oracle.sgemm_ex_f64(bool(transA), bool(transB), M, N, K, 2.0, A_h, ca, B_h, cb,
                                    0.5, C_h, N)
    got = C[: M * ldc].view(M, ldc)[:, :N].cpu().numpy()
    parity.assert_bitwise(got, ref, "general %d%d cfg %s" % (transA, transB, config))
    assert int((C != C0).sum().item()) <= M * N  # nothing outside the window changed
    assert torch.equal(C[M * ldc - ldc + N:], C0[M * ldc - ldc + N:])
