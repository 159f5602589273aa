"""GPU parity of blockwise attention against the oracle, through the C ABI of
include/attention.h.

O = softmax(scale Q K^T) V per head ("Tiling Strategies" section 5, the
FlashAttention row of the tiling-beyond-GEMM table), causal or not.  The
exponentials make every result real-valued, so the bar is a bound derived from
the arithmetic, per output:

    |O - O_ref| <= (2e-4 + 4 D 2^-24 smax_i) * mag_id,

mag_id = sum_j p_ij |V_jd| (the softmax-weighted |V|) and smax_i = the row's
largest scale * sum_d |q||k|: FP32 scores carry an absolute error up to about
D 2^-24 smax_i, which moves each weight by that much relative (twice through
the normalisation), and the FP32 sums add the 2e-4 share.  Where the result is
unique in FP32 (one allowed key: O = V row) it is checked bit for bit.  K and V
are followed by NaN rows that must never be read; O carries a sentinel guard.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import ATTN_WORKLOADS, attn_operands

import tiled_fp32_gemm_sgemm_amd as sg

pytestmark = pytest.mark.gpu

SENTINEL = -7.25
GUARD = 1024


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def attn_gpu(q, k, v, BH, Sq, Skv, D, scale, causal):
    """CPU float32 buffers in, O (BH, Sq, D) out; checks the guard regions."""
    dev = _dev()
    nan = torch.full((GUARD,), float("nan"))
    qd = q.reshape(-1).to(dev)
    kd = torch.cat([k.reshape(-1), nan]).to(dev)
    vd = torch.cat([v.reshape(-1), nan]).to(dev)
    n_out = BH * Sq * D
    od = torch.full((n_out + GUARD,), SENTINEL, device=dev)
    st = sg.attention_raw(BH, Sq, Skv, D, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                          od.data_ptr(), scale, causal, torch.cuda.current_stream(dev).cuda_stream)
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    oh = od.cpu().numpy()
    assert np.all(oh[n_out:] == SENTINEL), "O written past its end"
    return oh[:n_out].reshape(BH, Sq, D)


def assert_attention_close(got, ref, mag, smax, D, what):
    tol = (2e-4 + 4.0 * D * 2.0 ** -24 * smax)[..., None] * mag
    err = np.abs(got.astype(np.float64) - ref)
    bad = ~(err <= tol)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d of %d outside the bound, first at %s: got %r want %r "
                             "(bound %r)" % (what, int(bad.sum()), bad.size, i, got[i], ref[i],
                                             tol[i]))


def _inputs(BH, Sq, Skv, D, seed):
    gen = torch.Generator("cpu").manual_seed(seed)
    return (torch.randn(BH, Sq, D, generator=gen), torch.randn(BH, Skv, D, generator=gen),
            torch.randn(BH, Skv, D, generator=gen))


SHAPES = [(2, 256, 256, 64), (3, 100, 77, 128), (1, 300, 513, 64), (2, 511, 300, 128),
          (4, 64, 640, 128), (1, 257, 257, 64), (2, 1000, 129, 128), (1, 3, 70, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "BH%d_Sq%d_Skv%d_D%d" % s)
def test_attention_parity(shape, causal):
    BH, Sq, Skv, D = shape
    q, k, v = _inputs(BH, Sq, Skv, D, seed=BH + Sq + Skv + D)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    got = attn_gpu(q, k, v, BH, Sq, Skv, D, scale, causal)
    ref, mag, smax = oracle.attention_f64(q.numpy(), k.numpy(), v.numpy(), BH, Sq, Skv, D,
                                          scale, causal)
    assert_attention_close(got, ref, mag, smax, D, "attention %s causal=%d" % (shape, causal))


@pytest.mark.parametrize("D", [64, 128])
def test_attention_single_allowed_key_is_exact(D):
    # One key: every weight is 2^0 = 1, so O is that value row exactly.
    q, k, v = _inputs(3, 70, 1, D, seed=D)
    got = attn_gpu(q, k, v, 3, 70, 1, D, 0.125, False)
    assert np.array_equal(got, np.broadcast_to(v.numpy(), got.shape))
    # Causal: query 0 sees key 0 only.
    q, k, v = _inputs(2, 300, 300, D, seed=D + 1)
    got = attn_gpu(q, k, v, 2, 300, 300, D, 0.125, True)
    assert np.array_equal(got[:, 0], v.numpy()[:, 0])


def test_attention_degenerate_sizes():
    q, k, v = _inputs(2, 5, 0, 64, seed=3)
    got = attn_gpu(q, torch.zeros(0), torch.zeros(0), 2, 5, 0, 64, 1.0, False)
    assert np.all(got == 0.0) and not np.any(np.signbit(got))
    got = attn_gpu(torch.zeros(0), k, v, 2, 0, 0, 64, 1.0, True)
    assert got.size == 0


def test_attention_invalid_arguments_enqueue_nothing():
    dev = _dev()
    o = torch.full((256,), SENTINEL, device=dev)
    x = torch.zeros(256, device=dev)
    p = x.data_ptr()
    assert sg.attention_raw(1, 2, 2, 32, p, p, p, o.data_ptr(), 1.0) == -1
    assert sg.attention_raw(1, 2, 2, 64, p, p, p, o.data_ptr(), float("nan")) == -1
    assert sg.attention_raw(1, 2, 2, 64, 0, p, p, o.data_ptr(), 1.0) == -3
    torch.cuda.synchronize()
    assert torch.all(o == SENTINEL)


@pytest.mark.parametrize("name", sorted(ATTN_WORKLOADS))
def test_attention_workload_sampled(name):
    """The benchmark shapes, as the benchmark launches them, on sampled rows:
    the first and last query of every 256-query block of two heads, and random
    rows of all heads."""
    w = ATTN_WORKLOADS[name]
    q, k, v = attn_operands(w)
    dev = _dev()
    scale = float(np.float32(1.0 / np.sqrt(w.D)))
    out = sg.attention(q.to(dev).view(w.BH, w.Sq, w.D), k.to(dev).view(w.BH, w.Skv, w.D),
                       v.to(dev).view(w.BH, w.Skv, w.D), scale, w.causal)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(-1, w.D)
    rng = np.random.default_rng(21)
    rows = [h * w.Sq + i for h in (0, w.BH - 1) for b in range(0, w.Sq, 256)
            for i in (b, min(b + 255, w.Sq - 1))]
    rows = np.concatenate([np.asarray(rows, np.int64), rng.integers(0, w.BH * w.Sq, 512)])
    ref, mag, smax = oracle.attention_rows_f64(q.numpy(), k.numpy(), v.numpy(), w.BH, w.Sq,
                                               w.Skv, w.D, scale, rows, w.causal)
    assert_attention_close(got[rows], ref, mag, smax, w.D, "attention workload %s" % name)


def test_attention_tensor_api_matches_torch():
    dev = _dev()
    gen = torch.Generator("cpu").manual_seed(5)
    q = torch.randn(2, 4, 200, 64, generator=gen)
    k = torch.randn(2, 4, 300, 64, generator=gen)
    v = torch.randn(2, 4, 300, 64, generator=gen)
    got = sg.attention(q.to(dev), k.to(dev), v.to(dev), causal=True).cpu().double()
    ref = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double(),
                                                           is_causal=True)
    assert torch.allclose(got, ref, rtol=1e-4, atol=1e-5)
