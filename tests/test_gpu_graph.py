"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph).

Each entry point only enqueues kernels on the caller's stream (no memset, no
allocation, no synchronisation), so it can be captured.  Each test captures
calls into static output buffers, then replays the graph several times.
Between replays it does eager work of its own: the outputs are overwritten
with NaN and other library calls run on other operands.  Every replay must
reproduce the eager result bit for bit, because the same kernels run on the
same inputs.
"""
import numpy as np
import pytest
import torch

import tiled_fp32_gemm_sgemm_amd as sg

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _replays_match(capture, outputs, eager_between):
    """capture() enqueues the calls; outputs are the tensors they write."""
    # Eager reference, then the graph (warm-up on a side stream first, as
    # torch's capture rules ask).
    capture()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        capture()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for o in outputs:
            o.fill_(float("nan"))
        eager_between()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, want in zip(outputs, ref):
            assert torch.equal(o.view(torch.int32), want.view(torch.int32)), \
                "replay %d differs from the eager result" % r


def _other_work(dev):
    a = torch.randn(300, 200, device=dev)
    b = torch.randn(200, 100, device=dev)

    def run():
        sg.sgemm(a, b)
    return run


def test_graph_sgemm_and_batched():
    dev = _dev()
    gen = torch.Generator(device=dev).manual_seed(3)
    A = torch.randn(1000, 900, device=dev, generator=gen)
    B = torch.randn(900, 700, device=dev, generator=gen)
    C = torch.empty(1000, 700, device=dev)
    Ab = torch.randn(6, 130, 70, device=dev, generator=gen)
    Bb = torch.randn(6, 70, 90, device=dev, generator=gen)
    Cb = torch.empty(6, 130, 90, device=dev)

    def capture():
        sg.sgemm(A, B, C)
        sg.sgemm_strided_batched(Ab, Bb, Cb)
        sg.sgemm(A[:64, :64], B[:64, :64], C[:64, :64], path="valu")
    _replays_match(capture, [C, Cb], _other_work(dev))


def test_graph_general_form():
    dev = _dev()
    gen = torch.Generator(device=dev).manual_seed(5)
    At = torch.randn(513, 257, device=dev, generator=gen)  # stored K x M
    B = torch.randn(513, 300, device=dev, generator=gen)
    C0 = torch.randn(257, 300, device=dev, generator=gen)
    C = torch.empty_like(C0)

    def capture():
        torch.mul(C0, 1.0, out=C)  # the graph's own reset (a kernel), so beta reads the same C
        sg.sgemm_ex(At, B, C, alpha=1.5, beta=-0.5, transA=True)
    _replays_match(capture, [C], _other_work(dev))


def test_graph_window_conv_attention():
    dev = _dev()
    gen = torch.Generator(device=dev).manual_seed(7)
    x = torch.rand(100003 + 4, device=dev, generator=gen)
    y = torch.empty(100003, device=dev)
    xi = torch.randn(2, 9, 11, 64, device=dev, generator=gen)
    wt = torch.randn(40, 3, 3, 64, device=dev, generator=gen)
    yc = torch.empty(2, 9, 11, 40, device=dev)
    q = torch.randn(2, 300, 64, device=dev, generator=gen)
    k = torch.randn(2, 513, 64, device=dev, generator=gen)
    v = torch.randn(2, 513, 64, device=dev, generator=gen)
    o = torch.empty(2, 300, 64, device=dev)

    def capture():
        sg.window_sum(x, 5, out=y)
        sg.conv2d_nhwc(xi, wt, pad=1, out=yc)
        sg.attention(q, k, v, causal=True, out=o)
    _replays_match(capture, [y, yc, o], _other_work(dev))
    assert np.isfinite(o.cpu().numpy()).all()


def test_graph_splitk():
    """Split-K in a graph: the workspace counters must be back at zero after
    every replay (the join resets them; no memset is recorded)."""
    dev = _dev()
    gen = torch.Generator(device=dev).manual_seed(13)
    A = torch.randn(200, 3000, device=dev, generator=gen)
    B = torch.randn(3000, 150, device=dev, generator=gen)
    C = torch.empty(200, 150, device=dev)
    A2 = torch.randn(64, 5000, device=dev, generator=gen)
    B2 = torch.randn(5000, 96, device=dev, generator=gen)
    C2 = torch.empty(64, 96, device=dev)
    n1 = sg.splitk_plan(200, 150, 3000, 6)[2]
    n2 = sg.splitk_plan(64, 96, 5000, 4)[2]
    assert n1 > 0 and n2 > 0
    ws = torch.zeros(max(n1, n2), dtype=torch.uint8, device=dev)

    def capture():
        sg.sgemm_splitk(A, B, C, splits=6, workspace=ws)
        sg.sgemm_splitk(A2, B2, C2, splits=4, workspace=ws)
    _replays_match(capture, [C, C2], _other_work(dev))
    assert torch.count_nonzero(ws[:sg.SPLITK_HEADER_BYTES]).item() == 0


def test_graph_hybrid_splitk_and_conv():
    """Hybrid plans (whole tiles plus the chunks of the last partial layer),
    a product and a convolution, captured on one workspace."""
    dev = _dev()
    gen = torch.Generator(device=dev).manual_seed(17)
    M, N, K = 3300, 300, 1000
    assert sg.splitk_plan_full_tiles(M, N, K) > 0
    A = torch.randn(M, K, device=dev, generator=gen)
    B = torch.randn(K, N, device=dev, generator=gen)
    C = torch.empty(M, N, device=dev)
    xi = torch.randn(40, 15, 15, 96, device=dev, generator=gen)
    wt = torch.randn(96, 3, 3, 96, device=dev, generator=gen)
    yc = torch.empty(40, 15, 15, 96, device=dev)
    plan = sg.conv2d_splitk_plan(40, 15, 15, 96, 96, 3, 3, 1)
    assert plan[1] > 1 and plan[3] > 0
    ws = torch.zeros(max(sg.splitk_plan(M, N, K)[2], plan[2]), dtype=torch.uint8, device=dev)

    def capture():
        sg.sgemm_splitk(A, B, C, workspace=ws)
        sg.conv2d_nhwc_splitk(xi, wt, pad=1, out=yc, workspace=ws)
    _replays_match(capture, [C, yc], _other_work(dev))
    assert torch.count_nonzero(ws[:sg.SPLITK_HEADER_BYTES]).item() == 0


def test_graph_general_splitk():
    """The general form split over k, two layouts with beta != 0, captured on
    one workspace (C reset inside the graph by a kernel)."""
    dev = _dev()
    gen = torch.Generator(device=dev).manual_seed(19)
    At = torch.randn(4096, 300, device=dev, generator=gen)   # stored K x M
    B = torch.randn(4096, 200, device=dev, generator=gen)
    C0 = torch.randn(300, 200, device=dev, generator=gen)
    C = torch.empty_like(C0)
    A2 = torch.randn(128, 3000, device=dev, generator=gen)
    Bt2 = torch.randn(256, 3000, device=dev, generator=gen)  # stored N x K
    C20 = torch.randn(128, 256, device=dev, generator=gen)
    C2 = torch.empty_like(C20)
    n1 = sg.ex_splitk_plan(300, 200, 4096, True, False, 5)[2]
    n2 = sg.ex_splitk_plan(128, 256, 3000, False, True, 3)[2]
    assert n1 > 0 and n2 > 0
    ws = torch.zeros(max(n1, n2), dtype=torch.uint8, device=dev)

    def capture():
        torch.mul(C0, 1.0, out=C)
        sg.sgemm_ex_splitk(At, B, C, alpha=1.5, beta=-0.5, transA=True, splits=5, workspace=ws)
        torch.mul(C20, 1.0, out=C2)
        sg.sgemm_ex_splitk(A2, Bt2, C2, alpha=0.5, beta=2.0, transB=True, splits=3,
                           workspace=ws)
    _replays_match(capture, [C, C2], _other_work(dev))
    assert torch.count_nonzero(ws[:sg.SPLITK_HEADER_BYTES]).item() == 0


def test_host_threads_on_their_own_streams():
    """The library keeps no mutable global state: four host threads, each on
    its own stream, calling different entry points at once, give the same
    bits as the same calls made one after another."""
    import threading
    dev = _dev()
    gen = torch.Generator(device=dev).manual_seed(11)
    jobs = []
    for t in range(4):
        A = torch.randn(500 + 37 * t, 300 + 11 * t, device=dev, generator=gen)
        B = torch.randn(300 + 11 * t, 400 - 13 * t, device=dev, generator=gen)
        jobs.append((A, B, torch.empty(A.shape[0], B.shape[1], device=dev)))
    xs = torch.rand(50000, device=dev, generator=gen)
    ref = [sg.sgemm(A, B) for A, B, _ in jobs]
    ref_w = sg.window_sum(xs, 7)
    torch.cuda.synchronize()
    out_w = torch.empty_like(ref_w)
    errors = []

    def work(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(20):
                    A, B, C = jobs[t]
                    sg.sgemm(A, B, C, path="valu" if t == 3 else "mfma")
                    if t == 0:
                        sg.window_sum(xs, 7, out=out_w)
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t, (A, B, C) in enumerate(jobs):
        want = ref[t] if t != 3 else sg.sgemm(A, B, path="valu")
        torch.cuda.synchronize()
        assert torch.equal(C, want), "thread %d" % t
    assert torch.equal(out_w, ref_w)
