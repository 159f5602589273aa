"""GPU parity of the split-K entry point (sgemm_splitk) against the oracle.

The k range is cut into chunks whose partial tiles join inside the launch, in
chunk order.  Integer-valued inputs keep every partial sum exact, so the
result must equal the oracle bit for bit for any chunk count; real-valued
inputs are held to the parity bound 2e-4 * (|A||B|)_ij and must repeat bit
for bit from call to call (the join order does not depend on timing).  C's
row padding and a guard after C hold a sentinel that must come back
unchanged, A's and B's padding is NaN, and after every call the workspace's
per-tile counters must be zero again, so the next call can reuse it, whatever
its shape.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import parity
from workloads import WORKLOADS, operands, workload_operands

import tiled_fp32_gemm_sgemm_amd as sg
from tiled_fp32_gemm_sgemm_amd import _native

pytestmark = pytest.mark.gpu

SENTINEL = -7.25
GUARD = 257
SK_CONFIGS = [c for c in range(sg.num_configs()) if sg.config_has_splitk(c)]


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _tile(config):
    bm, bn, bk = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    thr = ctypes.c_int()
    buf = ctypes.create_string_buffer(64)
    st = _native.lib().sgemm_config_info(config, buf, 64, ctypes.byref(bm), ctypes.byref(bn),
                                         ctypes.byref(bk), ctypes.byref(thr))
    assert st == 0
    return bm.value, bn.value, bk.value


def run_splitk(M, N, K, A_cpu, lda, B_cpu, ldb, ldc, config, splits, ws=None, lib=None):
    """One sgemm_splitk call; returns (C window, workspace tensor, plan)."""
    dev = _dev()
    lib = lib or _native.lib()
    A, B = A_cpu.to(dev), B_cpu.to(dev)
    C = torch.full((M * ldc + GUARD,), SENTINEL, dtype=torch.float32, device=dev)
    plan_cfg, plan_splits = ctypes.c_int(), ctypes.c_int64()
    nbytes = lib.sgemm_splitk_plan(config, M, N, K, splits, ctypes.byref(plan_cfg),
                                   ctypes.byref(plan_splits))
    assert nbytes >= 0, sg.status_string(int(nbytes))
    if ws is None:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
    assert ws.numel() >= nbytes
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    st = lib.sgemm_splitk(config, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(),
                          ldc, splits, ws.data_ptr(), ws.numel(), stream)
    assert st == 0, sg.status_string(st)
    torch.cuda.synchronize()
    Ch = C.cpu().numpy()
    idx = np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
    written = np.zeros(Ch.size, dtype=bool)
    written[idx] = True
    assert np.all(Ch[~written] == SENTINEL), "C written outside its M x N window"
    if plan_splits.value > 1:
        assert torch.count_nonzero(ws[:sg.SPLITK_HEADER_BYTES]).item() == 0, "counters not reset"
    return Ch[idx], ws, (plan_cfg.value, plan_splits.value)


# (M, N, K, lda, ldb, ldc): ragged edges, partial last slices, odd leading
# dimensions, chunks that do not divide K evenly.
SHAPES = [(257, 129, 1000, 1003, 131, 133),
          (64, 640, 513, 515, 640, 641),
          (130, 70, 3001, 3003, 70, 75),
          (65, 63, 150, 151, 65, 66)]


@pytest.mark.parametrize("splits", [2, 3, 7])
@pytest.mark.parametrize("config", SK_CONFIGS)
def test_splitk_bitwise(config, splits):
    ws = None
    for i, (M, N, K, lda, ldb, ldc) in enumerate(SHAPES):
        A, B = operands(M, N, K, lda, ldb, seed=31 * config + 7 * splits + i, dist_a="int4")
        got, ws, plan = run_splitk(M, N, K, A, lda, B, ldb, ldc, config, splits, ws=ws)
        assert plan[0] == config
        ref, _, _ = oracle.sgemm_f64(M, N, K, A.numpy(), lda, B.numpy(), ldb)
        parity.assert_bitwise(got, ref, "splitk cfg%d splits=%d %s" % (config, splits,
                                                                    SHAPES[i]))
        # The same workspace, grown only when a later shape needs more.
        nxt = SHAPES[(i + 1) % len(SHAPES)]
        need = sg.splitk_plan(nxt[0], nxt[1], nxt[2], splits, config)[2]
        if ws.numel() < need:
            ws = None


def test_splitk_more_splits_than_slices():
    # K = 40 has three 16-wide (or one 64-wide) slices: the plan caps the count.
    M, N, K = 100, 90, 40
    A, B = operands(M, N, K, K, N, seed=5, dist_a="int4")
    for config in SK_CONFIGS:
        got, _, plan = run_splitk(M, N, K, A, K, B, N, N, config, 64)
        bk = _tile(config)[2]
        slices = -(-K // bk)
        kchunk = -(-slices // min(64, slices)) * bk
        assert plan[1] == -(-K // kchunk)
        ref, _, _ = oracle.sgemm_f64(M, N, K, A.numpy(), K, B.numpy(), N)
        parity.assert_bitwise(got, ref, "cfg%d" % config)


def test_splitk_degenerate():
    dev = _dev()
    for M, N, K in [(0, 5, 7), (5, 0, 7), (33, 17, 0)]:
        if M and N:
            A, B = operands(M, N, K, max(K, 1), max(N, 1), seed=1, dist_a="int4")
            got, _, _ = run_splitk(M, N, K, A, max(K, 1), B, max(N, 1), N, SK_CONFIGS[0], 4)
            assert np.all(got == 0.0) and not np.any(np.signbit(got))
        else:
            C = torch.full((GUARD,), SENTINEL, device=dev)
            st = _native.lib().sgemm_splitk(-1, M, N, K, None, max(K, 1), None, max(N, 1),
                                            C.data_ptr(), max(N, 1), 0, None, 0, None)
            assert st == 0
            assert torch.all(C == SENTINEL)


@pytest.mark.parametrize("shape", [(512, 4096, 4096), (256, 4096, 4096), (96, 200, 20000)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("splits", [0, 4, 8])
def test_splitk_real_valued_repeatable(shape, splits):
    """Normal-like data: within the parity bound on sampled entries (all of
    them for the small shape), and bit-identical across repeated calls."""
    M, N, K = shape
    A, B = operands(M, N, K, K, N, seed=M + N + K, dist_a="normal", scale_a=K ** -0.5,
                    scale_b=K ** -0.5)
    got, ws, plan = run_splitk(M, N, K, A, K, B, N, N, -1, splits)
    again, _, _ = run_splitk(M, N, K, A, K, B, N, N, -1, splits, ws=ws)
    assert np.array_equal(got.view(np.int32), again.view(np.int32)), "join not repeatable"
    g = np.random.default_rng(M)
    r = np.concatenate([np.arange(M), g.integers(0, M, 4000)])
    c = np.concatenate([(np.arange(M) * 37) % N, g.integers(0, N, 4000)])
    ref, mag = oracle.entries_f64(K, A.numpy(), K, B.numpy(), N, r, c)
    ratio = parity.assert_within_tolerance(got[r, c], ref, mag, "splitk %s plan %s" % (shape,
                                                                                       plan))
    print("splitk %s splits=%d plan=%s: max |err|/(|A||B|) = %.3e" % (shape, splits, plan, ratio))


def test_shard512_workload_splitk_sampled():
    """The 512 x 4096 x 4096 row shard (one GPU's eighth of 4096^3) at the
    split count the bench's split-K line times, sampled against the oracle."""
    w = WORKLOADS["shard512"]
    A, B = workload_operands(w)
    got, _, plan = run_splitk(w.M, w.N, w.K, A, w.lda, B, w.ldb, w.ldc, -1, 8)
    assert plan[1] == 8
    g = np.random.default_rng(w.seed)
    r = g.integers(0, w.M, 6000)
    c = g.integers(0, w.N, 6000)
    ref, mag = oracle.entries_f64(w.K, A.numpy(), w.lda, B.numpy(), w.ldb, r, c)
    parity.assert_within_tolerance(got[r, c], ref, mag, "shard512 splitk")


@pytest.mark.parametrize("config", SK_CONFIGS)
def test_racecheck_splitk_bitwise(config):
    """The race-check build (NaN-poisoned LDS, reversed tile order) through
    the split-K join."""
    rc = _native.racecheck_lib()
    M, N, K, lda, ldb, ldc = SHAPES[0]
    A, B = operands(M, N, K, lda, ldb, seed=99 + config, dist_a="int4")
    got, _, _ = run_splitk(M, N, K, A, lda, B, ldb, ldc, config, 5, lib=rc)
    ref, _, _ = oracle.sgemm_f64(M, N, K, A.numpy(), lda, B.numpy(), ldb)
    parity.assert_bitwise(got, ref, "racecheck splitk cfg%d" % config)


# Output tiles and chunks of the time model's plans: 16 tiles x 16 chunks,
# 128 tiles x 2 chunks (counters past the first 64 tiles), 16 tiles x 8.
SEQUENCE = [(128, 1024, 16384), (512, 1024, 2048), (128, 1024, 16384), (512, 512, 8192)]


def test_splitk_workspace_serves_any_shape():
    """One workspace through calls whose tile counts and chunk counts differ:
    the counters sit at fixed places, so a call with more tiles than the one
    before never reads the earlier call's partial sums as counters."""
    plans = [sg.splitk_plan(M, N, K) for M, N, K in SEQUENCE]
    assert all(p[1] > 1 for p in plans), plans
    tiles = []
    for (M, N, K), (cfg, _, _) in zip(SEQUENCE, plans):
        bm, bn, _ = _tile(cfg)
        tiles.append(-(-M // bm) * -(-N // bn))
    assert min(tiles) <= 64 < max(tiles), tiles
    ws = torch.zeros(max(p[2] for p in plans), dtype=torch.uint8, device=_dev())
    for i, (M, N, K) in enumerate(SEQUENCE):
        A, B = operands(M, N, K, K, N, seed=400 + i, dist_a="int4")
        got, _, plan = run_splitk(M, N, K, A, K, B, N, N, -1, 0, ws=ws)
        assert plan[1] == plans[i][1]
        ref, _, _ = oracle.sgemm_f64(M, N, K, A.numpy(), K, B.numpy(), N)
        parity.assert_bitwise(got, ref, "splitk sequence %s" % ((M, N, K),))


def test_splitk_default_workspace():
    """The binding's own workspace (kept per device and stream, grown on
    demand) through the same sequence, bit-exact on integer inputs."""
    dev = _dev()
    for i, (M, N, K) in enumerate(SEQUENCE):
        A, B = operands(M, N, K, K, N, seed=500 + i, dist_a="int4")
        C = sg.sgemm_splitk(A.view(M, K).to(dev), B.view(K, N).to(dev))
        got = C.cpu().numpy()
        ref, _, _ = oracle.sgemm_f64(M, N, K, A.numpy(), K, B.numpy(), N)
        parity.assert_bitwise(got, ref, "default workspace %s" % ((M, N, K),))
    s = torch.cuda.current_stream(dev)
    ws = sg.splitk_workspace(dev, 0, s)
    assert torch.count_nonzero(ws[:sg.SPLITK_HEADER_BYTES]).item() == 0


def test_splitk_two_streams_default_workspaces():
    """Two streams calling the binding at once with no workspace of their
    own: each stream gets its own, and both sequences equal the serial
    results bit for bit."""
    dev = _dev()
    jobs = []
    for t in range(2):
        for i, (M, N, K) in enumerate(SEQUENCE):
            A, B = operands(M, N, K, K, N, seed=600 + 10 * t + i, dist_a="int4")
            jobs.append((t, A.view(M, K).to(dev), B.view(K, N).to(dev)))
    ref = [sg.sgemm_splitk(A, B) for _, A, B in jobs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev) for _ in range(2)]
    outs = [None] * len(jobs)
    for rep in range(3):
        for j, (t, A, B) in enumerate(jobs):
            with torch.cuda.stream(streams[t]):
                outs[j] = sg.sgemm_splitk(A, B)
    torch.cuda.synchronize()
    for j, (t, _, _) in enumerate(jobs):
        assert torch.equal(outs[j], ref[j]), "stream %d job %d" % (t, j)
    keys = {(dev.index, int(s.cuda_stream)) for s in streams}
    assert len(keys) == 2


def test_splitk_default_workspaces_are_bounded():
    """Calls on more streams than the binding keeps workspaces for: the
    least recently used are dropped, and every result is still exact."""
    from tiled_fp32_gemm_sgemm_amd import api
    dev = _dev()
    M, N, K = 512, 512, 8192
    A, B = operands(M, N, K, K, N, seed=650, dist_a="int4")
    A, B = A.view(M, K).to(dev), B.view(K, N).to(dev)
    ref = sg.sgemm_splitk(A, B)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev) for _ in range(api.SPLITK_WORKSPACES_KEPT + 4)]
    outs = []
    for s in streams + streams[:2]:
        with torch.cuda.stream(s):
            outs.append(sg.sgemm_splitk(A, B))
    torch.cuda.synchronize()
    assert len(api._splitk_workspaces) <= api.SPLITK_WORKSPACES_KEPT
    for s in streams[:2]:
        assert (dev.index, int(s.cuda_stream)) in api._splitk_workspaces
    for o in outs:
        assert torch.equal(o, ref)


@pytest.mark.parametrize("name", ["square1024", "square1024_int"])
def test_square1024_splitk_full(name):
    """The 1024^3 workload through sgemm_splitk at the time model's plan and
    at 2, 4 and 8 chunks, every entry against the oracle (bit for bit on the
    integer variant)."""
    w = WORKLOADS[name]
    A, B = workload_operands(w)
    ref, mag, _ = oracle.sgemm_f64(w.M, w.N, w.K, A.numpy(), w.lda, B.numpy(), w.ldb)
    for splits in (0, 2, 4, 8):
        got, _, plan = run_splitk(w.M, w.N, w.K, A, w.lda, B, w.ldb, w.ldc, -1, splits)
        what = "%s splits=%d plan=%s" % (name, splits, plan)
        if name.endswith("_int"):
            parity.assert_bitwise(got, ref, what)
        else:
            parity.assert_within_tolerance(got, ref, mag, what)


# Shapes whose automatic plan is hybrid (whole layers of 256 tiles take all
# of K, the last partial layer is split), on four different tiles; odd
# leading dimensions and a ragged tile row and column.
HYBRID = [(3300, 300, 1000, 1001, 301, 307), (3456, 301, 1501, 1503, 305, 301),
          (2486, 903, 1501, 1501, 907, 910), (3262, 701, 1501, 1505, 701, 703)]


@pytest.mark.parametrize("shape", HYBRID, ids=lambda s: "x".join(map(str, s[:3])))
def test_hybrid_plan_bitwise(shape):
    M, N, K, lda, ldb, ldc = shape
    full = sg.splitk_plan_full_tiles(M, N, K)
    cfg, splits, nbytes = sg.splitk_plan(M, N, K)
    bm, bn, _ = _tile(cfg)
    tiles = -(-M // bm) * -(-N // bn)
    assert full > 0 and full % 256 == 0 and full < tiles and splits > 1, (full, cfg, splits)
    assert nbytes == sg.SPLITK_HEADER_BYTES + (tiles - full) * splits * bm * bn * 4
    A, B = operands(M, N, K, lda, ldb, seed=M + 3 * N + K, dist_a="int4")
    got, ws, plan = run_splitk(M, N, K, A, lda, B, ldb, ldc, -1, 0)
    assert plan == (cfg, splits)
    ref, _, _ = oracle.sgemm_f64(M, N, K, A.numpy(), lda, B.numpy(), ldb)
    parity.assert_bitwise(got, ref, "hybrid %s cfg%d splits=%d" % (shape, cfg, splits))
    # Again on the same workspace, and through the race-check build (reversed
    # block order, poisoned LDS).
    again, _, _ = run_splitk(M, N, K, A, lda, B, ldb, ldc, -1, 0, ws=ws)
    assert np.array_equal(got, again)
    rc, _, _ = run_splitk(M, N, K, A, lda, B, ldb, ldc, -1, 0, lib=_native.racecheck_lib())
    parity.assert_bitwise(rc, ref, "racecheck hybrid %s" % (shape,))


def test_hybrid_real_valued_matches_across_calls_and_tolerance():
    """Normal-like data on a hybrid plan: bit-identical when repeated, and
    within the parity bound on every entry."""
    M, N, K = 3300, 300, 1000
    assert sg.splitk_plan_full_tiles(M, N, K) > 0
    A, B = operands(M, N, K, K, N, seed=77, dist_a="normal", scale_a=K ** -0.5,
                    scale_b=K ** -0.5)
    got, ws, _ = run_splitk(M, N, K, A, K, B, N, N, -1, 0)
    again, _, _ = run_splitk(M, N, K, A, K, B, N, N, -1, 0, ws=ws)
    assert np.array_equal(got.view(np.int32), again.view(np.int32))
    ref, mag, _ = oracle.sgemm_f64(M, N, K, A.numpy(), K, B.numpy(), N)
    parity.assert_within_tolerance(got, ref, mag, "hybrid real-valued")
