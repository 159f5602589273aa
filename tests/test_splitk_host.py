"""Host-side checks of the split-K entry points (no GPU needed): the plan
the time model makes, the workspace size it reports, and the argument errors
sgemm_splitk returns before anything is enqueued."""
import ctypes

import pytest

import tiled_fp32_gemm_sgemm_amd as sg
from tiled_fp32_gemm_sgemm_amd import _native

FAKE = 0x1000  # never dereferenced: every call below fails its checks first


def _lib():
    return _native.lib()


def _tile(config):
    bm, bn, bk, thr = (ctypes.c_int() for _ in range(4))
    buf = ctypes.create_string_buffer(64)
    assert _lib().sgemm_config_info(config, buf, 64, ctypes.byref(bm), ctypes.byref(bn),
                                    ctypes.byref(bk), ctypes.byref(thr)) == 0
    return bm.value, bn.value, bk.value


SK = [c for c in range(sg.num_configs()) if sg.config_has_splitk(c)]


def test_splitk_variants_exist():
    assert len(SK) >= 4
    assert _lib().sgemm_config_has_splitk(sg.num_configs()) == -7
    assert _lib().sgemm_config_has_splitk(-1) == -7


@pytest.mark.parametrize("config", SK)
def test_plan_workspace_size(config):
    bm, bn, bk = _tile(config)
    M, N, K = 300, 200, 1000
    cfg, splits, nbytes = sg.splitk_plan(M, N, K, 5, config)
    assert cfg == config
    slices = -(-K // bk)
    kchunk = -(-slices // 5) * bk
    assert splits == -(-K // kchunk)
    tiles = -(-M // bm) * -(-N // bn)
    # A fixed header of per-tile counters, whatever the shape, then the partials.
    assert nbytes == sg.SPLITK_HEADER_BYTES + tiles * splits * bm * bn * 4
    # One chunk needs no workspace.
    assert sg.splitk_plan(M, N, K, 1, config)[2] == 0


def test_header_constants_match_the_c_header():
    import os
    import re
    text = open(os.path.join(os.path.dirname(__file__), "..", "include", "sgemm.h")).read()
    m = re.search(r"#define SGEMM_SPLITK_MAX_TILES (\d+)", text)
    assert m and int(m.group(1)) == sg.SPLITK_MAX_TILES
    assert sg.SPLITK_HEADER_BYTES == 4 * sg.SPLITK_MAX_TILES


@pytest.mark.parametrize("config", SK)
def test_more_tiles_than_the_header_are_not_split(config):
    bm, bn, _ = _tile(config)
    per_side = int(sg.SPLITK_MAX_TILES ** 0.5)
    M, N = per_side * bm, per_side * bn          # exactly the header's tile count
    assert sg.splitk_plan(M, N, 4096, 4, config)[1:] == (4, sg.SPLITK_HEADER_BYTES +
                                                         sg.SPLITK_MAX_TILES * 4 * bm * bn * 4)
    assert sg.splitk_plan(M + 1, N, 4096, 4, config)[1:] == (1, 0)


def test_plan_errors():
    plain = [c for c in range(sg.num_configs()) if not sg.config_has_splitk(c)]
    with pytest.raises(sg.SgemmError):
        sg.splitk_plan(10, 10, 10, 2, plain[0])
    with pytest.raises(sg.SgemmError):
        sg.splitk_plan(10, 10, 10, 65)
    with pytest.raises(sg.SgemmError):
        sg.splitk_plan(-1, 10, 10, 2)


def test_call_errors_enqueue_nothing():
    lib = _lib()
    cfg = SK[0]
    M, N, K = 64, 64, 4096
    need = sg.splitk_plan(M, N, K, 4, cfg)[2]
    assert need > 0
    call = lambda **kw: lib.sgemm_splitk(
        kw.get("config", cfg), M, N, K, FAKE, kw.get("lda", K), FAKE, N, FAKE, N,
        kw.get("splits", 4), kw.get("ws", FAKE), kw.get("nbytes", need), None)
    assert call(ws=None) == -9
    assert call(nbytes=need - 1) == -9
    assert call(splits=-1) == -1
    assert call(splits=65) == -1
    assert call(lda=K - 1) == -2
    assert call(config=sg.num_configs()) == -7
    assert "workspace" in sg.status_string(-9)


def test_noalloc_argument_errors_enqueue_nothing():
    """sgemm_splitk_noalloc checks its arguments and its plan against the
    library's buffer before touching the GPU."""
    lib = _lib()
    cfg = SK[0]
    M, N, K = 64, 64, 4096
    def call(**kw):
        n = kw.get("N", N)
        return lib.sgemm_splitk_noalloc(kw.get("config", cfg), kw.get("M", M), n, kw.get("K", K),
                                        FAKE, kw.get("lda", K), FAKE, n, FAKE, n,
                                        kw.get("splits", 4), None)
    assert call(splits=-1) == -1
    assert call(splits=65) == -1
    assert call(lda=K - 1) == -2
    assert call(config=sg.num_configs()) == -7
    assert call(M=-1) == -1
    # 4096 x 4096 tiles of a 64 x 64 tile at 8 chunks: far more than 64 MiB.
    big = dict(M=4096, N=4096, K=8192, lda=8192, splits=8)
    assert sg.splitk_plan(4096, 4096, 8192, 8, cfg)[2] > 64 * 1024 * 1024
    assert call(**big) == -10
    assert "scratch" in sg.status_string(-10)


def test_hybrid_plan_splits_only_the_last_partial_layer():
    """12544 x 256 x 2304 on 64 x 64 tiles: 784 tiles = 3 layers of 256 and
    16 more.  The automatic plan runs the 768 as whole tiles and splits the 16,
    so the workspace holds only their chunks."""
    M, N, K = 12544, 256, 2304
    cfg, splits, nbytes = sg.splitk_plan(M, N, K)
    full = sg.splitk_plan_full_tiles(M, N, K)
    info = sg.config_info(cfg)
    tiles = -(-M // info["bm"]) * -(-N // info["bn"])
    assert full == tiles - tiles % 256 and 0 < full < tiles
    assert splits > 1 and ((tiles - full) * splits) % 8 == 0
    assert nbytes == sg.SPLITK_HEADER_BYTES + (tiles - full) * splits * info["bm"] * info["bn"] * 4
    # An explicit chunk count splits every tile; whole layers never go hybrid.
    assert sg.splitk_plan_full_tiles(M, N, K, 4, cfg) == 0
    assert sg.splitk_plan_full_tiles(12288, 256, 2304) == 0
    assert sg.splitk_plan_full_tiles(512, 512, 8192) == 0


CONV_SK = [c for c in range(sg.num_configs()) if sg.conv2d_config_has_splitk(c)]


def test_conv_splitk_variants_are_convolution_tiles_with_split_k():
    assert len(CONV_SK) >= 4
    for c in CONV_SK:
        assert sg.conv2d_config_available(c) and sg.config_has_splitk(c)
    with pytest.raises(sg.SgemmError):
        sg.conv2d_config_has_splitk(sg.num_configs())


def test_conv_hybrid_plan_on_a_3x3_layer():
    """64 images of 14 x 14 x 256, 256 filters of 3 x 3: the implicit GEMM is
    12544 x 256 x 2304, 784 tiles of 64 x 64 = three layers of 256 and 16
    more.  The automatic plan runs the 768 whole and splits the 16."""
    cfg, splits, nbytes, full = sg.conv2d_splitk_plan(64, 14, 14, 256, 256, 3, 3, 1)
    info = sg.config_info(cfg)
    assert cfg in CONV_SK
    tiles = -(-12544 // info["bm"]) * -(-256 // info["bn"])
    assert full == tiles - tiles % 256 and 0 < full < tiles
    assert splits > 1 and ((tiles - full) * splits) % 8 == 0
    assert nbytes == sg.SPLITK_HEADER_BYTES + (tiles - full) * splits * info["bm"] * info["bn"] * 4
    # An explicit chunk count splits every tile.
    _, s4, nb4, full4 = sg.conv2d_splitk_plan(64, 14, 14, 256, 256, 3, 3, 1, 1, 1, 4, cfg)
    assert (s4, full4) == (4, 0)
    assert nb4 == sg.SPLITK_HEADER_BYTES + tiles * 4 * info["bm"] * info["bn"] * 4
    # 16 x 16 images make 1024 tiles, four whole layers: nothing to even out.
    assert sg.conv2d_splitk_plan(64, 16, 16, 256, 256, 3, 3, 1)[3] == 0
    # Nothing to compute: no workspace.
    assert sg.conv2d_splitk_plan(2, 4, 4, 0, 3, 3, 3, 1)[2] == 0
    assert sg.conv2d_splitk_plan(1, 2, 2, 4, 3, 5, 5)[2] == 0


def test_conv_splitk_call_errors_enqueue_nothing():
    lib = _lib()
    cfg = CONV_SK[0]
    need = sg.conv2d_splitk_plan(1, 8, 8, 64, 64, 3, 3, 1, 1, 1, 4, cfg)[2]
    assert need > 0
    call = lambda **kw: lib.conv2d_nhwc_splitk(
        kw.get("config", cfg), 1, 8, 8, 64, 64, 3, 3, 1, 1, kw.get("stride", 1), 1, 1, 1,
        kw.get("x", FAKE), FAKE, FAKE, kw.get("splits", 4), kw.get("ws", FAKE),
        kw.get("nbytes", need), None)
    assert call(ws=None) == -9
    assert call(nbytes=need - 1) == -9
    assert call(splits=-1) == -1
    assert call(splits=65) == -1
    assert call(stride=0) == -1
    assert call(x=None) == -3
    assert call(config=sg.num_configs()) == -7
    no_conv_split = [c for c in range(sg.num_configs()) if not sg.conv2d_config_has_splitk(c)]
    assert call(config=no_conv_split[0]) == -7
    with pytest.raises(sg.SgemmError):
        sg.conv2d_splitk_plan(1, 8, 8, 64, 64, 3, 3, 1, 1, 1, 4, no_conv_split[0])
