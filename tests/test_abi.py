"""The C ABI on the CPU: the library loads, exports what include/sgemm.h
declares, and rejects bad arguments with the documented codes before touching
any device (these calls enqueue nothing, so no GPU is needed)."""
import ctypes

import pytest

import tiled_fp32_gemm_sgemm_amd as sg
from tiled_fp32_gemm_sgemm_amd import _native

FAKE = 0x1000  # never dereferenced: every call below fails validation first


def test_library_exports_every_header_function():
    lib = _native.lib()
    names = _native.header_functions()
    assert {"sgemm", "sgemm_strided_batched", "sgemm_valu", "sgemm_valu_strided_batched",
            "sgemm_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    # and the exported dynamic symbols are exactly C names (no C++ mangling)
    for n in names:
        ctypes.cast(getattr(lib, n), ctypes.c_void_p)


def test_racecheck_library_exports_the_same_abi():
    """The race-check build (used by the GPU race-sensitivity tests) exports
    every function the headers declare, with the same tile table."""
    lib = _native.lib()
    rc = _native.racecheck_lib()
    for n in _native.header_functions():
        assert hasattr(rc, n), n
    assert rc.sgemm_num_configs() == lib.sgemm_num_configs()
    # Host-side argument checks behave alike (nothing is enqueued).
    assert rc.sgemm(-1, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, None) == \
        lib.sgemm(-1, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, None)


@pytest.mark.parametrize("path", ["mfma", "valu"])
@pytest.mark.parametrize("args,code", [
    ((-1, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4), -1),        # negative M
    ((4, -1, 4, FAKE, 4, FAKE, 4, FAKE, 4), -1),        # negative N
    ((4, 4, -1, FAKE, 4, FAKE, 4, FAKE, 4), -1),        # negative K
    ((4, 4, 4, FAKE, 3, FAKE, 4, FAKE, 4), -2),         # lda < K
    ((4, 4, 4, FAKE, 4, FAKE, 3, FAKE, 4), -2),         # ldb < N
    ((4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 3), -2),         # ldc < N
    ((4, 4, 0, FAKE, 0, FAKE, 4, FAKE, 4), -2),         # lda < 1
    ((4, 4, 4, 0, 4, FAKE, 4, FAKE, 4), -3),            # NULL A
    ((4, 4, 4, FAKE, 4, 0, 4, FAKE, 4), -3),            # NULL B
    ((4, 4, 4, FAKE, 4, FAKE, 4, 0, 4), -3),            # NULL C
    ((2 ** 31, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4), -4),   # M too large
    ((4, 4, 4, FAKE, 2 ** 62, FAKE, 4, FAKE, 4), -4),   # offsets overflow int64
])
def test_argument_errors(path, args, code):
    assert sg.sgemm_raw(*args, stream=0, path=path) == code


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_noop_sizes_touch_nothing(path):
    # M == 0, N == 0 or batch == 0 return success without reading any pointer.
    assert sg.sgemm_raw(0, 4, 4, 0, 4, 0, 4, 0, 4, stream=0, path=path) == 0
    assert sg.sgemm_raw(4, 0, 4, 0, 4, 0, 1, 0, 1, stream=0, path=path) == 0
    assert sg.sgemm_strided_batched_raw(4, 4, 4, 0, 4, 16, 0, 4, 16, 0, 4, 16, 0,
                                        stream=0, path=path) == 0


def test_batched_stride_errors():
    # negative stride
    assert sg.sgemm_strided_batched_raw(4, 4, 4, FAKE, 4, -1, FAKE, 4, 16, FAKE, 4, 16, 2) == -5
    # C matrices would overlap: strideC < (M-1)*ldc + N
    assert sg.sgemm_strided_batched_raw(4, 4, 4, FAKE, 4, 16, FAKE, 4, 16, FAKE, 4, 15, 2) == -5
    # negative batch
    assert sg.sgemm_strided_batched_raw(4, 4, 4, FAKE, 4, 16, FAKE, 4, 16, FAKE, 4, 16, -1) == -1


def test_config_table_and_errors():
    n = sg.num_configs()
    assert n >= 1
    names = set()
    for i in range(n):
        info = sg.config_info(i)
        names.add(info["name"])
        assert info["bm"] % 32 == 0 and info["bn"] % 32 == 0 and info["threads"] % 64 == 0
    assert len(names) == n
    assert _native.lib().sgemm_with_config(n, 4, 4, 4, FAKE, 4, 0, FAKE, 4, 0, FAKE, 4, 0, 1,
                                           0) == -7
    with pytest.raises(sg.SgemmError):
        sg.config_info(n)


def test_select_config_host_logic():
    n = sg.num_configs()
    for shape in [(4096, 4096, 4096, 1), (1024, 1024, 1024, 1), (4000, 3000, 4100, 1),
                  (16384, 4096, 4096, 1), (128, 128, 128, 1024), (1, 1, 1, 1)]:
        c = sg.select_config(*shape)
        assert 0 <= c < n
        # the unswizzled control build exists for the bank-conflict counter only
        assert "unswizzled" not in sg.config_info(c)["name"]
    assert _native.lib().sgemm_select_config(-1, 1, 1, 1) == -1


def test_selection_is_the_smallest_predicted_time():
    n = sg.num_configs()
    selectable = [c for c in range(n) if sg.config_selectable(c)]
    assert 0 < len(selectable) < n  # the control build is listed but never chosen
    for c in range(n):
        if not sg.config_selectable(c):
            assert _native.lib().sgemm_config_predict_us(c, 64, 64, 64, 1) == -7
    for shape in [(4096, 4096, 4096, 1), (1024, 1024, 1024, 1), (4000, 3000, 4100, 1),
                  (16384, 4096, 4096, 1), (128, 128, 128, 1024), (512, 4096, 4096, 1),
                  (7, 9, 11, 3), (100000, 64, 64, 1)]:
        pred = {c: sg.predict_us(c, *shape) for c in selectable}
        assert all(t > 0 for t in pred.values())
        chosen = sg.select_config(*shape)
        assert pred[chosen] == min(pred.values())


def test_predicted_time_grows_with_the_work():
    for c in range(sg.num_configs()):
        if not sg.config_selectable(c):
            continue
        t = [sg.predict_us(c, 4096, 4096, k) for k in (256, 1024, 4096)]
        assert t[0] < t[1] < t[2]
        assert sg.predict_us(c, 8192, 4096, 4096) >= t[2]


def test_autotune_argument_errors():
    lib = _native.lib()
    best = ctypes.c_int(-1)
    args = (4, 4, 4, FAKE, 4, 0, FAKE, 4, 0, FAKE, 4, 0, 1, 0)
    assert lib.sgemm_autotune(*args, 0, ctypes.byref(best), None) == -1      # reps < 1
    assert lib.sgemm_autotune(*args, 1, None, None) == -3                    # no result slot
    assert lib.sgemm_autotune(4, 4, 4, FAKE, 3, 0, FAKE, 4, 0, FAKE, 4, 0, 1, 0, 1,
                              ctypes.byref(best), None) == -2                # lda < K
    # empty product: the automatic choice, nothing timed or launched
    assert lib.sgemm_autotune(0, 4, 4, None, 4, 0, None, 4, 0, None, 4, 0, 1, 0, 1,
                              ctypes.byref(best), None) == 0


def test_status_strings():
    for code in list(_native.STATUS) + [12345]:
        s = sg.status_string(code)
        assert isinstance(s, str) and s
    assert sg.status_string(0) == "success"


def test_general_form_argument_errors_enqueue_nothing():
    lib = _native.lib()
    F = FAKE
    # transpose flag out of range
    assert lib.sgemm_ex(2, 0, 4, 4, 4, 1.0, F, 4, F, 4, 0.0, F, 4, 0) == -8
    assert lib.sgemm_ex(0, -1, 4, 4, 4, 1.0, F, 4, F, 4, 0.0, F, 4, 0) == -8
    # transposed A needs lda >= M; transposed B needs ldb >= K
    assert lib.sgemm_ex(1, 0, 8, 4, 4, 1.0, F, 4, F, 4, 0.0, F, 4, 0) == -2
    assert lib.sgemm_ex(0, 1, 4, 4, 8, 1.0, F, 8, F, 4, 0.0, F, 4, 0) == -2
    # plain layouts keep the plain rules
    assert lib.sgemm_ex(0, 0, 4, 4, 8, 1.0, F, 4, F, 4, 0.0, F, 4, 0) == -2
    # A and B may be NULL only when they are not read
    assert lib.sgemm_ex(0, 0, 4, 4, 4, 1.0, None, 4, F, 4, 0.0, F, 4, 0) == -3
    assert lib.sgemm_ex(0, 0, 4, 4, 4, 1.0, F, 4, F, 4, 0.0, None, 4, 0) == -3
    # empty products succeed without touching anything
    assert lib.sgemm_ex(1, 1, 0, 4, 4, 1.0, None, 1, None, 4, 0.0, None, 4, 0) == 0
    # strided batch: overlapping C matrices
    assert lib.sgemm_ex_strided_batched(0, 0, 4, 4, 4, 1.0, F, 4, 16, F, 4, 16, 0.0, F, 4, 15,
                                        2, 0) == -5
    # a tile without the general form, and an unknown tile
    plain = [c for c in range(sg.num_configs()) if not sg.config_has_general_form(c)]
    assert plain
    assert lib.sgemm_ex_with_config(plain[0], 0, 0, 4, 4, 4, 1.0, F, 4, 0, F, 4, 0, 0.0, F, 4,
                                    0, 1, 0) == -7
    assert lib.sgemm_ex_with_config(sg.num_configs(), 0, 0, 4, 4, 4, 1.0, F, 4, 0, F, 4, 0,
                                    0.0, F, 4, 0, 1, 0) == -7
    assert sg.status_string(-8).startswith("invalid transpose")


def test_general_config_selection():
    general = [c for c in range(sg.num_configs()) if sg.config_has_general_form(c)]
    assert len(general) >= 4
    for shape in [(4096, 4096, 4096, 1), (1024, 1024, 1024, 1), (4000, 3000, 4100, 1),
                  (512, 4096, 4096, 1), (128, 128, 128, 1024), (3, 5, 7, 1)]:
        c = sg.select_general_config(*shape)
        assert c in general
        pred = {g: sg.predict_us(g, *shape) for g in general}
        assert pred[c] == min(pred.values())


def test_window_sum_argument_errors():
    lib = _native.lib()
    assert lib.window_sum(-1, 5, FAKE, FAKE, 0) == -1
    assert lib.window_sum(10, 0, FAKE, FAKE, 0) == -1
    assert lib.window_sum(10, 1025, FAKE, FAKE, 0) == -1
    assert lib.window_sum(10, 5, None, FAKE, 0) == -3
    assert lib.window_sum(10, 5, FAKE, None, 0) == -3
    assert lib.window_sum(2 ** 62, 5, FAKE, FAKE, 0) == -4     # more than 2^31 blocks
    assert lib.window_sum(0, 5, None, None, 0) == 0            # nothing to do


def test_conv2d_host_logic_and_argument_errors():
    lib = _native.lib()
    # output extents: (H + 2 pad - dil (R - 1) - 1) / stride + 1, floored, 0 when negative
    assert sg.conv2d_output_size(56, 56, 3, 3, 1, 1, 1) == (56, 56)
    assert sg.conv2d_output_size(56, 56, 3, 3, 1, 2, 1) == (28, 28)
    assert sg.conv2d_output_size(7, 9, 3, 2, (0, 1), (2, 1), (1, 3)) == (3, 8)
    assert sg.conv2d_output_size(2, 2, 5, 5) == (0, 0)
    ok = [c for c in range(sg.num_configs()) if sg.conv2d_config_available(c)]
    assert ok and all(sg.config_has_general_form(c) for c in ok)
    for shape in [(64, 14, 14, 256, 256, 3, 3, 1), (64, 28, 28, 128, 128, 3, 3, 1),
                  (8, 32, 32, 3, 64, 7, 7, 3, 2)]:
        assert sg.conv2d_select_config(*shape) in ok
    # a tile whose BK divides C is preferred (direct staging)
    assert sg.config_info(sg.conv2d_select_config(64, 14, 14, 256, 256, 3, 3, 1))["bk"] % 32 == 0

    def call(*a, **kw):
        return sg.conv2d_nhwc_raw(*a, **kw)
    base = (1, 8, 8, 16, 16, 3, 3)
    assert call(*base, FAKE, FAKE, FAKE, stride=(0, 1)) == -1
    assert call(*base, FAKE, FAKE, FAKE, dil=(1, 0)) == -1
    assert call(*base, FAKE, FAKE, FAKE, pad=(-1, 1)) == -1
    assert call(-1, 8, 8, 16, 16, 3, 3, FAKE, FAKE, FAKE) == -1
    assert call(*base, None, FAKE, FAKE, pad=1) == -3
    assert call(*base, FAKE, None, FAKE, pad=1) == -3
    assert call(*base, FAKE, FAKE, None, pad=1) == -3
    assert call(*base, FAKE, FAKE, FAKE, pad=1, config=0) == -7
    assert call(*base, FAKE, FAKE, FAKE, pad=1, config=10 ** 6) == -7
    assert call(1, 2 ** 29, 8, 16, 16, 3, 3, FAKE, FAKE, FAKE) == -4   # padded span too large
    assert call(2 ** 20, 2 ** 10, 2 ** 10, 1, 1, 1, 1, FAKE, FAKE, FAKE) == -4  # N*P*Q >= 2^31
    assert call(0, 8, 8, 16, 16, 3, 3, None, None, None) == 0         # no outputs
    assert call(1, 2, 2, 16, 16, 5, 5, None, None, None) == 0         # P = Q = 0
    assert call(1, 8, 8, 16, 0, 3, 3, None, None, None) == 0          # no output channels
    assert lib.conv2d_config_available(-1) == -7


def test_attention_argument_errors():
    lib = _native.lib()
    F = FAKE
    assert lib.attention_fwd(-1, 4, 4, 64, F, F, F, F, 1.0, 0, 0) == -1
    assert lib.attention_fwd(1, 4, 4, 96, F, F, F, F, 1.0, 0, 0) == -1       # head dim 64 or 128
    assert lib.attention_fwd(1, 4, 4, 64, F, F, F, F, float("inf"), 0, 0) == -1
    assert lib.attention_fwd(1, 4, 4, 64, F, F, F, F, 1.0, 2, 0) == -8
    assert lib.attention_fwd(1, 2 ** 31, 4, 64, F, F, F, F, 1.0, 0, 0) == -4
    assert lib.attention_fwd(1, 2 ** 31 - 300, 4, 64, F, F, F, F, 1.0, 0, 0) == -4
    assert lib.attention_fwd(1, 4, 4, 64, None, F, F, F, 1.0, 0, 0) == -3
    assert lib.attention_fwd(1, 4, 4, 64, F, F, F, None, 1.0, 0, 0) == -3
    assert lib.attention_fwd(0, 4, 4, 64, None, None, None, None, 1.0, 0, 0) == 0
    assert lib.attention_fwd(3, 0, 4, 128, None, None, None, None, 1.0, 1, 0) == 0
