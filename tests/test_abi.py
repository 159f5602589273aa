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


def test_status_strings():
    for code in list(_native.STATUS) + [12345]:
        s = sg.status_string(code)
        assert isinstance(s, str) and s
    assert sg.status_string(0) == "success"
