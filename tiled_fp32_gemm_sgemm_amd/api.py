"""Python entry points over the C ABI (include/sgemm.h).

PyTorch supplies device memory and the stream; the product itself runs in
libsgemm.so.  Operands are row-major: a 2-D tensor with unit column stride,
whose row stride is its leading dimension.  Nothing is copied or converted:
an operand that does not already have that layout, dtype float32 and a CUDA
device is rejected.
"""
from __future__ import annotations

import ctypes

from . import _native

PATHS = ("mfma", "valu")

# The split-K workspace header (include/sgemm.h): one uint32 arrival counter
# per output tile, at the same place for every shape.
SPLITK_MAX_TILES = 16384
SPLITK_HEADER_BYTES = SPLITK_MAX_TILES * 4


def _stream_handle(stream, device) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, what: str) -> None:
    if status != 0:
        raise _native.SgemmError(status, what)


def sgemm_raw(M, N, K, A_ptr, lda, B_ptr, ldb, C_ptr, ldc, stream=0, path="mfma",
              config=None) -> int:
    """Direct call on raw device addresses; returns the status code."""
    lib = _native.lib()
    if config is not None:
        return lib.sgemm_with_config(int(config), M, N, K, A_ptr, lda, 0, B_ptr, ldb, 0,
                                     C_ptr, ldc, 0, 1, stream)
    fn = lib.sgemm if path == "mfma" else lib.sgemm_valu
    if path not in PATHS:
        raise ValueError("path must be one of %s" % (PATHS,))
    return fn(M, N, K, A_ptr, lda, B_ptr, ldb, C_ptr, ldc, stream)


def sgemm_strided_batched_raw(M, N, K, A_ptr, lda, strideA, B_ptr, ldb, strideB, C_ptr, ldc,
                              strideC, batch, stream=0, path="mfma", config=None) -> int:
    lib = _native.lib()
    if config is not None:
        return lib.sgemm_with_config(int(config), M, N, K, A_ptr, lda, strideA, B_ptr, ldb,
                                     strideB, C_ptr, ldc, strideC, batch, stream)
    if path not in PATHS:
        raise ValueError("path must be one of %s" % (PATHS,))
    fn = lib.sgemm_strided_batched if path == "mfma" else lib.sgemm_valu_strided_batched
    return fn(M, N, K, A_ptr, lda, strideA, B_ptr, ldb, strideB, C_ptr, ldc, strideC, batch,
              stream)


def _operand(t, name, ndim):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != torch.float32:
        raise TypeError("%s must be float32, got %s" % (name, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU" % name)
    if t.dim() != ndim:
        raise ValueError("%s must have %d dimensions" % (name, ndim))
    if t.size(-1) > 1 and t.stride(-1) != 1:
        raise ValueError("%s must be row-major (unit stride along its last dimension)" % name)


def _ld(t) -> int:
    return max(int(t.stride(-2)), int(t.size(-1)), 1)


def sgemm(A, B, out=None, *, path: str = "mfma", config=None, stream=None):
    """C = A @ B for float32 CUDA tensors A (M, K) and B (K, N); returns C (M, N)."""
    import torch
    _operand(A, "A", 2)
    _operand(B, "B", 2)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _operand(out, "out", 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out must have shape (%d, %d)" % (M, N))
    with torch.cuda.device(A.device):
        st = sgemm_raw(M, N, K, A.data_ptr(), _ld(A), B.data_ptr(), _ld(B), out.data_ptr(),
                       _ld(out), _stream_handle(stream, A.device), path, config)
    _check(st, "sgemm")
    return out


def sgemm_strided_batched(A, B, out=None, *, path: str = "mfma", config=None, stream=None):
    """Batched C[b] = A[b] @ B[b] for 3-D float32 CUDA tensors; returns C (batch, M, N)."""
    import torch
    _operand(A, "A", 3)
    _operand(B, "B", 3)
    batch, M, K = A.shape
    batch2, K2, N = B.shape
    if K != K2 or batch != batch2:
        raise ValueError("shapes differ: %s vs %s" % (tuple(A.shape), tuple(B.shape)))
    if out is None:
        out = torch.empty((batch, M, N), dtype=torch.float32, device=A.device)
    _operand(out, "out", 3)
    if tuple(out.shape) != (batch, M, N):
        raise ValueError("out must have shape (%d, %d, %d)" % (batch, M, N))
    with torch.cuda.device(A.device):
        st = sgemm_strided_batched_raw(
            M, N, K, A.data_ptr(), _ld(A), int(A.stride(0)), B.data_ptr(), _ld(B),
            int(B.stride(0)), out.data_ptr(), _ld(out), int(out.stride(0)), batch,
            _stream_handle(stream, A.device), path, config)
    _check(st, "sgemm_strided_batched")
    return out


def splitk_plan(M: int, N: int, K: int, splits: int = 0, config=None):
    """(config, splits, workspace bytes) that sgemm_splitk runs for this shape."""
    cfg = ctypes.c_int(-1)
    sp = ctypes.c_int64(0)
    st = _native.lib().sgemm_splitk_plan(-1 if config is None else int(config), M, N, K,
                                         int(splits), ctypes.byref(cfg), ctypes.byref(sp))
    if st < 0:
        raise _native.SgemmError(int(st), "sgemm_splitk_plan")
    return cfg.value, sp.value, int(st)


def splitk_plan_full_tiles(M: int, N: int, K: int, splits: int = 0, config=None) -> int:
    """Output tiles of sgemm_splitk's plan that take all of K with no join."""
    st = _native.lib().sgemm_splitk_plan_full_tiles(-1 if config is None else int(config), M, N,
                                                    K, int(splits))
    if st < 0:
        raise _native.SgemmError(int(st), "sgemm_splitk_plan_full_tiles")
    return int(st)


def config_has_splitk(config: int) -> bool:
    st = _native.lib().sgemm_config_has_splitk(int(config))
    if st < 0:
        raise _native.SgemmError(st, "sgemm_config_has_splitk")
    return bool(st)


# One zero-filled split-K workspace per (device, stream), grown on demand.
# It is allocated and zeroed on the stream whose launches use it, so the
# zeros land before the first join reads them, and a buffer dropped when it
# grows goes back to the allocator on that stream, behind every launch that
# used it.  Calls on different streams never share one.  At most
# SPLITK_WORKSPACES_KEPT are kept, the least recently used dropped first
# (its memory, too, is reused only behind that stream's queued launches), so
# workspaces of streams that are gone do not pile up.
SPLITK_WORKSPACES_KEPT = 8
_splitk_workspaces = {}


def _torch_stream(stream, device):
    import torch
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def splitk_workspace(device, nbytes: int, stream=None):
    """A zero-filled uint8 device tensor of at least nbytes for sgemm_splitk
    calls on `stream` (None: the device's current stream), made on that
    stream.  Its header of per-tile counters is back at zero after every
    completed call, so it serves calls of any shape on the same stream."""
    import torch
    device = torch.device(device)
    if device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    s = _torch_stream(stream, device)
    key = (device.index, int(s.cuda_stream))
    ws = _splitk_workspaces.pop(key, None)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.device(device), torch.cuda.stream(s):
            ws = None
            ws = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    _splitk_workspaces[key] = ws  # most recently used last
    while len(_splitk_workspaces) > SPLITK_WORKSPACES_KEPT:
        _splitk_workspaces.pop(next(iter(_splitk_workspaces)))
    return ws


def sgemm_splitk(A, B, out=None, *, splits: int = 0, config=None, workspace=None, stream=None):
    """C = A @ B with the k range split over `splits` workgroups per output
    tile (0: the time model's choice), joined in the same launch.  workspace:
    a device tensor of at least splitk_plan(...)[2] bytes whose header starts
    at zero, or None for the one kept for this device and stream."""
    import torch
    _operand(A, "A", 2)
    _operand(B, "B", 2)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _operand(out, "out", 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out must have shape (%d, %d)" % (M, N))
    cfg = -1 if config is None else int(config)
    _, _, nbytes = splitk_plan(M, N, K, splits, config)
    if workspace is None:
        workspace = splitk_workspace(A.device, nbytes, stream)
    with torch.cuda.device(A.device):
        st = _native.lib().sgemm_splitk(cfg, M, N, K, A.data_ptr(), _ld(A), B.data_ptr(), _ld(B),
                                        out.data_ptr(), _ld(out), int(splits),
                                        workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(),
                                        _stream_handle(stream, A.device))
    _check(st, "sgemm_splitk")
    return out


def sgemm_splitk_noalloc(A, B, out, *, splits: int = 0, config=None, stream=None):
    """sgemm_splitk with the workspace taken from the library's own per-GPU
    buffer: nothing is allocated, so `out` must be given.  Calls that may
    overlap on one GPU share that buffer and race."""
    _operand(A, "A", 2)
    _operand(B, "B", 2)
    _operand(out, "out", 2)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    if tuple(out.shape) != (M, N):
        raise ValueError("out must have shape (%d, %d)" % (M, N))
    import torch
    with torch.cuda.device(A.device):
        st = _native.lib().sgemm_splitk_noalloc(-1 if config is None else int(config), M, N, K,
                                                A.data_ptr(), _ld(A), B.data_ptr(), _ld(B),
                                                out.data_ptr(), _ld(out), int(splits),
                                                _stream_handle(stream, A.device))
    _check(st, "sgemm_splitk_noalloc")
    return out


def num_configs() -> int:
    return _native.lib().sgemm_num_configs()


def config_info(config: int) -> dict:
    buf = ctypes.create_string_buffer(64)
    bm, bn, bk, nt = (ctypes.c_int() for _ in range(4))
    st = _native.lib().sgemm_config_info(int(config), buf, 64, ctypes.byref(bm), ctypes.byref(bn),
                                         ctypes.byref(bk), ctypes.byref(nt))
    _check(st, "sgemm_config_info")
    return {"name": buf.value.decode(), "bm": bm.value, "bn": bn.value, "bk": bk.value,
            "threads": nt.value}


def select_config(M: int, N: int, K: int, batch: int = 1) -> int:
    st = _native.lib().sgemm_select_config(M, N, K, batch)
    if st < 0:
        raise _native.SgemmError(st, "sgemm_select_config")
    return st


def config_selectable(config: int) -> bool:
    st = _native.lib().sgemm_config_selectable(int(config))
    if st < 0:
        raise _native.SgemmError(st, "sgemm_config_selectable")
    return bool(st)


def workgroups_per_cu(config: int) -> int:
    """Workgroups of this configuration one CU holds at once."""
    st = _native.lib().sgemm_config_workgroups_per_cu(int(config))
    if st < 0:
        raise _native.SgemmError(st, "sgemm_config_workgroups_per_cu")
    return st


def predict_us(config: int, M: int, N: int, K: int, batch: int = 1) -> float:
    """Predicted microseconds of one launch of `config` on this shape."""
    t = _native.lib().sgemm_config_predict_us(int(config), M, N, K, batch)
    if t < 0:
        raise _native.SgemmError(int(t), "sgemm_config_predict_us")
    return t


def autotune_raw(M, N, K, A_ptr, lda, strideA, B_ptr, ldb, strideB, C_ptr, ldc, strideC, batch,
                 stream=0, reps=10):
    """(status, best config, best milliseconds per launch); C holds A x B."""
    best = ctypes.c_int(-1)
    ms = ctypes.c_float(0.0)
    st = _native.lib().sgemm_autotune(M, N, K, A_ptr, lda, strideA, B_ptr, ldb, strideB, C_ptr,
                                      ldc, strideC, batch, stream, int(reps), ctypes.byref(best),
                                      ctypes.byref(ms))
    return st, best.value, ms.value


def autotune(A, B, out=None, reps: int = 10, stream=None):
    """Time every selectable configuration on these operands (2-D: one
    product; 3-D: a strided batch) and return (config, ms per launch, out)."""
    import torch
    batched = A.dim() == 3
    _operand(A, "A", 3 if batched else 2)
    _operand(B, "B", 3 if batched else 2)
    if batched:
        batch, M, K = A.shape
        batch2, K2, N = B.shape
    else:
        (M, K), (K2, N) = A.shape, B.shape
        batch = batch2 = 1
    if K != K2 or batch != batch2:
        raise ValueError("shapes differ: %s vs %s" % (tuple(A.shape), tuple(B.shape)))
    shape = (batch, M, N) if batched else (M, N)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=A.device)
    _operand(out, "out", 3 if batched else 2)
    if tuple(out.shape) != shape:
        raise ValueError("out must have shape %s" % (shape,))
    sa = int(A.stride(0)) if batched else 0
    sb = int(B.stride(0)) if batched else 0
    sc = int(out.stride(0)) if batched else 0
    with torch.cuda.device(A.device):
        st, cfg, ms = autotune_raw(M, N, K, A.data_ptr(), _ld(A), sa, B.data_ptr(), _ld(B), sb,
                                   out.data_ptr(), _ld(out), sc, batch,
                                   _stream_handle(stream, A.device), reps)
    _check(st, "sgemm_autotune")
    return cfg, ms, out


def sgemm_ex_raw(transA, transB, M, N, K, alpha, A_ptr, lda, B_ptr, ldb, beta, C_ptr, ldc,
                 stream=0, config=None, batch=1, strideA=0, strideB=0, strideC=0) -> int:
    """C = alpha op(A) op(B) + beta C on device addresses; returns the status."""
    lib = _native.lib()
    if config is not None:
        return lib.sgemm_ex_with_config(int(config), int(transA), int(transB), M, N, K,
                                        float(alpha), A_ptr, lda, strideA, B_ptr, ldb, strideB,
                                        float(beta), C_ptr, ldc, strideC, batch, stream)
    if batch == 1 and strideA == 0 and strideB == 0 and strideC == 0:
        return lib.sgemm_ex(int(transA), int(transB), M, N, K, float(alpha), A_ptr, lda, B_ptr,
                            ldb, float(beta), C_ptr, ldc, stream)
    return lib.sgemm_ex_strided_batched(int(transA), int(transB), M, N, K, float(alpha), A_ptr,
                                        lda, strideA, B_ptr, ldb, strideB, float(beta), C_ptr,
                                        ldc, strideC, batch, stream)


def sgemm_ex(A, B, C=None, alpha: float = 1.0, beta: float = 0.0, transA: bool = False,
             transB: bool = False, stream=None, config=None):
    """C = alpha op(A) op(B) + beta C.  A and B are the stored matrices
    (2-D, or 3-D for a strided batch): A is M x K, or K x M with transA; B is
    K x N, or N x K with transB.  C (M x N, or batch x M x N) is required when
    beta != 0 and is updated in place; otherwise a new tensor is returned."""
    import torch
    batched = A.dim() == 3
    nd = 3 if batched else 2
    _operand(A, "A", nd)
    _operand(B, "B", nd)
    ra, ca = A.shape[-2:]
    rb, cb = B.shape[-2:]
    M, K = (ca, ra) if transA else (ra, ca)
    K2, N = (cb, rb) if transB else (rb, cb)
    batch = A.shape[0] if batched else 1
    if K != K2 or (batched and B.shape[0] != batch):
        raise ValueError("shapes differ: %s vs %s" % (tuple(A.shape), tuple(B.shape)))
    shape = (batch, M, N) if batched else (M, N)
    if C is None:
        if beta != 0.0:
            raise ValueError("C is required when beta != 0")
        C = torch.empty(shape, dtype=torch.float32, device=A.device)
    _operand(C, "C", nd)
    if tuple(C.shape) != shape:
        raise ValueError("C must have shape %s" % (shape,))
    sa = int(A.stride(0)) if batched else 0
    sb = int(B.stride(0)) if batched else 0
    sc = int(C.stride(0)) if batched else 0
    with torch.cuda.device(A.device):
        st = sgemm_ex_raw(transA, transB, M, N, K, alpha, A.data_ptr(), _ld(A), B.data_ptr(),
                          _ld(B), beta, C.data_ptr(), _ld(C), _stream_handle(stream, A.device),
                          config, batch, sa, sb, sc)
    _check(st, "sgemm_ex")
    return C


def ex_splitk_plan(M: int, N: int, K: int, transA: bool = False, transB: bool = False,
                   splits: int = 0, config=None):
    """(config, splits, workspace bytes) that sgemm_ex_splitk runs for this
    shape and layout."""
    cfg = ctypes.c_int(-1)
    sp = ctypes.c_int64(0)
    st = _native.lib().sgemm_ex_splitk_plan(-1 if config is None else int(config), int(transA),
                                            int(transB), M, N, K, int(splits), ctypes.byref(cfg),
                                            ctypes.byref(sp))
    if st < 0:
        raise _native.SgemmError(int(st), "sgemm_ex_splitk_plan")
    return cfg.value, sp.value, int(st)


def ex_splitk_plan_full_tiles(M: int, N: int, K: int, transA: bool = False,
                              transB: bool = False, splits: int = 0, config=None) -> int:
    """Output tiles of sgemm_ex_splitk's plan that take all of K with no join."""
    st = _native.lib().sgemm_ex_splitk_plan_full_tiles(-1 if config is None else int(config),
                                                       int(transA), int(transB), M, N, K,
                                                       int(splits))
    if st < 0:
        raise _native.SgemmError(int(st), "sgemm_ex_splitk_plan_full_tiles")
    return int(st)


def sgemm_ex_splitk_raw(transA, transB, M, N, K, alpha, A_ptr, lda, B_ptr, ldb, beta, C_ptr,
                        ldc, ws_ptr, ws_bytes, stream=0, splits: int = 0, config=None) -> int:
    """The general form with its reduction split, on device addresses;
    returns the status."""
    return _native.lib().sgemm_ex_splitk(-1 if config is None else int(config), int(transA),
                                         int(transB), M, N, K, float(alpha), A_ptr, lda, B_ptr,
                                         ldb, float(beta), C_ptr, ldc, int(splits), ws_ptr,
                                         int(ws_bytes), stream)


def sgemm_ex_splitk(A, B, C=None, alpha: float = 1.0, beta: float = 0.0, transA: bool = False,
                    transB: bool = False, *, splits: int = 0, config=None, workspace=None,
                    stream=None):
    """sgemm_ex (2-D operands) with the k range split as in sgemm_splitk.
    workspace: a device tensor of at least ex_splitk_plan(...)[2] bytes whose
    header starts at zero, or None for the one kept for this device and
    stream (shared with sgemm_splitk)."""
    import torch
    _operand(A, "A", 2)
    _operand(B, "B", 2)
    ra, ca = A.shape
    rb, cb = B.shape
    M, K = (ca, ra) if transA else (ra, ca)
    K2, N = (cb, rb) if transB else (rb, cb)
    if K != K2:
        raise ValueError("shapes differ: %s vs %s" % (tuple(A.shape), tuple(B.shape)))
    if C is None:
        if beta != 0.0:
            raise ValueError("C is required when beta != 0")
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _operand(C, "C", 2)
    if tuple(C.shape) != (M, N):
        raise ValueError("C must have shape (%d, %d)" % (M, N))
    _, _, nbytes = ex_splitk_plan(M, N, K, transA, transB, splits, config)
    if workspace is None:
        workspace = splitk_workspace(A.device, nbytes, stream)
    with torch.cuda.device(A.device):
        st = sgemm_ex_splitk_raw(transA, transB, M, N, K, alpha, A.data_ptr(), _ld(A),
                                 B.data_ptr(), _ld(B), beta, C.data_ptr(), _ld(C),
                                 workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(),
                                 _stream_handle(stream, A.device), splits, config)
    _check(st, "sgemm_ex_splitk")
    return C


def config_has_general_splitk(config: int) -> bool:
    st = _native.lib().sgemm_config_has_general_splitk(int(config))
    if st < 0:
        raise _native.SgemmError(st, "sgemm_config_has_general_splitk")
    return bool(st)


def config_has_general_form(config: int) -> bool:
    st = _native.lib().sgemm_config_has_general_form(int(config))
    if st < 0:
        raise _native.SgemmError(st, "sgemm_config_has_general_form")
    return bool(st)


def select_general_config(M: int, N: int, K: int, batch: int = 1) -> int:
    st = _native.lib().sgemm_select_general_config(M, N, K, batch)
    if st < 0:
        raise _native.SgemmError(st, "sgemm_select_general_config")
    return st


def window_sum_raw(n: int, W: int, x_ptr: int, y_ptr: int, stream=0) -> int:
    """y[i] = sum_{d<W} x[i+d], i < n, on device addresses; returns the status."""
    return _native.lib().window_sum(n, W, x_ptr, y_ptr, stream)


def window_sum(x, W: int, out=None, stream=None):
    """Sliding window sums of a 1-D float32 CUDA tensor x: n = len(x) - W + 1
    outputs (x[i] + ... + x[i+W-1])."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or x.device.type != "cuda":
        raise TypeError("x must be a float32 CUDA tensor")
    if x.dim() != 1 or (x.numel() > 1 and x.stride(0) != 1):
        raise ValueError("x must be a contiguous 1-D tensor")
    n = x.numel() - W + 1
    if W < 1 or n < 0:
        raise ValueError("need 1 <= W <= len(x) + 1")
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=x.device)
    if out.dim() != 1 or out.numel() != n or (n > 1 and out.stride(0) != 1):
        raise ValueError("out must be a contiguous 1-D tensor of %d values" % n)
    with torch.cuda.device(x.device):
        st = window_sum_raw(n, W, x.data_ptr(), out.data_ptr(), _stream_handle(stream, x.device))
    _check(st, "window_sum")
    return out


def _pair(v, name):
    if isinstance(v, int):
        return (v, v)
    t = tuple(int(e) for e in v)
    if len(t) != 2:
        raise ValueError("%s must be an int or a pair" % name)
    return t


def conv2d_output_size(H: int, W: int, R: int, S: int, pad=0, stride=1, dil=1):
    """(P, Q) of a convolution (the library's conv2d_nhwc_output_size)."""
    ph, pw = _pair(pad, "pad")
    sh, sw = _pair(stride, "stride")
    dh, dw = _pair(dil, "dil")
    P, Q = ctypes.c_int64(), ctypes.c_int64()
    st = _native.lib().conv2d_nhwc_output_size(H, W, R, S, ph, pw, sh, sw, dh, dw,
                                               ctypes.byref(P), ctypes.byref(Q))
    _check(st, "conv2d_nhwc_output_size")
    return P.value, Q.value


def conv2d_nhwc_raw(N, H, W, C, K, R, S, x_ptr, w_ptr, y_ptr, pad=0, stride=1, dil=1, stream=0,
                    config=None) -> int:
    """2-D convolution on device addresses: NHWC input, KRSC filters, NPQK
    output (include/conv2d.h); returns the status."""
    ph, pw = _pair(pad, "pad")
    sh, sw = _pair(stride, "stride")
    dh, dw = _pair(dil, "dil")
    lib = _native.lib()
    if config is not None:
        return lib.conv2d_nhwc_with_config(int(config), N, H, W, C, K, R, S, ph, pw, sh, sw, dh,
                                           dw, x_ptr, w_ptr, y_ptr, stream)
    return lib.conv2d_nhwc(N, H, W, C, K, R, S, ph, pw, sh, sw, dh, dw, x_ptr, w_ptr, y_ptr,
                           stream)


def conv2d_nhwc(x, wt, pad=0, stride=1, dil=1, out=None, stream=None, config=None):
    """Convolution of a contiguous float32 CUDA tensor x (N, H, W, C) with
    filters wt (K, R, S, C); returns y (N, P, Q, K)."""
    import torch
    for t, name in ((x, "x"), (wt, "wt")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.device.type != "cuda":
            raise TypeError("%s must be a float32 CUDA tensor" % name)
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous 4-D tensor" % name)
    N, H, W, C = x.shape
    K, R, S, C2 = wt.shape
    if C2 != C:
        raise ValueError("channel counts differ: x has %d, wt has %d" % (C, C2))
    P, Q = conv2d_output_size(H, W, R, S, pad, stride, dil)
    if out is None:
        out = torch.empty((N, P, Q, K), dtype=torch.float32, device=x.device)
    if tuple(out.shape) != (N, P, Q, K) or not out.is_contiguous():
        raise ValueError("out must be a contiguous (%d, %d, %d, %d) tensor" % (N, P, Q, K))
    with torch.cuda.device(x.device):
        st = conv2d_nhwc_raw(N, H, W, C, K, R, S, x.data_ptr(), wt.data_ptr(), out.data_ptr(),
                             pad, stride, dil, _stream_handle(stream, x.device), config)
    _check(st, "conv2d_nhwc")
    return out


def conv2d_splitk_plan(N, H, W, C, K, R, S, pad=0, stride=1, dil=1, splits: int = 0,
                       config=None):
    """(config, splits, workspace bytes, full tiles) of the plan
    conv2d_nhwc_splitk would run (the library's conv2d_nhwc_splitk_plan)."""
    ph, pw = _pair(pad, "pad")
    sh, sw = _pair(stride, "stride")
    dh, dw = _pair(dil, "dil")
    cfg = ctypes.c_int()
    sp = ctypes.c_int64()
    full = ctypes.c_int64()
    nbytes = _native.lib().conv2d_nhwc_splitk_plan(
        -1 if config is None else int(config), N, H, W, C, K, R, S, ph, pw, sh, sw, dh, dw,
        int(splits), ctypes.byref(cfg), ctypes.byref(sp), ctypes.byref(full))
    if nbytes < 0:
        raise _native.SgemmError(int(nbytes), "conv2d_nhwc_splitk_plan")
    return cfg.value, sp.value, int(nbytes), full.value


def conv2d_nhwc_splitk_raw(N, H, W, C, K, R, S, x_ptr, w_ptr, y_ptr, ws_ptr, ws_bytes, pad=0,
                           stride=1, dil=1, splits=0, stream=0, config=None) -> int:
    """conv2d_nhwc_splitk on device addresses (include/conv2d.h); returns the
    status."""
    ph, pw = _pair(pad, "pad")
    sh, sw = _pair(stride, "stride")
    dh, dw = _pair(dil, "dil")
    return _native.lib().conv2d_nhwc_splitk(-1 if config is None else int(config), N, H, W, C, K,
                                            R, S, ph, pw, sh, sw, dh, dw, x_ptr, w_ptr, y_ptr,
                                            int(splits), ws_ptr, int(ws_bytes), stream)


def conv2d_nhwc_splitk(x, wt, pad=0, stride=1, dil=1, out=None, *, splits: int = 0, config=None,
                       workspace=None, stream=None):
    """conv2d_nhwc with the reduction over R*S*C split across workgroups as in
    sgemm_splitk (splits = 0: the time model's choice, possibly splitting only
    the last partial layer of tiles).  workspace: a device tensor of at least
    conv2d_splitk_plan(...)[2] bytes whose header starts at zero, or None for
    the one kept for this device and stream (shared with sgemm_splitk)."""
    import torch
    for t, name in ((x, "x"), (wt, "wt")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.device.type != "cuda":
            raise TypeError("%s must be a float32 CUDA tensor" % name)
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous 4-D tensor" % name)
    N, H, W, C = x.shape
    K, R, S, C2 = wt.shape
    if C2 != C:
        raise ValueError("channel counts differ: x has %d, wt has %d" % (C, C2))
    P, Q = conv2d_output_size(H, W, R, S, pad, stride, dil)
    if out is None:
        out = torch.empty((N, P, Q, K), dtype=torch.float32, device=x.device)
    if tuple(out.shape) != (N, P, Q, K) or not out.is_contiguous():
        raise ValueError("out must be a contiguous (%d, %d, %d, %d) tensor" % (N, P, Q, K))
    _, _, nbytes, _ = conv2d_splitk_plan(N, H, W, C, K, R, S, pad, stride, dil, splits, config)
    if workspace is None:
        workspace = splitk_workspace(x.device, nbytes, stream)
    with torch.cuda.device(x.device):
        st = conv2d_nhwc_splitk_raw(N, H, W, C, K, R, S, x.data_ptr(), wt.data_ptr(),
                                    out.data_ptr(), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), pad, stride,
                                    dil, splits, _stream_handle(stream, x.device), config)
    _check(st, "conv2d_nhwc_splitk")
    return out


def conv2d_config_has_splitk(config: int) -> bool:
    st = _native.lib().conv2d_config_has_splitk(int(config))
    if st < 0:
        raise _native.SgemmError(st, "conv2d_config_has_splitk")
    return bool(st)


def conv2d_config_available(config: int) -> bool:
    st = _native.lib().conv2d_config_available(int(config))
    if st < 0:
        raise _native.SgemmError(st, "conv2d_config_available")
    return bool(st)


def conv2d_select_config(N, H, W, C, K, R, S, pad=0, stride=1, dil=1) -> int:
    ph, pw = _pair(pad, "pad")
    sh, sw = _pair(stride, "stride")
    dh, dw = _pair(dil, "dil")
    st = _native.lib().conv2d_select_config(N, H, W, C, K, R, S, ph, pw, sh, sw, dh, dw)
    if st < 0:
        raise _native.SgemmError(st, "conv2d_select_config")
    return st


def attention_raw(BH, Sq, Skv, D, q_ptr, k_ptr, v_ptr, o_ptr, scale, causal=False,
                  stream=0) -> int:
    """Blockwise attention on device addresses (include/attention.h); returns
    the status."""
    return _native.lib().attention_fwd(BH, Sq, Skv, D, q_ptr, k_ptr, v_ptr, o_ptr, float(scale),
                                       int(bool(causal)), stream)


def attention(q, k, v, scale=None, causal=False, out=None, stream=None):
    """softmax(scale q k^T) v per head for contiguous float32 CUDA tensors
    shaped (..., S, D) (leading dimensions are heads); scale defaults to
    1/sqrt(D).  Returns a tensor shaped like q."""
    import math
    import torch
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.device.type != "cuda":
            raise TypeError("%s must be a float32 CUDA tensor" % name)
        if t.dim() < 2 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous tensor of at least 2 dimensions" % name)
    if q.shape[:-2] != k.shape[:-2] or k.shape != v.shape or q.shape[-1] != k.shape[-1]:
        raise ValueError("shapes do not match: q %s, k %s, v %s"
                         % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    Sq, D = q.shape[-2], q.shape[-1]
    Skv = k.shape[-2]
    BH = math.prod(q.shape[:-2])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped like q")
    with torch.cuda.device(q.device):
        st = attention_raw(BH, Sq, Skv, D, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                           out.data_ptr(), scale, causal, _stream_handle(stream, q.device))
    _check(st, "attention_fwd")
    return out
