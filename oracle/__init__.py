"""CPU oracle for C = A x B in FP32 inputs with an FP64 result (and for the
sliding window sum, the 2-D convolution and blockwise attention built on the
same staging idea).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
imports, links or calls it, and it imports nothing from the GPU library.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc, OpenMP over
rows).  This module only builds that file and marshals numpy arrays to it.
What it computes and the passages it follows are stated in ``oracle.c``:
the inner-product definition ("Tiling Hierarchy on GPUs", section "Inner
Product"; "Tiling Strategies", section 2), with zero-initialised accumulators
and no read of C ("CMU DLSys Lecture 12: GPU Acceleration", section 5).

Every function returns FP64 arrays: the product ``C`` and the magnitude sum
``Cabs[i, j] = sum_k |A[i, k]| |B[k, j]|`` that the acceptance bound uses.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP, no fast-math)."""
    if (not force and os.path.exists(_LIB)
            and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC)):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_sgemm_f64.argtypes = [i64, i64, i64, p, i64, p, i64, p, p, i64, ctypes.c_int]
    lib.oracle_sgemm_f64.restype = ctypes.c_int
    lib.oracle_sgemm_strided_batched_f64.argtypes = [
        i64, i64, i64, p, i64, i64, p, i64, i64, p, p, i64, i64, i64, ctypes.c_int]
    lib.oracle_sgemm_strided_batched_f64.restype = ctypes.c_int
    lib.oracle_sgemm_entries_f64.argtypes = [i64, p, i64, p, i64, i64, p, p, p, p]
    lib.oracle_sgemm_entries_f64.restype = None
    lib.oracle_conv2d_nhwc_f64.argtypes = [i64] * 13 + [p, p, p, p]
    lib.oracle_conv2d_nhwc_f64.restype = ctypes.c_int
    lib.oracle_conv2d_nhwc_entries_f64.argtypes = [i64] * 13 + [p, p, i64, p, p, p]
    lib.oracle_conv2d_nhwc_entries_f64.restype = ctypes.c_int
    lib.oracle_attention_f64.argtypes = [i64, i64, i64, i64, p, p, p, ctypes.c_float,
                                         ctypes.c_int, p, p, p]
    lib.oracle_attention_f64.restype = ctypes.c_int
    lib.oracle_attention_rows_f64.argtypes = [i64, i64, i64, i64, p, p, p, ctypes.c_float,
                                              ctypes.c_int, i64, p, p, p, p]
    lib.oracle_attention_rows_f64.restype = ctypes.c_int
    lib.oracle_sgemm_ex_f64.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                        ctypes.c_float, p, i64, p, i64, ctypes.c_float, p, i64,
                                        p, p, i64, ctypes.c_int]
    lib.oracle_sgemm_ex_f64.restype = ctypes.c_int
    lib.oracle_sgemm_ex_entries_f64.argtypes = [ctypes.c_int, ctypes.c_int, i64, ctypes.c_float,
                                                p, i64, p, i64, ctypes.c_float, p, i64, i64, p,
                                                p, p, p]
    lib.oracle_sgemm_ex_entries_f64.restype = None
    lib.oracle_window_sum_f64.argtypes = [i64, i64, p, p, p]
    lib.oracle_window_sum_f64.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _f32_flat(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype != np.float32:
        raise TypeError("oracle operands must be float32, got %s" % a.dtype)
    return np.ascontiguousarray(a.reshape(-1))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def max_threads() -> int:
    return _load().oracle_max_threads()


def sgemm_f64(M: int, N: int, K: int, A, lda: int, B, ldb: int, nthreads: int = 0):
    """C = A x B from flat row-major buffers with leading dimensions.

    ``A`` holds at least (M-1)*lda + K floats and ``B`` at least
    (K-1)*ldb + N floats; padding past each row's end is never read.
    Returns ``(C, Cabs, threads_used)`` with C and Cabs of shape (M, N), FP64.
    """
    lib = _load()
    a, b = _f32_flat(A), _f32_flat(B)
    if M > 0 and K > 0 and a.size < (M - 1) * lda + K:
        raise ValueError("A buffer too small")
    if K > 0 and N > 0 and b.size < (K - 1) * ldb + N:
        raise ValueError("B buffer too small")
    C = np.empty((M, N), dtype=np.float64)
    Cabs = np.empty((M, N), dtype=np.float64)
    used = 1
    if M > 0 and N > 0:
        used = lib.oracle_sgemm_f64(M, N, K, _ptr(a), lda, _ptr(b), ldb,
                                    _ptr(C), _ptr(Cabs), N, nthreads)
    return C, Cabs, used


def matmul_f64(A, B, nthreads: int = 0):
    """Convenience form on 2-D float32 arrays (rows may be strided views)."""
    A = np.asarray(A)
    B = np.asarray(B)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    C, Cabs, _ = sgemm_f64(M, N, K, np.ascontiguousarray(A), K,
                           np.ascontiguousarray(B), N, nthreads)
    return C, Cabs


def sgemm_strided_batched_f64(M, N, K, A, lda, strideA, B, ldb, strideB, batch,
                              nthreads: int = 0):
    """Batched product; returns C and Cabs of shape (batch, M, N)."""
    lib = _load()
    a, b = _f32_flat(A), _f32_flat(B)
    C = np.empty((batch, M, N), dtype=np.float64)
    Cabs = np.empty((batch, M, N), dtype=np.float64)
    if batch > 0 and M > 0 and N > 0:
        need_a = (batch - 1) * strideA + (M - 1) * lda + K if K > 0 else 0
        need_b = (batch - 1) * strideB + (K - 1) * ldb + N if K > 0 else 0
        if a.size < need_a or b.size < need_b:
            raise ValueError("operand buffer too small")
        lib.oracle_sgemm_strided_batched_f64(M, N, K, _ptr(a), lda, strideA, _ptr(b), ldb,
                                             strideB, _ptr(C), _ptr(Cabs), N, M * N, batch,
                                             nthreads)
    return C, Cabs


def entries_f64(K: int, A, lda: int, B, ldb: int, rows, cols):
    """Selected entries C[rows[e], cols[e]] and their magnitude sums, FP64.

    Bitwise equal to the same entries of :func:`sgemm_f64` (same k order).
    """
    lib = _load()
    a, b = _f32_flat(A), _f32_flat(B)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    c = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    if r.shape != c.shape:
        raise ValueError("rows and cols differ in length")
    out = np.empty(r.size, dtype=np.float64)
    out_abs = np.empty(r.size, dtype=np.float64)
    if r.size:
        if K > 0:
            if a.size < int(r.max()) * lda + K or b.size < (K - 1) * ldb + int(c.max()) + 1:
                raise ValueError("entry index outside the operands")
        lib.oracle_sgemm_entries_f64(K, _ptr(a), lda, _ptr(b), ldb, r.size, _ptr(r), _ptr(c),
                                     _ptr(out), _ptr(out_abs))
    return out, out_abs


def _stored_shape(trans: bool, rows: int, cols: int):
    """Rows and columns of the stored matrix whose op() is rows x cols."""
    return (cols, rows) if trans else (rows, cols)


def _need(rows: int, cols: int, ld: int) -> int:
    return (rows - 1) * ld + cols if rows > 0 and cols > 0 else 0


def sgemm_ex_f64(transA: bool, transB: bool, M: int, N: int, K: int, alpha: float, A, lda: int,
                 B, ldb: int, beta: float, C_in=None, ldc: int = 0, nthreads: int = 0):
    """C = alpha op(A) op(B) + beta C_in (definitions in oracle.c); FP64
    (C, Cabs, threads_used) of shape (M, N).  A is stored K x M when transA,
    B is stored N x K when transB; C_in is read only when beta != 0."""
    lib = _load()
    alpha = float(np.float32(alpha))
    beta = float(np.float32(beta))
    a = _f32_flat(A) if A is not None else np.zeros(1, np.float32)
    b = _f32_flat(B) if B is not None else np.zeros(1, np.float32)
    if alpha != 0.0 and K > 0 and M > 0 and N > 0:
        if a.size < _need(*_stored_shape(transA, M, K), lda):
            raise ValueError("A buffer too small")
        if b.size < _need(*_stored_shape(transB, K, N), ldb):
            raise ValueError("B buffer too small")
    c = np.zeros(1, np.float32)
    if beta != 0.0:
        c = _f32_flat(C_in)
        if c.size < _need(M, N, ldc):
            raise ValueError("C buffer too small")
    out = np.empty((M, N), dtype=np.float64)
    out_abs = np.empty((M, N), dtype=np.float64)
    used = 1
    if M > 0 and N > 0:
        used = lib.oracle_sgemm_ex_f64(int(bool(transA)), int(bool(transB)), M, N, K, alpha,
                                       _ptr(a), lda, _ptr(b), ldb, beta, _ptr(c), ldc,
                                       _ptr(out), _ptr(out_abs), N, nthreads)
    return out, out_abs, used


def ex_entries_f64(transA: bool, transB: bool, K: int, alpha: float, A, lda: int, B, ldb: int,
                   beta: float, C_in, ldc: int, rows, cols):
    """Selected entries of :func:`sgemm_ex_f64`, bitwise equal to the full form."""
    lib = _load()
    alpha = float(np.float32(alpha))
    beta = float(np.float32(beta))
    a = _f32_flat(A)
    b = _f32_flat(B)
    c = _f32_flat(C_in) if beta != 0.0 else np.zeros(1, np.float32)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    cc = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    if r.shape != cc.shape:
        raise ValueError("rows and cols differ in length")
    if r.size and K > 0 and alpha != 0.0:
        m_need, n_need = int(r.max()) + 1, int(cc.max()) + 1
        if a.size < _need(*_stored_shape(transA, m_need, K), lda):
            raise ValueError("entry index outside A")
        if b.size < _need(*_stored_shape(transB, K, n_need), ldb):
            raise ValueError("entry index outside B")
    if r.size and beta != 0.0 and c.size < int(r.max()) * ldc + int(cc.max()) + 1:
        raise ValueError("entry index outside C")
    out = np.empty(r.size, dtype=np.float64)
    out_abs = np.empty(r.size, dtype=np.float64)
    if r.size:
        lib.oracle_sgemm_ex_entries_f64(int(bool(transA)), int(bool(transB)), K, alpha, _ptr(a),
                                        lda, _ptr(b), ldb, beta, _ptr(c), ldc, r.size, _ptr(r),
                                        _ptr(cc), _ptr(out), _ptr(out_abs))
    return out, out_abs


def window_sum_f64(n: int, W: int, x):
    """y[i] = sum_{d<W} x[i+d] for i < n (the lecture's sliding window, see
    oracle.c); returns FP64 (y, yabs).  x holds at least n + W - 1 floats."""
    lib = _load()
    xx = _f32_flat(x)
    if n < 0 or W < 1:
        raise ValueError("need n >= 0 and W >= 1")
    if n > 0 and xx.size < n + W - 1:
        raise ValueError("x holds fewer than n + W - 1 values")
    y = np.empty(n, dtype=np.float64)
    yabs = np.empty(n, dtype=np.float64)
    if n > 0:
        lib.oracle_window_sum_f64(n, W, _ptr(xx), _ptr(y), _ptr(yabs))
    return y, yabs


def conv_out_size(size: int, pad: int, f: int, stride: int, dil: int) -> int:
    """Output extent of the convolution along one axis (see oracle.c)."""
    span = size + 2 * pad - dil * (f - 1) - 1
    return 0 if span < 0 else span // stride + 1


def conv2d_nhwc_f64(x, wt, N: int, H: int, W: int, C: int, K: int, R: int, S: int,
                    pad=(0, 0), stride=(1, 1), dil=(1, 1)):
    """2-D convolution of NHWC input x (N*H*W*C floats) with KRSC filters wt
    (K*R*S*C floats), zero padding, stride and dilation (see oracle.c).
    Returns FP64 (y, yabs), each shaped (N, P, Q, K)."""
    lib = _load()
    xx = _f32_flat(x)
    ww = _f32_flat(wt)
    if min(stride) < 1 or min(dil) < 1 or min(pad) < 0:
        raise ValueError("stride and dilation must be positive, padding not negative")
    if xx.size < N * H * W * C or ww.size < K * R * S * C:
        raise ValueError("input or filter buffer too small")
    P = conv_out_size(H, pad[0], R, stride[0], dil[0])
    Q = conv_out_size(W, pad[1], S, stride[1], dil[1])
    y = np.empty((N, P, Q, K), dtype=np.float64)
    yabs = np.empty((N, P, Q, K), dtype=np.float64)
    st = lib.oracle_conv2d_nhwc_f64(N, H, W, C, K, R, S, pad[0], pad[1], stride[0], stride[1],
                                    dil[0], dil[1], _ptr(xx), _ptr(ww), _ptr(y), _ptr(yabs))
    if st != 0:
        raise ValueError("invalid convolution arguments")
    return y, yabs


def conv2d_nhwc_entries_f64(x, wt, N: int, H: int, W: int, C: int, K: int, R: int, S: int,
                            idx, pad=(0, 0), stride=(1, 1), dil=(1, 1)):
    """Selected outputs (flat indices into the N x P x Q x K output) of the
    convolution above; returns FP64 (y, yabs) of len(idx)."""
    lib = _load()
    xx = _f32_flat(x)
    ww = _f32_flat(wt)
    if min(stride) < 1 or min(dil) < 1 or min(pad) < 0:
        raise ValueError("stride and dilation must be positive, padding not negative")
    P = conv_out_size(H, pad[0], R, stride[0], dil[0])
    Q = conv_out_size(W, pad[1], S, stride[1], dil[1])
    ii = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).ravel())
    if ii.size and (ii.min() < 0 or ii.max() >= N * P * Q * K):
        raise ValueError("output index out of range")
    y = np.empty(ii.size, dtype=np.float64)
    yabs = np.empty(ii.size, dtype=np.float64)
    if ii.size:
        st = lib.oracle_conv2d_nhwc_entries_f64(N, H, W, C, K, R, S, pad[0], pad[1], stride[0],
                                                stride[1], dil[0], dil[1], _ptr(xx), _ptr(ww),
                                                ii.size, _ptr(ii), _ptr(y), _ptr(yabs))
        if st != 0:
            raise ValueError("invalid convolution arguments")
    return y, yabs


def attention_f64(Q, K, V, H: int, Sq: int, Skv: int, D: int, scale: float, causal: bool = False):
    """Scaled dot-product attention per head (see oracle.c): Q (H*Sq*D floats),
    K and V (H*Skv*D floats), row-major per head.  Returns FP64 (O, mag, smax):
    O and mag shaped (H, Sq, D), smax shaped (H, Sq)."""
    lib = _load()
    q, k, v = _f32_flat(Q), _f32_flat(K), _f32_flat(V)
    if min(H, Sq, Skv, D) < 0:
        raise ValueError("negative size")
    if q.size < H * Sq * D or k.size < H * Skv * D or v.size < H * Skv * D:
        raise ValueError("operand buffer too small")
    O = np.empty((H, Sq, D), dtype=np.float64)
    mag = np.empty((H, Sq, D), dtype=np.float64)
    smax = np.empty((H, Sq), dtype=np.float64)
    st = lib.oracle_attention_f64(H, Sq, Skv, D, _ptr(q), _ptr(k), _ptr(v), float(scale),
                                  int(bool(causal)), _ptr(O), _ptr(mag), _ptr(smax))
    if st != 0:
        raise ValueError("invalid attention arguments")
    return O, mag, smax


def attention_rows_f64(Q, K, V, H: int, Sq: int, Skv: int, D: int, scale: float, rows,
                       causal: bool = False):
    """Selected rows (flat index h * Sq + i) of the attention above; returns
    FP64 (O, mag, smax) shaped (len(rows), D), (len(rows), D), (len(rows),)."""
    lib = _load()
    q, k, v = _f32_flat(Q), _f32_flat(K), _f32_flat(V)
    rr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).ravel())
    if rr.size and (rr.min() < 0 or rr.max() >= H * Sq):
        raise ValueError("row index out of range")
    O = np.empty((rr.size, D), dtype=np.float64)
    mag = np.empty((rr.size, D), dtype=np.float64)
    smax = np.empty(rr.size, dtype=np.float64)
    if rr.size:
        st = lib.oracle_attention_rows_f64(H, Sq, Skv, D, _ptr(q), _ptr(k), _ptr(v),
                                           float(scale), int(bool(causal)), rr.size, _ptr(rr),
                                           _ptr(O), _ptr(mag), _ptr(smax))
        if st != 0:
            raise ValueError("invalid attention arguments")
    return O, mag, smax
