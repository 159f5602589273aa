"""Comparison of GPU results with the oracle, to the acceptance bar.

* Integer-valued inputs whose partial sums stay below 2^24: every partial sum
  is exact in FP32 whatever the order, so the result is unique and must match
  the oracle bit for bit (as FP32, so -0 and +0 differ).
* Otherwise, elementwise |C - C_ref| <= 2e-4 * sum_k |A[i,k]| |B[k,j]|, in FP64.
  Where that magnitude sum is 0 the element must be exactly 0.
"""
import numpy as np

REL_TOL = 2e-4


def assert_bitwise(C_gpu, C_ref, what=""):
    got = np.ascontiguousarray(np.asarray(C_gpu, dtype=np.float32))
    want = np.ascontiguousarray(np.asarray(C_ref, dtype=np.float64).astype(np.float32))
    assert got.shape == want.shape, (got.shape, want.shape)
    diff = got.view(np.uint32) != want.view(np.uint32)
    if diff.any():
        idx = np.argwhere(diff)[:5]
        raise AssertionError("%s: %d of %d elements differ bitwise, first at %s: got %s want %s"
                             % (what, int(diff.sum()), diff.size, idx.tolist(),
                                got[tuple(idx[0])], want[tuple(idx[0])]))


def assert_within_tolerance(C_gpu, C_ref, C_abs, what=""):
    """Returns the largest |err| / (|A||B|) ratio seen."""
    got = np.asarray(C_gpu, dtype=np.float64)
    ref = np.asarray(C_ref, dtype=np.float64)
    mag = np.asarray(C_abs, dtype=np.float64)
    assert got.shape == ref.shape == mag.shape
    err = np.abs(got - ref)
    bad = ~(err <= REL_TOL * mag)  # NaN counts as bad
    if bad.any():
        idx = np.argwhere(bad)[:5]
        i0 = tuple(idx[0])
        raise AssertionError("%s: %d of %d elements outside tolerance, first at %s: got %r "
                             "want %r (|A||B| = %r)" % (what, int(bad.sum()), bad.size,
                                                         idx.tolist(), got[i0], ref[i0], mag[i0]))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(mag > 0, err / mag, 0.0)
    return float(ratio.max()) if ratio.size else 0.0
