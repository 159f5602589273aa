"""Seeded synthetic inputs for the FP32 GEMM workloads.

This module holds input recipes only (shapes, layouts, value distributions,
seeds); none of the product's arithmetic.  Both sides of every parity check,
the HIP library and the CPU oracle, receive the very same float32 bits built
here on the CPU with ``torch.Generator`` (A is drawn first, then B).  Operands
too large for the host (the size-limit tests) are drawn on the device by
``device_operand``; the oracle then gets the rows it needs copied back, bit for
bit.

Layouts are row-major with leading dimensions; when a leading dimension
exceeds the row length the padding is filled with ``pad`` (NaN by default, so
a kernel that reads padding is caught by the NaN it picks up).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    lda: int
    ldb: int
    ldc: int
    dist_a: str          # "uniform" | "normal" | "int4"
    dist_b: str
    scale_a: float = 1.0
    scale_b: float = 1.0
    seed: int = 0
    batch: int = 1
    strideA: int = 0
    strideB: int = 0
    strideC: int = 0
    about: str = field(default="", compare=False)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch

    def describe(self) -> str:
        s = "sgemm M=%d N=%d K=%d lda=%d ldb=%d ldc=%d" % (
            self.M, self.N, self.K, self.lda, self.ldb, self.ldc)
        if self.batch != 1:
            s += " batch=%d strides=%d/%d/%d" % (self.batch, self.strideA, self.strideB,
                                                 self.strideC)
        return s + " A~%s B~%s seed=%d" % (_dist_text(self.dist_a, self.scale_a, self.K),
                                            _dist_text(self.dist_b, self.scale_b, self.K),
                                            self.seed)


def _dist_text(dist: str, scale: float, K: int) -> str:
    """The value distribution as drawn, scale included: normal(0, std),
    uniform[-a, a), or the integers -4..4."""
    if dist == "int4":
        return "int{-4..4}"
    sq = " (1/sqrt(K))" if K > 0 and abs(scale * math.sqrt(K) - 1.0) < 1e-12 and scale != 1.0 else ""
    if dist == "normal":
        return "normal(0,%g)%s" % (scale, sq)
    return "uniform[-%g,%g)%s" % (scale, scale, sq)


def _square(n, dist, scale, seed, about):
    return Workload("square%d" % n, n, n, n, n, n, n, dist, dist, scale, scale, seed,
                    about=about)


# The GEMM workloads.  The 4096^3 product is the headline one.
WORKLOADS = {
    "square1024": _square(1024, "uniform", 1.0, 0,
                          "1024^3 contiguous, uniform[-1,1), seed 0"),
    "square1024_int": Workload("square1024_int", 1024, 1024, 1024, 1024, 1024, 1024,
                               "int4", "int4", seed=0,
                               about="1024^3 contiguous, integers in {-4..4}, seed 0"),
    "square4096": _square(4096, "normal", 1.0 / math.sqrt(4096), 1,
                          "4096^3 contiguous, normal(0,1)/sqrt(K), seed 1"),
    "ragged": Workload("ragged", 4000, 3000, 4100, 4103, 3005, 3007, "uniform", "uniform",
                       seed=2, about="4000x3000x4100, lda=K+3, ldb=N+5, ldc=N+7, seed 2"),
    "tall": Workload("tall", 16384, 4096, 4096, 4096, 4096, 4096, "normal", "normal",
                     1.0, 0.02, 3, about="16384x4096x4096, A~normal(0,1), B~normal(0,0.02)"),
    "shard512": Workload("shard512", 512, 4096, 4096, 4096, 4096, 4096, "normal", "normal",
                         1.0 / math.sqrt(4096), 1.0 / math.sqrt(4096), 5,
                         about="512x4096x4096 (one of 8 row panels of 4096^3), "
                               "normal(0,1)/sqrt(K), seed 5"),
    "longk512": Workload("longk512", 512, 512, 8192, 8192, 512, 512, "normal", "normal",
                         1.0 / math.sqrt(8192), 1.0 / math.sqrt(8192), 6,
                         about="512x512x8192 (16 tiles of 128^2 for 256 CUs: the split-K "
                               "case), normal(0,1)/sqrt(K), seed 6"),
    "batched128": Workload("batched128", 128, 128, 128, 128, 128, 128, "uniform", "uniform",
                           seed=4, batch=1024, strideA=128 * 128, strideB=128 * 128,
                           strideC=128 * 128,
                           about="1024 x 128^3, contiguous strided batches, seed 4"),
}


@dataclass(frozen=True)
class WindowWorkload:
    """Sliding window sums y[i] = sum_{d<W} x[i+d], i < n; x holds n + W - 1
    values."""
    name: str
    n: int
    W: int
    dist: str
    seed: int
    about: str = field(default="", compare=False)

    @property
    def bytes(self) -> int:
        # each input read once, each output written once
        return 4 * (self.n + self.W - 1) + 4 * self.n

    def describe(self) -> str:
        return "window_sum n=%d W=%d x~%s seed=%d" % (self.n, self.W, self.dist, self.seed)


# The lecture's five-wide window over 2^28 outputs (1 GiB in, 1 GiB out), and a
# wide one.
WINDOW_WORKLOADS = {
    "window5": WindowWorkload("window5", 1 << 28, 5, "uniform", 6,
                              about="2^28 outputs, W = 5, uniform[-1,1), seed 6"),
    "window33": WindowWorkload("window33", 1 << 28, 33, "uniform", 7,
                               about="2^28 outputs, W = 33, uniform[-1,1), seed 7"),
}


def window_input(w: WindowWorkload) -> torch.Tensor:
    """The n + W - 1 float32 inputs of a window workload (CPU)."""
    gen = torch.Generator("cpu").manual_seed(w.seed)
    return draw(gen, w.n + w.W - 1, w.dist)


@dataclass(frozen=True)
class ConvWorkload:
    """2-D convolution: NHWC input (N, H, W, C), KRSC filters (K, R, S, C)."""
    name: str
    N: int
    H: int
    W: int
    C: int
    K: int
    R: int
    S: int
    pad: tuple
    stride: tuple
    dil: tuple
    seed: int
    about: str = field(default="", compare=False)

    @property
    def out_hw(self):
        P = (self.H + 2 * self.pad[0] - self.dil[0] * (self.R - 1) - 1) // self.stride[0] + 1
        Q = (self.W + 2 * self.pad[1] - self.dil[1] * (self.S - 1) - 1) // self.stride[1] + 1
        return max(P, 0), max(Q, 0)

    @property
    def flops(self) -> int:
        # every multiply-add of the implicit product, zero-padded taps included
        # (the dense-equivalent count)
        P, Q = self.out_hw
        return 2 * self.N * P * Q * self.K * self.R * self.S * self.C

    def _valid_taps_1d(self, size, pad, stride, dil, taps, out):
        """Sum over the output positions of the filter taps that land inside
        the input along one axis."""
        return sum(1 for o in range(out) for t in range(taps)
                   if 0 <= o * stride - pad + t * dil < size)

    @property
    def useful_flops(self) -> int:
        # multiply-adds whose input pixel lies inside the image: the taps on
        # the zero padding left out
        P, Q = self.out_hw
        rows = self._valid_taps_1d(self.H, self.pad[0], self.stride[0], self.dil[0], self.R, P)
        cols = self._valid_taps_1d(self.W, self.pad[1], self.stride[1], self.dil[1], self.S, Q)
        return 2 * self.N * rows * cols * self.K * self.C

    def describe(self) -> str:
        return ("conv2d_nhwc N=%d H=%d W=%d C=%d K=%d R=%d S=%d pad=%s stride=%s dil=%s "
                "x~normal(0,1) w~normal(0,1/sqrt(RSC)) seed=%d" % (
                    self.N, self.H, self.W, self.C, self.K, self.R, self.S, self.pad,
                    self.stride, self.dil, self.seed))


# ResNet-style 3x3 layers at batch 64 (14.8 GFLOP each), and a strided one.
CONV_WORKLOADS = {
    "conv3x3_c256": ConvWorkload("conv3x3_c256", 64, 14, 14, 256, 256, 3, 3, (1, 1), (1, 1),
                                 (1, 1), 8, about="64 x 14x14x256 -> 256, 3x3, pad 1"),
    "conv3x3_c128": ConvWorkload("conv3x3_c128", 64, 28, 28, 128, 128, 3, 3, (1, 1), (1, 1),
                                 (1, 1), 9, about="64 x 28x28x128 -> 128, 3x3, pad 1"),
    "conv3x3_s2": ConvWorkload("conv3x3_s2", 64, 28, 28, 128, 256, 3, 3, (1, 1), (2, 2),
                               (1, 1), 10, about="64 x 28x28x128 -> 256, 3x3, pad 1, stride 2"),
}


def conv_operands(w: ConvWorkload):
    """Flat float32 CPU buffers (x, wt) of a convolution workload: x drawn
    first, normal(0, 1); filters normal(0, 1/sqrt(R*S*C))."""
    gen = torch.Generator("cpu").manual_seed(w.seed)
    x = draw(gen, w.N * w.H * w.W * w.C, "normal")
    wt = draw(gen, w.K * w.R * w.S * w.C, "normal", 1.0 / math.sqrt(w.R * w.S * w.C))
    return x, wt


@dataclass(frozen=True)
class AttnWorkload:
    """Attention per head: Q (BH, Sq, D), K and V (BH, Skv, D)."""
    name: str
    BH: int
    Sq: int
    Skv: int
    D: int
    causal: bool
    seed: int
    about: str = field(default="", compare=False)

    @property
    def flops(self) -> int:
        # two products (scores, values) over the allowed query/key pairs
        if self.causal:
            pairs = sum(min(i + 1, self.Skv) for i in range(self.Sq))
        else:
            pairs = self.Sq * self.Skv
        return 4 * self.BH * pairs * self.D

    def describe(self) -> str:
        return ("attention BH=%d Sq=%d Skv=%d D=%d causal=%d q,k,v~normal(0,1) seed=%d"
                % (self.BH, self.Sq, self.Skv, self.D, int(self.causal), self.seed))


# Batch 4 x 16 heads of 2048 tokens, head dimension 128 (137 GFLOP without the
# mask), the same with the causal mask, and 32 heads of 4096 tokens at D = 64.
ATTN_WORKLOADS = {
    "attn_s2048_d128": AttnWorkload("attn_s2048_d128", 64, 2048, 2048, 128, False, 11),
    "attn_s2048_d128_causal": AttnWorkload("attn_s2048_d128_causal", 64, 2048, 2048, 128, True,
                                           12),
    "attn_s4096_d64": AttnWorkload("attn_s4096_d64", 32, 4096, 4096, 64, False, 13),
}


def attn_operands(w: AttnWorkload):
    """Flat float32 CPU buffers (Q, K, V), drawn in that order, normal(0, 1)."""
    gen = torch.Generator("cpu").manual_seed(w.seed)
    q = draw(gen, w.BH * w.Sq * w.D, "normal")
    k = draw(gen, w.BH * w.Skv * w.D, "normal")
    v = draw(gen, w.BH * w.Skv * w.D, "normal")
    return q, k, v


def draw(gen: torch.Generator, n: int, dist: str, scale: float = 1.0) -> torch.Tensor:
    """n float32 values from one of the recipes, using ``gen``."""
    if dist == "uniform":
        # uniform on [-1, 1)
        v = torch.rand(n, generator=gen, dtype=torch.float32) * 2.0 - 1.0
    elif dist == "normal":
        v = torch.randn(n, generator=gen, dtype=torch.float32)
    elif dist == "int4":
        v = torch.randint(-4, 5, (n,), generator=gen).to(torch.float32)
    elif dist == "ones":
        v = torch.ones(n, dtype=torch.float32)
    else:
        raise ValueError("unknown distribution %r" % dist)
    if scale != 1.0:
        v = v * scale
    return v


def place(values: torch.Tensor, rows: int, cols: int, ld: int, pad: float) -> torch.Tensor:
    """Lay ``rows x cols`` values row-major into a flat buffer with leading dim ``ld``."""
    if ld < cols:
        raise ValueError("leading dimension below row length")
    size = (rows - 1) * ld + cols if rows > 0 and cols > 0 else 0
    buf = torch.full((max(rows * ld, size),), pad, dtype=torch.float32)
    if rows > 0 and cols > 0:
        buf.view(-1)[: rows * ld].view(rows, ld)[:, :cols] = values.view(rows, cols)
    return buf


def operands(M: int, N: int, K: int, lda: int, ldb: int, seed: int,
             dist_a: str = "uniform", dist_b: str | None = None,
             scale_a: float = 1.0, scale_b: float = 1.0, pad: float = float("nan"),
             batch: int = 1, strideA: int | None = None, strideB: int | None = None):
    """Flat float32 CPU buffers (A, B) for one product or a strided batch.

    Matrix b of A starts at b*strideA floats (default: the padded matrix size);
    likewise B.  Values are drawn batch by batch, A before B within each.
    """
    dist_b = dist_a if dist_b is None else dist_b
    gen = torch.Generator("cpu").manual_seed(seed)
    one_a = M * lda
    one_b = K * ldb
    sa = one_a if strideA is None else strideA
    sb = one_b if strideB is None else strideB
    if batch > 1 and (sa < one_a or sb < one_b):
        raise ValueError("batch stride below one padded matrix")
    A = torch.full(((batch - 1) * sa + one_a,), pad, dtype=torch.float32)
    B = torch.full(((batch - 1) * sb + one_b,), pad, dtype=torch.float32)
    for b in range(batch):
        a_vals = draw(gen, M * K, dist_a, scale_a)
        b_vals = draw(gen, K * N, dist_b, scale_b)
        A[b * sa: b * sa + one_a] = place(a_vals, M, K, lda, pad)[:one_a]
        B[b * sb: b * sb + one_b] = place(b_vals, K, N, ldb, pad)[:one_b]
    return A, B


def workload_operands(w: Workload, pad: float = float("nan")):
    """Flat float32 CPU buffers (A, B) for one of the named workloads."""
    if w.batch == 1:
        return operands(w.M, w.N, w.K, w.lda, w.ldb, w.seed, w.dist_a, w.dist_b,
                        w.scale_a, w.scale_b, pad)
    return operands(w.M, w.N, w.K, w.lda, w.ldb, w.seed, w.dist_a, w.dist_b,
                    w.scale_a, w.scale_b, pad, batch=w.batch, strideA=w.strideA,
                    strideB=w.strideB)


def stored_operands(transA: bool, transB: bool, M: int, N: int, K: int, lda: int, ldb: int,
                    seed: int, dist_a: str = "uniform", dist_b: str | None = None,
                    pad: float = float("nan"), scale_a: float = 1.0, scale_b: float = 1.0):
    """Flat float32 CPU buffers (A, B) as stored for the general form: A is
    M x K, or K x M when transA; B is K x N, or N x K when transB.  A is drawn
    before B."""
    dist_b = dist_a if dist_b is None else dist_b
    gen = torch.Generator("cpu").manual_seed(seed)
    ra, ca = (K, M) if transA else (M, K)
    rb, cb = (N, K) if transB else (K, N)
    A = place(draw(gen, ra * ca, dist_a, scale_a), ra, ca, lda, pad)
    B = place(draw(gen, rb * cb, dist_b, scale_b), rb, cb, ldb, pad)
    return A, B


@dataclass(frozen=True)
class GeneralWorkload:
    """C = alpha op(A) op(B) + beta C with stored layouts: A is M x K, or
    K x M when transA; B is K x N, or N x K when transB."""
    name: str
    M: int
    N: int
    K: int
    transA: int
    transB: int
    lda: int
    ldb: int
    ldc: int
    alpha: float
    beta: float
    dist: str            # A and B (scaled) and C (unscaled)
    scale: float
    seed: int
    about: str = field(default="", compare=False)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def describe(self) -> str:
        return ("sgemm_ex transA=%d transB=%d M=%d N=%d K=%d lda=%d ldb=%d ldc=%d alpha=%g "
                "beta=%g A,B~%s C~%s seed=%d"
                % (self.transA, self.transB, self.M, self.N, self.K, self.lda, self.ldb, self.ldc,
                   self.alpha, self.beta, _dist_text(self.dist, self.scale, self.K),
                   _dist_text(self.dist, 1.0, self.K), self.seed))


# The general form at the headline size in the lecture's C = A^T B layout (A
# stored K x M), with beta != 0 so that C is read as well as written.
GENERAL_WORKLOADS = {
    "atb4096": GeneralWorkload("atb4096", 4096, 4096, 4096, 1, 0, 4096, 4096, 4096, 1.0, 0.5,
                               "normal", 1.0 / math.sqrt(4096), 14,
                               about="C = A^T B + 0.5 C at 4096^3, A stored K x M, "
                                     "normal(0,1)/sqrt(K) operands, normal(0,1) C, seed 14"),
    "atb_longk512": GeneralWorkload("atb_longk512", 512, 512, 8192, 1, 0, 512, 512, 512, 1.0,
                                    0.5, "normal", 1.0 / math.sqrt(8192), 16,
                                    about="C = A^T B + 0.5 C at 512x512x8192 (the thin long-K "
                                          "case, for sgemm_ex_splitk), normal(0,1)/sqrt(K) "
                                          "operands, normal(0,1) C, seed 16"),
}


def general_operands(w: GeneralWorkload, pad: float = float("nan")):
    """Flat float32 CPU buffers (A, B, C) for a general-form workload: A and B
    as stored_operands draws them, then C from seed + 1."""
    A, B = stored_operands(bool(w.transA), bool(w.transB), w.M, w.N, w.K, w.lda, w.ldb, w.seed,
                           w.dist, w.dist, pad, w.scale, w.scale)
    C = matrix(w.M, w.N, w.ldc, w.seed + 1, w.dist, pad)
    return A, B, C


def matrix(rows: int, cols: int, ld: int, seed: int, dist: str = "uniform",
           pad: float = float("nan")) -> torch.Tensor:
    """One flat float32 CPU buffer holding a rows x cols matrix (e.g. C's
    initial values for beta != 0)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    return place(draw(gen, rows * cols, dist), rows, cols, ld, pad)


def device_operand(batch: int, rows: int, cols: int, ld: int, stride: int, seed: int, device,
                   dist: str = "int4", pad: float = float("nan"), extra: int = 0) -> torch.Tensor:
    """A flat float32 buffer on ``device`` of (batch - 1) * stride + rows * ld
    + extra floats holding ``batch`` rows x cols matrices (matrix b at b *
    stride, leading dimension ld), drawn in place, matrix by matrix, from a
    seeded generator on that device: "int4" = integers -4..4, "uniform" =
    [-1, 1).  Everything else holds ``pad``."""
    if ld < cols or (batch > 1 and stride < rows * ld):
        raise ValueError("leading dimension or stride too small")
    gen = torch.Generator(device).manual_seed(seed)
    size = (batch - 1) * stride + rows * ld + extra if batch > 0 else extra
    buf = torch.full((size,), pad, dtype=torch.float32, device=device)
    for b in range(batch):
        view = buf[b * stride: b * stride + rows * ld].view(rows, ld)[:, :cols]
        if dist == "int4":
            view.random_(-4, 5, generator=gen)
        elif dist == "uniform":
            view.uniform_(-1.0, 1.0, generator=gen)
        else:
            raise ValueError("unknown distribution %r" % dist)
    return buf
