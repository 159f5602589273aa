"""Work and traffic models of the tiled product, used to judge measurements.

These are the closed forms the pages give, generalised from the square case
to M x N x K and rectangular tiles; each function names its source.  They
count scalar values or instructions, not cache transactions.
"""
from __future__ import annotations


def ceil_div(a: int, b: int) -> int:
    """Blocks needed to cover `a` items with `b` per block ("CMU DLSys Lecture
    12: GPU Acceleration", section 1: ceil(n/T) blocks, the last one guarded)."""
    if b <= 0:
        raise ValueError("block size must be positive")
    return -(-a // b)


def flops(M: int, N: int, K: int, batch: int = 1) -> int:
    """2MNK: one multiply and one add per fused multiply-add ("Tiling
    Hierarchy on GPUs", sections "Where the FLOPs come from" and "Inner
    Product": the product is M*N*K FMAs)."""
    return 2 * M * N * K * batch


def compulsory_bytes(M: int, N: int, K: int, batch: int = 1, elem: int = 4) -> int:
    """Each input read once and the output written once."""
    return elem * (M * K + K * N + M * N) * batch


def untiled_input_loads(M: int, N: int, K: int) -> int:
    """One output per thread, every operand from global memory: 2K values per
    output ("Tiling Hierarchy on GPUs", "Inner Product"; "CMU DLSys Lecture 12"
    introduction and section 5 table: 2N^3 for a square product)."""
    return 2 * M * N * K


def register_tile_input_loads(M: int, N: int, K: int, m: int, n: int) -> int:
    """Each thread owns an m x n output tile and loads m + n values per k
    step, with no shared staging ("CMU DLSys Lecture 12", section 4:
    (N/V)^2 tiles x N steps x 2V = 2N^3/V)."""
    return (M // m) * (N // n) * K * (m + n)


def global_to_shared_loads(M: int, N: int, K: int, BM: int, BN: int, BK: int | None = None,
                           padded: bool = False) -> int:
    """Scalar values copied from global memory into block-shared staging.

    A block owning a BM x BN output tile stages BM*BK + BK*BN values per
    reduction stage ("CMU DLSys Lecture 12", section 5, "Count each memory
    boundary separately": (N/L)^2 blocks x N/S stages x 2SL = 2N^3/L; the
    stage depth cancels).  For M x N x K this is M*N*K*(1/BN + 1/BM).  With
    `padded`, whole tiles are counted (ragged edges load zero-filled padding).
    """
    if not padded:
        if M % BM or N % BN:
            raise ValueError("unpadded count needs tile-aligned M and N")
        return M * N * K // BN + M * N * K // BM
    if BK is None:
        raise ValueError("padded count needs BK")
    tiles = ceil_div(M, BM) * ceil_div(N, BN)
    return tiles * ceil_div(K, BK) * (BM + BN) * BK


def shared_to_register_loads(M: int, N: int, K: int, WM: int, WN: int) -> int:
    """Values read from shared staging into registers: each register tile of
    WM x WN outputs reads WM + WN values per k step ("CMU DLSys Lecture 12",
    section 5: 2N^3/V).  For the matrix-core path (WM, WN) is the wave tile."""
    if M % WM or N % WN:
        raise ValueError("count needs tile-aligned M and N")
    return (M // WM) * (N // WN) * K * (WM + WN)


def flop_per_global_byte(N: int, L: int, elem: int = 4, with_output: bool = False):
    """Logical arithmetic intensity of the square product with L x L block
    tiles: 2N^3 FLOPs over 4 * 2N^3/L input bytes = L/4 ("CMU DLSys Lecture
    12", section 5), optionally adding the N^2 output write.  Returned as a
    (numerator, denominator) pair of integers."""
    num = 2 * N ** 3
    den = elem * (2 * N ** 3 // L) + (elem * N * N if with_output else 0)
    from math import gcd
    g = gcd(num, den)
    return num // g, den // g


def register_budget(m: int, n: int, prefetch: bool = True) -> int:
    """Registers of an m x n thread tile before bookkeeping: m*n accumulators
    plus one (m + n) operand set, or two with register prefetching ("Tiling
    Hierarchy on GPUs", "Register Tiling", "Register prefetching", "Reducing
    Overhead Slots": m*n + 2(m+n))."""
    return m * n + (2 if prefetch else 1) * (m + n)


def threads_per_block(BM: int, BN: int, m: int, n: int) -> int:
    """Threads in a BM x BN block whose threads own m x n tiles ("Tiling
    Hierarchy on GPUs", "Reducing Overhead Slots")."""
    return (BM * BN) // (m * n)


def issue_slot_efficiency(useful: int, overhead: int, idle: int) -> float:
    """eta = FMA-issuing cycles over all cycles ("Tiling Hierarchy on GPUs",
    "Issue Slot Efficiency")."""
    return useful / (useful + overhead + idle)


def mfma_instructions(M: int, N: int, K: int, BM: int, BN: int, BK: int, MI: int,
                      batch: int = 1) -> int:
    """Matrix instructions one launch issues, padded tiles included:
    v_mfma_f32_32x32x2_f32 (MI = 32) covers a 32x32 tile and 2 k values,
    v_mfma_f32_16x16x4_f32 (MI = 16) a 16x16 tile and 4 k values."""
    kstep = {32: 2, 16: 4}[MI]
    tiles = ceil_div(M, BM) * ceil_div(N, BN) * batch
    return tiles * (BM // MI) * (BN // MI) * ceil_div(K, BK) * (BK // kstep)


def valu_fma_instructions(M: int, N: int, K: int, BM: int = 128, BN: int = 128, BK: int = 8,
                          batch: int = 1) -> int:
    """Wave-level FP32 FMA instructions of the register-tiled vector path: one
    64-lane instruction per 64 FMAs, padded tiles included."""
    tiles = ceil_div(M, BM) * ceil_div(N, BN) * batch
    return tiles * BM * BN * ceil_div(K, BK) * BK // 64


def window_independent_loads(n: int, W: int) -> int:
    """Input reads of n window sums when every output loads its own W values
    ("CMU DLSys Lecture 12", section 3: T(2R+1) for a block of T outputs)."""
    return n * W


def window_staged_loads(n: int, W: int, T: int) -> int:
    """Input values staged by blocks of T outputs: each full block loads its T
    outputs' span plus the W - 1 halo values (T + 2R with W = 2R + 1); a last
    partial block of r outputs loads r + W - 1 (section 3)."""
    if T <= 0:
        raise ValueError("block size must be positive")
    full, rest = divmod(n, T)
    return full * (T + W - 1) + (rest + W - 1 if rest else 0)


def window_bytes(n: int, W: int, elem: int = 4) -> int:
    """Compulsory traffic of the window sum: the n + W - 1 inputs read once
    and the n outputs written once."""
    return elem * ((n + W - 1 if n > 0 else 0) + n)
