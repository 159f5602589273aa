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


def l2_read_requests(M: int, N: int, K: int, BM: int, BN: int, BK: int, batch: int = 1,
                     lda: int | None = None, ldb: int | None = None, line: int = 128,
                     elem: int = 4) -> int:
    """Read requests from the vector L1 to L2 for the staging of
    `global_to_shared_loads`: each tile reads, per BK slice, the valid part
    of each of its BM rows of A (k in [k0, min(k0 + BK, K))) and of each of
    the slice's rows of B (its valid BN columns), one request per `line`
    bytes each piece touches.  Rows start at multiples of lda (ldb) elements
    from a line-aligned base, so a piece that straddles a line costs one
    request more, and a piece shorter than a line (a BK = 16 slice reads 64
    bytes of each A row) costs a whole one.  Every tile of a tile row reads
    its A panel and every tile of a tile column its B panel."""
    import numpy as np
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    k0 = np.arange(0, K, BK, dtype=np.int64)
    kend = np.minimum(k0 + BK, K)
    r = np.arange(M, dtype=np.int64)[:, None]
    first = (r * lda + k0[None, :]) * elem // line
    last = ((r * lda + kend[None, :]) * elem - 1) // line
    a = int(np.sum(last - first + 1)) * ceil_div(N, BN)
    n0 = np.arange(0, N, BN, dtype=np.int64)
    nend = np.minimum(n0 + BN, N)
    k = np.arange(K, dtype=np.int64)[:, None]
    first = (k * ldb + n0[None, :]) * elem // line
    last = ((k * ldb + nend[None, :]) * elem - 1) // line
    b = int(np.sum(last - first + 1)) * ceil_div(M, BM)
    return (a + b) * batch


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


def xcd_of_blocks(nblocks: int, xcds: int = 8):
    """Tile id handled by each workgroup, by XCD: workgroups go to the XCDs
    round-robin (block id % xcds), and the kernels renumber them so that each
    XCD owns a contiguous run of tile ids (the first nblocks % xcds XCDs one
    more).  Returns a list of (first tile id, count) per XCD."""
    q, r = divmod(nblocks, xcds)
    out = []
    first = 0
    for x in range(xcds):
        n = q + (1 if x < r else 0)
        out.append((first, n))
        first += n
    return out


def grouped_tile(pid: int, tiles_m: int, tiles_n: int, group_m: int):
    """(tile row, tile column) of tile id pid in the grouped order: groups of
    group_m tile rows, the tile row varying fastest inside a group."""
    per_group = group_m * tiles_n
    group = pid // per_group
    first_m = group * group_m
    gsize = min(tiles_m - first_m, group_m)
    in_group = pid - group * per_group
    return first_m + in_group % gsize, in_group // gsize


def per_xcd_operand_bytes(M: int, N: int, K: int, BM: int, BN: int, batch: int = 1,
                          group_m: int = 8, xcds: int = 8, resident: int = 0,
                          elem: int = 4) -> int:
    """Bytes of A and B that reach the L2 caches when each XCD's L2 fetches
    every operand row panel and column panel that a round of its tiles uses
    exactly once.

    Each XCD has its own L2, so a panel used by tiles on several XCDs crosses
    into L2 once per XCD.  An XCD runs its tiles in rounds of `resident`
    (the workgroups its CUs hold at once; 0: all of them in one round), in
    tile-id order; a round streams its panels through K, far more than one
    L2 holds, so a panel used again in a later round is fetched again.  The
    count is the sum over XCDs and rounds of the distinct A panels (BM rows x
    K, clipped at M) and B panels (K x BN, clipped at N).  The output is not
    included.  Compulsory traffic counts each panel once for the whole chip.
    """
    tiles_m, tiles_n = ceil_div(M, BM), ceil_div(N, BN)
    per_matrix = tiles_m * tiles_n
    total = 0
    for first, count in xcd_of_blocks(per_matrix * batch, xcds):
        step = resident if resident > 0 else max(count, 1)
        for r0 in range(first, first + count, step):
            rows, cols = set(), set()
            for pid in range(r0, min(first + count, r0 + step)):
                b, t = divmod(pid, per_matrix)
                tm, tn = grouped_tile(t, tiles_m, tiles_n, group_m)
                rows.add((b, tm))
                cols.add((b, tn))
            total += sum(min(BM, M - tm * BM) for _, tm in rows) * K
            total += sum(min(BN, N - tn * BN) for _, tn in cols) * K
    return elem * total
