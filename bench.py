"""Throughput of the FP32 GEMM C = A x B on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--path mfma|valu]
                    [--workload square4096] [--no-cpu-baseline]
    python bench.py --workload window5      (sliding window sums, GB/s)
    python bench.py --workload conv3x3_c256 (2-D convolution, TFLOP/s)
    python bench.py --workload attn_s2048_d128 (blockwise attention, TFLOP/s)

One step is one call of the library on the named workload (default: the
4096^3 product, A and B ~ normal(0,1)/sqrt(K), seed 1), inputs resident in
device memory before timing starts.  W untimed calls, then K calls timed with
HIP events recorded on the stream the kernel is launched on, bracketed by
device synchronisation (GEMM defaults: W and K each fill about 0.1 s).
Prints one JSON line:

  value      whole-job TFLOP/s = 2MNK / (time per step); with --cold, the mean
             of single launches each preceded by a 512 MiB write that evicts the
             operands from the caches
  single_launch  median and best of launches timed one by one
  roofline   achieved TFLOP/s of the GEMM kernel against the FP32 matrix peak
             (157.3 TFLOP/s), and HBM traffic measured with rocprofv3 counters
             when the committed counter summary matches the current kernel source
  cpu_baseline  the CPU oracle on a bounded sample (leading rows of C) of the
             same workload, on all host threads
  comparators   the vector-ALU path and torch.mm / torch.bmm (hipBLASLt) on the
             same operands with the same timing
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP32 GEMM TFLOP/s at M=N=K=4096 on 1 MI355X; % of FP32 peak"
PEAK_FP32_TFLOPS = 157.3      # MI355X dense FP32 (vector and matrix)
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "tiled_fp32_gemm_sgemm_amd", "csrc")
def gemm_traffic_file(path: str, workload: str) -> str:
    """The committed counter summary of a GEMM workload on a path."""
    return os.path.join(ROOT, "profiles", "sgemm_%s_%s_counters.txt" % (path, workload))


def conv_traffic_file(path: str, workload: str) -> str:
    """The committed counter summary of a convolution workload: conv2d_nhwc
    (path mfma) or conv2d_nhwc_splitk (path splitk)."""
    return os.path.join(ROOT, "profiles", "conv2d_%s%s_counters.txt"
                        % ("splitk_" if path == "splitk" else "", workload))
COPY_BYTES = 512 * 1024 * 1024   # larger than the 256 MB last-level cache
GEMM_WORK_S = 0.1                # default warm-up and timed work per GEMM phase (s)
SETTLE_S = 0.1                   # GEMM launches before the warm-up steps (clock settle)


def gemm_metric(w) -> str:
    """The metric a GEMM line reports: the headline string for the 4096^3
    product, the workload's own shape otherwise."""
    if w.name == "square4096":
        return METRIC
    shape = "M=%d N=%d K=%d" % (w.M, w.N, w.K)
    if w.batch != 1:
        shape = "batch %d x %s" % (w.batch, shape)
    return "FP32 GEMM TFLOP/s at %s on 1 MI355X; %% of FP32 peak" % shape


# Sources each kernel family is compiled from, the host table that gives the
# tiles their template arguments included.  A counter summary is used only
# while these hash to the value recorded in it and it names the tile the run
# uses.
GEMM_SOURCES = ("tile_common.hpp", "mfma_dl_kernel.hpp", "mfma_kernel.hpp", "valu_kernel.hpp",
                "sgemm.hip")
WINDOW_SOURCES = ("window.hip", "window_kernel.hpp", "tile_common.hpp")
WINDOW_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "window_sum_window5_counters.txt")
ATTN_SOURCES = ("attention.hip", "attention_kernel.hpp", "mfma_dl_kernel.hpp", "mfma_kernel.hpp",
                "tile_common.hpp")
ATTN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_attn_s2048_d128_counters.txt")


def kernel_source_hash(names=GEMM_SOURCES) -> str:
    h = hashlib.sha256()
    for name in sorted(names):
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(path: str, names=GEMM_SOURCES, tile=None, chunks=None):
    """HBM bytes per launch from a committed counter summary, or None when it
    is missing, was taken on a different kernel source, on another tile or
    (split-K) with another chunk count."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(names):
        return None
    if tile is not None and not vals.get("mfma_instructions_closed_form", "").endswith(
            "(tile %s)" % tile):
        return None
    if chunks is not None and vals.get("splitk_chunks", "").split()[:1] != [str(chunks)]:
        return None
    try:
        return float(vals["beyond_l2_bytes_per_launch"].split()[0])
    except (KeyError, ValueError):
        return None


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _per_dispatch(rows, name_part):
    """{dispatch id: {counter: value, 'dur_s': seconds}} for kernels whose name
    contains name_part."""
    out = {}
    for r in rows:
        if name_part not in r["Kernel_Name"]:
            continue
        d = out.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["dur_s"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    return out


def _mean(vals):
    vals = list(vals)
    return sum(vals) / len(vals) if vals else float("nan")


def summarize_trace(stats_csv: str, out: str, command: str, trace_csv: str = None,
                    timed: int = 0, made_by: str = None, after: int = 0) -> None:
    """Text summary of a rocprofv3 --kernel-trace --stats kernel_stats.csv.
    With the kernel_trace.csv and the bench's timed step count, also the
    average over the `timed` dispatches of each kernel that precede its last
    `after` ones (the launches the bench times in one event pair; before them
    come the warm-up, after them the launches timed one by one)."""
    rows = _read_csv(stats_csv)
    per_kernel = {}
    if trace_csv:
        for r in sorted(_read_csv(trace_csv), key=lambda r: int(r["Dispatch_Id"])):
            per_kernel.setdefault(r["Kernel_Name"], []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# rocprofv3 kernel statistics (durations in microseconds)",
             "# command: " + command]
    if made_by:
        lines.append("# summary: " + made_by)
    lines.append("")
    for r in rows:
        name = r.get("Name") or r.get("KernelName") or r.get("Kernel_Name")
        calls = int(float(r.get("Calls", 0)))
        avg_us = float(r.get("AverageNs", 0)) / 1e3
        lines.append("kernel: %s" % name)
        lines.append("  calls: %d  average_us: %.2f  min_us: %.2f  max_us: %.2f  percent: %s"
                     % (calls, avg_us, float(r.get("MinNs", 0)) / 1e3,
                        float(r.get("MaxNs", 0)) / 1e3, r.get("Percentage", "")))
        durs = per_kernel.get(name, [])
        if timed and len(durs) >= timed + after:
            sel = durs[len(durs) - after - timed:len(durs) - after]
            where = ("last %d dispatches" % timed if after == 0 else
                     "%d dispatches before the last %d" % (timed, after))
            lines.append("  timed_average_us (%s): %.2f" % (where, sum(sel) / timed))
    open(out, "w").write("\n".join(lines) + "\n")


def conv_compulsory_bytes(w) -> int:
    """Input, filters and output, each moved once."""
    P, Q = w.out_hw
    return 4 * (w.N * w.H * w.W * w.C + w.K * w.R * w.S * w.C + w.N * P * Q * w.K)


def trace_average_us(path: str):
    """The kernel's average duration from a committed trace summary: the
    timed dispatches' average when recorded, else the plain average (first
    kernel listed), or None."""
    if not path or not os.path.exists(path):
        return None
    plain = None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("timed_average_us"):
                return float(line.rsplit(":", 1)[1])
            if plain is None and line.startswith("calls:") and "average_us:" in line:
                plain = float(line.split("average_us:")[1].split()[0])
    return plain


MAX_CLOCK_GHZ = 2.4           # MI355X peak engine clock
SIMDS = 1024                  # 256 CUs x 4 SIMDs
MFMA_FLOP_PER_SIMD_CYCLE = 64  # 157.3 TFLOP/s / (1024 SIMDs x 2.4 GHz)


def summarize_counters(out: str, workload: str, path: str, kernel_part: str, fetch_csv: str,
                       write_csv: str, sq_csvs, commands, config=None, trace_summary=None,
                       splits: int = 0) -> None:
    """Counter summary: instruction counts against the closed forms, LDS bank
    conflicts, utilisation and the bytes that cross from L2 to memory.

    Utilisation is taken over the kernel's duration without the profiler
    (the trace summary's timed average), at the 2.4 GHz peak clock: busy
    cycles / (SIMDs x 2.4 GHz x duration).  That denominator is the most
    cycles the kernel could have had, so the fraction never exceeds 1 and
    times peak it gives the rate the trace timed.  GRBM_GUI_ACTIVE over the
    counter run's own dispatch gives a clock only for dispatches long enough
    that the profiler's set-up and drain around them do not count: it is left
    out when it comes above 2.4 GHz.
    Memory side: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) count requests
    from the L2 caches to memory, that is misses of each XCD's L2, which the
    256 MB last-level cache (MALL) in front of HBM may still serve; they are
    scaled by the same counters on a copy kernel of known size.  The read
    requests by size (32, 64 and 128 bytes) give the same bytes without a
    scale, as a check of it."""
    from workloads import WINDOW_WORKLOADS, WORKLOADS
    from tiled_fp32_gemm_sgemm_amd import model
    import tiled_fp32_gemm_sgemm_amd as sg
    from workloads import ATTN_WORKLOADS, CONV_WORKLOADS, GENERAL_WORKLOADS
    window = workload in WINDOW_WORKLOADS
    conv = workload in CONV_WORKLOADS
    attn = workload in ATTN_WORKLOADS
    general = workload in GENERAL_WORKLOADS
    gemm = not (window or conv or attn or general)
    w = (WINDOW_WORKLOADS[workload] if window else
         CONV_WORKLOADS[workload] if conv else
         ATTN_WORKLOADS[workload] if attn else
         GENERAL_WORKLOADS[workload] if general else WORKLOADS[workload])
    L = ["# rocprofv3 hardware counters, %s path, workload %s" % (path, w.describe()),
         "# commands (one counter pass each, run from the repository root):"]
    L += ["#   " + c for c in commands]
    L.append("kernel_source_sha256_16: %s" % kernel_source_hash(
        WINDOW_SOURCES if window else ATTN_SOURCES if attn else GEMM_SOURCES))
    if attn or conv:
        L.append("flops_per_launch: %d" % w.flops)
    t_us = trace_average_us(trace_summary)
    if t_us is not None:
        L.append("trace_average_us: %.2f (%s, timed dispatches without the profiler)"
                 % (t_us, os.path.relpath(trace_summary, ROOT)))

    merged = {}
    durs = []
    for c in sq_csvs:
        for d in _per_dispatch(_read_csv(c), kernel_part).values():
            for k, v in d.items():
                if k not in ("name", "dur_s"):
                    merged.setdefault(k, []).append(v)
            if "GRBM_GUI_ACTIVE" in d:
                merged.setdefault("_clk", []).append(d["GRBM_GUI_ACTIVE"] / 8 / d["dur_s"])
            durs.append(d["dur_s"])
            merged.setdefault("_name", []).append(d["name"])
    val = {k: _mean(v) for k, v in merged.items() if not k.startswith("_")}
    if merged.get("_name"):
        L.append("kernel: %s" % merged["_name"][0])
    if durs:
        L.append("counter_run_dispatch_average_us: %.2f" % (_mean(durs) * 1e6))
    for k in sorted(val):
        L.append("%s: %.6g" % (k, val[k]))

    # ------------------------------------------------------------ utilisation
    cap = SIMDS * MAX_CLOCK_GHZ * 1e9 * (t_us * 1e-6) if t_us else None
    if "_clk" in merged:
        g = _mean(merged["_clk"]) / 1e9
        if g <= MAX_CLOCK_GHZ:
            L.append("grbm_clock_ghz_counter_run: %.3f (GRBM_GUI_ACTIVE / 8 XCDs / counter-run "
                     "dispatch duration)" % g)
        else:
            L.append("grbm_clock_ghz_counter_run: omitted (GRBM_GUI_ACTIVE / 8 / dispatch "
                     "duration = %.3f GHz exceeds the %.1f GHz maximum: on a dispatch this short "
                     "the active count includes the profiler's set-up and drain)"
                     % (g, MAX_CLOCK_GHZ))
    if "SQ_VALU_MFMA_BUSY_CYCLES" in val:
        busy = val["SQ_VALU_MFMA_BUSY_CYCLES"]
        if val.get("SQ_INSTS_VALU_MFMA_F32"):
            L.append("mfma_busy_cycles_per_instruction: %.2f (the counter adds the instruction's "
                     "issue cycles: busy / peak cycles is achieved / peak FLOP rate)"
                     % (busy / val["SQ_INSTS_VALU_MFMA_F32"]))
        if cap:
            u = busy / cap
            L.append("mfma_busy_fraction_at_2.4GHz: %.4f (SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs "
                     "x 2.4 GHz x trace_average_us))" % u)
            L.append("mfma_rate_tflops_from_busy: %.2f (fraction x 157.3)" % (u * PEAK_FP32_TFLOPS))
            flops = (w.flops if (attn or conv) else w.flops) if not window else 0
            if flops:
                L.append("trace_rate_tflops: %.2f (FLOPs per launch / trace_average_us)"
                         % (flops / (t_us * 1e-6) / 1e12))
    if "SQ_ACTIVE_INST_VALU" in val and "SQ_ACTIVE_INST_VALU2" in val and cap:
        # Quad-cycles summed over every SIMD: SQ_ACTIVE_INST_VALU adds one per
        # wave64 VALU instruction, SQ_ACTIVE_INST_VALU2 one per quad-cycle in
        # which a SIMD issued two (from two waves), so quad-cycles with any
        # VALU issue = ACTIVE - ACTIVE2.
        quads = cap / 4
        act, act2 = val["SQ_ACTIVE_INST_VALU"], val["SQ_ACTIVE_INST_VALU2"]
        L.append("valu_issue_quad_cycle_fraction_at_2.4GHz: %.4f ((SQ_ACTIVE_INST_VALU - "
                 "SQ_ACTIVE_INST_VALU2) / quad-cycles of 1024 SIMDs at 2.4 GHz over "
                 "trace_average_us)" % ((act - act2) / quads))
        L.append("valu_dual_issue_quad_cycle_fraction_at_2.4GHz: %.4f (SQ_ACTIVE_INST_VALU2 / "
                 "the same quad-cycles: a SIMD issued two VALU instructions)" % (act2 / quads))
        if "SQ_INSTS_VALU_FMA_F32" in val:
            # Two issue slots per SIMD quad-cycle, each a wave64 instruction
            # of 64 FMAs: all of them v_fmac_f32 is the 157.3 TFLOP/s peak.
            L.append("valu_fma_issue_slot_efficiency: %.4f (SQ_INSTS_VALU_FMA_F32 / (2 x the "
                     "quad-cycles): the pages' eta, FMA-issuing slots over all slots)"
                     % (val["SQ_INSTS_VALU_FMA_F32"] / (2 * quads)))
    if "SQ_INSTS_VALU_FMA_F32" in val and cap:
        # one wave64 v_fmac_f32 is 64 FMAs = 128 FLOPs
        L.append("valu_fma_rate_tflops: %.2f (SQ_INSTS_VALU_FMA_F32 x 128 FLOP / trace_average_us)"
                 % (val["SQ_INSTS_VALU_FMA_F32"] * 128 / (t_us * 1e-6) / 1e12))

    # ----------------------------------------------------------- memory side
    compulsory = (w.bytes if window else conv_compulsory_bytes(w) if conv else
                  4 * w.BH * w.D * (2 * w.Sq + 2 * w.Skv) if attn else
                  4 * (w.M * w.K + w.K * w.N + 2 * w.M * w.N) if general and w.beta != 0 else
                  model.compulsory_bytes(w.M, w.N, w.K) if general else
                  model.compulsory_bytes(w.M, w.N, w.K, w.batch))
    copy_part = "MulFunctor"
    fetch = _per_dispatch(_read_csv(fetch_csv), kernel_part) if fetch_csv else {}
    write = _per_dispatch(_read_csv(write_csv), kernel_part) if write_csv else {}
    if fetch and write:
        cf = _per_dispatch(_read_csv(fetch_csv), copy_part)
        cw = _per_dispatch(_read_csv(write_csv), copy_part)
        f_copy = _mean(d["FETCH_SIZE"] for d in cf.values())
        w_copy = _mean(d["WRITE_SIZE"] for d in cw.values())
        f_scale = COPY_BYTES / (f_copy * 1024.0)
        w_scale = COPY_BYTES / (w_copy * 1024.0)
        f_kib = _mean(d["FETCH_SIZE"] for d in fetch.values())
        w_kib = _mean(d["WRITE_SIZE"] for d in write.values())
        rd = f_kib * 1024 * f_scale
        wr = w_kib * 1024 * w_scale
        L += ["copy_kernel_bytes_each_way: %d" % COPY_BYTES,
              "copy_fetch_size_kib: %.1f" % f_copy, "copy_write_size_kib: %.1f" % w_copy,
              "fetch_scale: %.4f" % f_scale, "write_scale: %.4f" % w_scale,
              "kernel_fetch_size_kib: %.1f" % f_kib, "kernel_write_size_kib: %.1f" % w_kib,
              "beyond_l2_read_bytes_per_launch: %.0f (FETCH_SIZE x fetch_scale)" % rd,
              "beyond_l2_write_bytes_per_launch: %.0f (WRITE_SIZE x write_scale)" % wr,
              "beyond_l2_bytes_per_launch: %.0f" % (rd + wr),
              "compulsory_bytes: %d" % compulsory,
              "beyond_l2_over_compulsory: %.3f" % ((rd + wr) / compulsory)]
    if all(k in val for k in ("TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum",
                              "TCC_EA0_RDREQ_128B_sum")):
        by_size = (32 * val["TCC_EA0_RDREQ_32B_sum"] + 64 * val["TCC_EA0_RDREQ_64B_sum"] +
                   128 * val["TCC_EA0_RDREQ_128B_sum"])
        L.append("beyond_l2_read_bytes_by_request_size: %.0f (32 x RDREQ_32B + 64 x RDREQ_64B + "
                 "128 x RDREQ_128B)" % by_size)
        if fetch:
            L.append("fetch_scale_check: %.4f (read bytes by request size / FETCH_SIZE x "
                     "fetch_scale)" % (by_size / rd))
        if "TCC_EA0_RDREQ_sum" in val:
            n = (val["TCC_EA0_RDREQ_32B_sum"] + val["TCC_EA0_RDREQ_64B_sum"] +
                 val["TCC_EA0_RDREQ_128B_sum"])
            L.append("read_requests_by_size_over_all: %.4f" % (n / max(val["TCC_EA0_RDREQ_sum"], 1)))
    if "TCC_EA0_RDREQ_DRAM_sum" in val and "TCC_EA0_RDREQ_sum" in val:
        L.append("read_requests_to_dram_share: %.4f (TCC_EA0_RDREQ_DRAM / TCC_EA0_RDREQ)"
                 % (val["TCC_EA0_RDREQ_DRAM_sum"] / max(val["TCC_EA0_RDREQ_sum"], 1)))

    # --------------------------------------------------- closed forms, models
    if conv:
        P, Q = w.out_hw
        n_split, full = 1, 0
        if path == "splitk":
            cfg, n_split, _, full = sg.conv2d_splitk_plan(w.N, w.H, w.W, w.C, w.K, w.R, w.S,
                                                          w.pad, w.stride, w.dil, splits, config)
        else:
            cfg = config if config is not None else sg.conv2d_select_config(
                w.N, w.H, w.W, w.C, w.K, w.R, w.S, w.pad, w.stride, w.dil)
        info = sg.config_info(cfg)
        # Chunks of whole BK slices: a split tile does the slices of a whole one.
        want = model.mfma_instructions(w.N * P * Q, w.K, w.R * w.S * w.C, info["bm"], info["bn"],
                                       info["bk"], 32, 1)
        L.append("mfma_instructions_closed_form: %d (tile %s)" % (want, info["name"]))
        if n_split > 1:
            tiles = model.ceil_div(w.N * P * Q, info["bm"]) * model.ceil_div(w.K, info["bn"])
            part = (tiles - full) * n_split * info["bm"] * info["bn"] * 4
            L.append("splitk_chunks: %d" % n_split)
            L.append("splitk_full_tiles: %d of %d (all of R*S*C, no join)" % (full, tiles))
            L.append("splitk_partial_bytes_model: %d (split tiles x chunks x BM x BN x 4, "
                     "written once and read once by the join)" % part)
    if attn:
        # Each of the 8 waves issues 2 D v_mfma_f32_32x32x2_f32 per visited
        # (256-query, 64-key) block pair: D for the scores, D for P V.
        import math
        qb = math.ceil(w.Sq / 256)
        nkv = math.ceil(w.Skv / 64)
        pairs = sum(min(nkv, (min(w.Sq, 256 * b + 256) - 1) // 64 + 1) if w.causal else nkv
                    for b in range(qb))
        L.append("mfma_instructions_closed_form: %d (attention, 256 x 64 blocks)"
                 % (w.BH * pairs * 8 * 2 * w.D))
    if general:
        # The general form's tile; its A and B panels are the plain product's
        # (only their stored orientation differs), and with beta != 0 each
        # XCD also reads its tiles' part of C once.  Split (path splitk):
        # chunk b of every tile runs as batch member b over K / chunks, and
        # the join writes and reads the partial tiles once.
        n_split = 1
        if path == "splitk":
            cfg, n_split, _ = sg.ex_splitk_plan(w.M, w.N, w.K, bool(w.transA), bool(w.transB),
                                                splits)
        else:
            cfg = sg.select_general_config(w.M, w.N, w.K)
        info = sg.config_info(cfg)
        mi = 16 if info["name"].startswith("dl16") else 32
        L.append("mfma_instructions_closed_form: %d (tile %s)" % (
            model.mfma_instructions(w.M, w.N, w.K, info["bm"], info["bn"], info["bk"], mi, 1),
            info["name"]))
        resident = 32 * sg.workgroups_per_cu(cfg)
        panels = model.per_xcd_operand_bytes(w.M, w.N, model.ceil_div(w.K, n_split), info["bm"],
                                             info["bn"], n_split, resident=resident)
        c_read = 4 * w.M * w.N if w.beta != 0 else 0
        L.append("per_xcd_panel_read_bytes_model: %d (each XCD's L2 fetches the A and B panels "
                 "of each round of %d resident tiles once)" % (panels, resident))
        L.append("c_read_bytes: %d (beta != 0: C read once)" % c_read)
        part = 0
        if n_split > 1:
            tiles = model.ceil_div(w.M, info["bm"]) * model.ceil_div(w.N, info["bn"])
            full = sg.ex_splitk_plan_full_tiles(w.M, w.N, w.K, bool(w.transA), bool(w.transB),
                                                splits)
            part = (tiles - full) * n_split * info["bm"] * info["bn"] * 4
            L.append("splitk_chunks: %d" % n_split)
            L.append("splitk_full_tiles: %d of %d (all of K, no join)" % (full, tiles))
            L.append("splitk_partial_bytes_model: %d (split tiles x chunks x BM x BN x 4, "
                     "written once and read once by the join)" % part)
        if fetch:
            L.append("beyond_l2_read_over_panel_model_plus_c: %.4f" % (rd / (panels + c_read)))
            if part:
                L.append("beyond_l2_read_minus_panels_and_c_over_partials: %.4f ((read bytes - "
                         "panel model - C) / partial bytes)" % ((rd - panels - c_read) / part))
        if fetch and write and part:
            L.append("beyond_l2_write_minus_output_over_partials: %.4f ((write bytes - 4MN) "
                     "/ partial bytes)" % ((wr - 4.0 * w.M * w.N) / part))
    if path in ("mfma", "splitk") and gemm:
        n_split = 1
        if path == "splitk":
            cfg, n_split, _ = sg.splitk_plan(w.M, w.N, w.K, splits)
        else:
            cfg = sg.select_config(w.M, w.N, w.K, w.batch) if config is None else config
        info = sg.config_info(cfg)
        mi = 16 if info["name"].startswith("dl16") or info["name"].startswith("mfma16") else 32
        want = model.mfma_instructions(w.M, w.N, w.K, info["bm"], info["bn"], info["bk"], mi,
                                       w.batch)
        L.append("mfma_instructions_closed_form: %d (tile %s)" % (want, info["name"]))
        staged = model.global_to_shared_loads(w.M, w.N, w.K, info["bm"], info["bn"],
                                              info["bk"], padded=True) * w.batch
        L.append("global_to_lds_values_model: %d" % staged)
        # one 64-lane dwordx4 instruction moves 256 values
        L.append("global_dwordx4_wave_instructions_closed_form: %d" % (staged // 256))
        if "TCP_TCC_READ_REQ_sum" in val:
            # L1 -> L2 read requests, taken as one 128-byte line each
            req = val["TCP_TCC_READ_REQ_sum"]
            L.append("l2_read_request_bytes_at_128B: %.0f (%.4f x the global-to-LDS model)"
                     % (req * 128, req * 128 / (4.0 * staged)))
            nreq = model.l2_read_requests(w.M, w.N, w.K, info["bm"], info["bn"], info["bk"],
                                          w.batch, w.lda, w.ldb)
            what = "per tile and slice, the 128-byte lines each valid row piece of A and B touches"
            if n_split > 1:
                # the join reads every split tile's partials once, in whole lines
                tiles = model.ceil_div(w.M, info["bm"]) * model.ceil_div(w.N, info["bn"])
                full = sg.splitk_plan_full_tiles(w.M, w.N, w.K, splits)
                nreq += (tiles - full) * n_split * info["bm"] * info["bn"] * 4 // 128
                what += ", plus the join's reads of the partial tiles"
            L.append("l2_read_requests_model: %d (%s)" % (nreq, what))
            L.append("l2_read_requests_over_model: %.4f" % (req / nreq))
        resident = 32 * sg.workgroups_per_cu(cfg)
        # Split-K: chunk b of every tile runs as batch member b over K / chunks.
        panels = model.per_xcd_operand_bytes(w.M, w.N, model.ceil_div(w.K, n_split), info["bm"],
                                             info["bn"], w.batch * n_split, resident=resident)
        L.append("per_xcd_panel_read_bytes_model: %d (each XCD's L2 fetches the A and B panels "
                 "of each round of %d resident tiles once)" % (panels, resident))
        if fetch:
            L.append("beyond_l2_read_over_panel_model: %.4f" % (rd / panels))
        if n_split > 1:
            tiles = model.ceil_div(w.M, info["bm"]) * model.ceil_div(w.N, info["bn"])
            full = sg.splitk_plan_full_tiles(w.M, w.N, w.K, splits)
            part = (tiles - full) * n_split * info["bm"] * info["bn"] * 4
            L.append("splitk_chunks: %d" % n_split)
            L.append("splitk_full_tiles: %d of %d (all of K, no join)" % (full, tiles))
            L.append("splitk_partial_bytes_model: %d (split tiles x chunks x BM x BN x 4, "
                     "written once and read once by the join)" % part)
            if fetch and write:
                L.append("beyond_l2_write_minus_output_over_partials: %.4f ((write bytes - 4MN) "
                         "/ partial bytes)" % ((wr - 4.0 * w.M * w.N) / part))
                L.append("beyond_l2_read_minus_panels_over_partials: %.4f ((read bytes - panel "
                         "model) / partial bytes)" % ((rd - panels) / part))
    if path == "valu" and "SQ_INSTS_VALU_FMA_F32" in val:
        L.append("valu_fma_instructions_closed_form: %d" % model.valu_fma_instructions(
            w.M, w.N, w.K, batch=w.batch))
    if "SQ_WAIT_ANY" in val and "SQ_WAVE_CYCLES" in val:
        L.append("wave_cycles_waiting_fraction: %.4f"
                 % (val["SQ_WAIT_ANY"] / val["SQ_WAVE_CYCLES"]))
    if "SQ_LDS_BANK_CONFLICT" in val and "SQ_LDS_IDX_ACTIVE" in val:
        c = val["SQ_LDS_BANK_CONFLICT"]
        a = val["SQ_LDS_IDX_ACTIVE"]
        L.append("lds_bank_conflicts_per_access: %.4f" % (c / max(1.0, a - c)))
    open(out, "w").write("\n".join(L) + "\n")


def cpu_baseline(w, A, B, target_s: float = 12.0, keep=None):
    """The oracle, untouched, on the leading rows of C of the same workload.
    With a dict `keep`, the rows' reference values and magnitude sums are
    left in it (for the parity check beside the timing)."""
    import oracle
    a = A.numpy()
    b = B.numpy()
    rows0 = 16
    t0 = time.perf_counter()
    _, _, used = oracle.sgemm_f64(rows0, w.N, w.K, a, w.lda, b, w.ldb)
    dt0 = time.perf_counter() - t0
    rows = int(min(w.M, max(rows0, rows0 * target_s / max(dt0, 1e-6))))
    t0 = time.perf_counter()
    ref, mag, used = oracle.sgemm_f64(rows, w.N, w.K, a, w.lda, b, w.ldb)
    dt = time.perf_counter() - t0
    if keep is not None:
        keep.update(rows=rows, ref=ref, mag=mag)
    flops = 2.0 * rows * w.N * w.K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(used), "kind": "oracle",
            "sample": "rows 0..%d of C for %s (%dx%dx%d, %.3g GFLOP) in %.2f s, FP64 "
                      "accumulation, OpenMP over rows" % (rows - 1, w.name, rows, w.N, w.K,
                                                          flops / 1e9, dt),
            "seconds": dt}


def gemm_parity(C_rows, keep, rel_tol: float = 2e-4):
    """The timed kernel's output rows against the oracle's: the largest
    |C - C_ref| / sum_k |A||B| (the acceptance bound is 2e-4)."""
    import numpy as np
    got = np.asarray(C_rows, dtype=np.float64)
    ref, mag = keep["ref"], keep["mag"]
    err = np.abs(got - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(mag > 0, err / mag, np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max())
    return {"rows_checked": int(keep["rows"]), "max_err_over_abs_products": worst,
            "bound": rel_tol, "within_bound": bool(worst <= rel_tol),
            "bitwise_equal_to_rounded_oracle": bool(np.array_equal(
                got.astype(np.float32).view(np.uint32),
                ref.astype(np.float32).view(np.uint32)))}


def host_info():
    import torch
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "torch": torch.__version__, "hip": torch.version.hip}


def window_cpu_baseline(w, x_cpu):
    """The oracle, untouched, over the whole window workload (one pass)."""
    import oracle
    x = x_cpu.numpy()
    t0 = time.perf_counter()
    oracle.window_sum_f64(w.n, w.W, x)
    dt = time.perf_counter() - t0
    return {"value": w.bytes / dt / 1e9, "unit": "GB/s", "cores": int(oracle.max_threads()),
            "kind": "oracle",
            "sample": "the whole workload (%d outputs, W = %d) in %.2f s, FP64 sums, OpenMP "
                      "over outputs" % (w.n, w.W, dt),
            "seconds": dt}


def bench_window(args) -> int:
    """Sliding window sums: algorithmic bytes (inputs once, outputs once) per
    second, against the HBM roofline."""
    import torch
    from workloads import WINDOW_WORKLOADS, window_input
    import tiled_fp32_gemm_sgemm_amd as sg

    w = WINDOW_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x_cpu = window_input(w)
    x = x_cpu.to(dev)
    y = torch.empty(w.n, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream

    def step():
        st = sg.window_sum_raw(w.n, w.W, x.data_ptr(), y.data_ptr(), handle)
        if st != 0:
            raise sg.SgemmError(st, "window_sum")

    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def timed(fn, n_steps, n_warm):
        for _ in range(n_warm):
            fn()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(n_steps):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n_steps

    ms = timed(step, args.steps, args.warmup)
    gbs = w.bytes / (ms * 1e-3) / 1e9
    comparators = {}
    if not args.no_comparator:
        # A plain device copy of the same bytes (n floats read, n written).
        dst = torch.empty_like(y)
        cms = timed(lambda: dst.copy_(x[:w.n]), max(5, args.steps // 2), 3)
        comparators["copy"] = {"GB/s": 8.0 * w.n / (cms * 1e-3) / 1e9, "ms_per_step": cms}
        del dst
    traffic = (read_traffic(WINDOW_TRAFFIC_FILE, WINDOW_SOURCES)
               if args.workload == "window5" else None)
    out = {
        "metric": "sliding window sum GB/s (inputs read once, outputs written once)",
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.describe(), "n": w.n, "W": w.W},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "window_sum_kernel", "event_ms_per_launch": ms},
        "cpu_baseline": None if args.no_cpu_baseline else window_cpu_baseline(w, x_cpu),
        "comparators": comparators,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(out), flush=True)
    return 0


def conv_cpu_baseline(w, x_cpu, wt_cpu, target_s: float = 10.0):
    """The oracle, untouched, on the first images of the convolution workload
    (the same layer at a smaller batch)."""
    import oracle
    x = x_cpu.numpy()
    wt = wt_cpu.numpy()
    P, Q = w.out_hw
    per_image = 2.0 * P * Q * w.K * w.R * w.S * w.C
    n0 = 1
    t0 = time.perf_counter()
    oracle.conv2d_nhwc_f64(x, wt, n0, w.H, w.W, w.C, w.K, w.R, w.S, w.pad, w.stride, w.dil)
    dt0 = time.perf_counter() - t0
    n = int(min(w.N, max(n0, n0 * target_s / max(dt0, 1e-6))))
    t0 = time.perf_counter()
    oracle.conv2d_nhwc_f64(x, wt, n, w.H, w.W, w.C, w.K, w.R, w.S, w.pad, w.stride, w.dil)
    dt = time.perf_counter() - t0
    return {"value": per_image * n / dt / 1e12, "unit": "TFLOP/s",
            "cores": int(oracle.max_threads()), "kind": "oracle",
            "sample": "images 0..%d of %s (%.3g GFLOP) in %.2f s, FP64 accumulation, OpenMP "
                      "over outputs" % (n - 1, w.name, per_image * n / 1e9, dt),
            "seconds": dt}


def bench_conv(args) -> int:
    """2-D convolution (implicit GEMM): TFLOP/s of the definition's
    multiply-adds against the FP32 matrix peak."""
    import torch
    from workloads import CONV_WORKLOADS, conv_operands
    import tiled_fp32_gemm_sgemm_amd as sg

    w = CONV_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x_cpu, wt_cpu = conv_operands(w)
    x = x_cpu.to(dev).view(w.N, w.H, w.W, w.C)
    wt = wt_cpu.to(dev).view(w.K, w.R, w.S, w.C)
    P, Q = sg.conv2d_output_size(w.H, w.W, w.R, w.S, w.pad, w.stride, w.dil)
    y = torch.empty((w.N, P, Q, w.K), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream
    splitk = args.path == "splitk"
    if splitk:
        # conv2d_nhwc_splitk: the reduction split over workgroups (the time
        # model's plan at --splits 0), joined through a workspace zeroed once.
        cfg, n_split, ws_bytes, full_tiles = sg.conv2d_splitk_plan(
            w.N, w.H, w.W, w.C, w.K, w.R, w.S, w.pad, w.stride, w.dil, args.splits, args.config)
        ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

        def step():
            st = sg.conv2d_nhwc_splitk_raw(w.N, w.H, w.W, w.C, w.K, w.R, w.S, x.data_ptr(),
                                           wt.data_ptr(), y.data_ptr(), ws.data_ptr(),
                                           ws.numel(), w.pad, w.stride, w.dil, args.splits,
                                           handle, args.config)
            if st != 0:
                raise sg.SgemmError(st, "conv2d_nhwc_splitk")
    else:
        cfg = args.config if args.config is not None else sg.conv2d_select_config(
            w.N, w.H, w.W, w.C, w.K, w.R, w.S, w.pad, w.stride, w.dil)

        def step():
            st = sg.conv2d_nhwc_raw(w.N, w.H, w.W, w.C, w.K, w.R, w.S, x.data_ptr(),
                                    wt.data_ptr(), y.data_ptr(), w.pad, w.stride, w.dil, handle,
                                    args.config)
            if st != 0:
                raise sg.SgemmError(st, "conv2d_nhwc")

    def timed(fn, n_steps, n_warm):
        for _ in range(n_warm):
            fn()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(n_steps):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n_steps

    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    ms = timed(step, args.steps, args.warmup)
    tflops = w.flops / (ms * 1e-3) / 1e12
    tile = sg.config_info(cfg)["name"]
    comparators = {}
    if not args.no_comparator:
        # MIOpen through torch, FP32, on the same NHWC memory (channels_last).
        torch.backends.cudnn.allow_tf32 = False
        xt = x.permute(0, 3, 1, 2)
        wtt = wt.permute(0, 3, 1, 2)
        tms = timed(lambda: torch.nn.functional.conv2d(xt, wtt, stride=w.stride, padding=w.pad,
                                                       dilation=w.dil),
                    max(5, args.steps // 2), 3)
        comparators["torch_conv2d_channels_last"] = {
            "tflops": w.flops / (tms * 1e-3) / 1e12, "ms_per_step": tms}
    conf = {"workload": w.describe(), "N": w.N, "H": w.H, "W": w.W, "C": w.C, "K": w.K,
            "R": w.R, "S": w.S, "tile": tile,
            "entry": "conv2d_nhwc_splitk" if splitk else "conv2d_nhwc"}
    if splitk:
        conf["splitk"] = {"chunks": n_split, "full_tiles": full_tiles,
                          "workspace_bytes": ws_bytes}
    out = {
        "metric": "FP32 2-D convolution TFLOP/s (implicit GEMM, NHWC)",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_of_fp32_peak": 100.0 * tflops / PEAK_FP32_TFLOPS,
        # value counts every multiply-add of the implicit product (dense
        # equivalent); the useful rate leaves out the taps on the zero padding
        "useful_tflops": w.useful_flops / (ms * 1e-3) / 1e12,
        "useful_flop_share": w.useful_flops / w.flops,
        "config": conf,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / PEAK_FP32_TFLOPS,
                     "traffic": read_traffic(conv_traffic_file(args.path, args.workload),
                                             GEMM_SOURCES, tile,
                                             n_split if splitk else None),
                     "kernel": tile, "event_ms_per_launch": ms},
        "cpu_baseline": None if args.no_cpu_baseline else conv_cpu_baseline(w, x_cpu, wt_cpu),
        "comparators": comparators,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(out), flush=True)
    return 0


def attn_cpu_baseline(w, q, k, v, scale, target_s: float = 10.0):
    """The oracle, untouched, on the first query rows of head 0 (then of the
    following heads) of the attention workload."""
    import numpy as np
    import oracle
    qn, kn, vn = q.numpy(), k.numpy(), v.numpy()

    def rows_flops(n):
        rows = np.arange(n, dtype=np.int64)
        pairs = sum(min(int(r % w.Sq) + 1, w.Skv) if w.causal else w.Skv for r in rows)
        return rows, 4.0 * pairs * w.D

    n0 = 64
    rows, _ = rows_flops(n0)
    t0 = time.perf_counter()
    oracle.attention_rows_f64(qn, kn, vn, w.BH, w.Sq, w.Skv, w.D, scale, rows, w.causal)
    dt0 = time.perf_counter() - t0
    n = int(min(w.BH * w.Sq, max(n0, n0 * target_s / max(dt0, 1e-6))))
    rows, flops = rows_flops(n)
    t0 = time.perf_counter()
    oracle.attention_rows_f64(qn, kn, vn, w.BH, w.Sq, w.Skv, w.D, scale, rows, w.causal)
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(oracle.max_threads()),
            "kind": "oracle",
            "sample": "query rows 0..%d (head-major) of %s (%.3g GFLOP) in %.2f s, FP64, OpenMP "
                      "over rows" % (n - 1, w.name, flops / 1e9, dt),
            "seconds": dt}


def bench_attention(args) -> int:
    """Blockwise attention: TFLOP/s of the two products over the allowed
    query/key pairs, against the FP32 matrix peak."""
    import math
    import torch
    from workloads import ATTN_WORKLOADS, attn_operands
    import tiled_fp32_gemm_sgemm_amd as sg

    w = ATTN_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q_cpu, k_cpu, v_cpu = attn_operands(w)
    q = q_cpu.to(dev).view(w.BH, w.Sq, w.D)
    k = k_cpu.to(dev).view(w.BH, w.Skv, w.D)
    v = v_cpu.to(dev).view(w.BH, w.Skv, w.D)
    o = torch.empty_like(q)
    scale = float(torch.tensor(1.0 / math.sqrt(w.D), dtype=torch.float32))
    stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream

    def step():
        st = sg.attention_raw(w.BH, w.Sq, w.Skv, w.D, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              o.data_ptr(), scale, w.causal, handle)
        if st != 0:
            raise sg.SgemmError(st, "attention_fwd")

    def timed(fn, n_steps, n_warm):
        for _ in range(n_warm):
            fn()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(n_steps):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n_steps

    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    ms = timed(step, args.steps, args.warmup)
    tflops = w.flops / (ms * 1e-3) / 1e12
    comparators = {}
    if not args.no_comparator:
        q4, k4, v4 = (t.unsqueeze(0) for t in (q, k, v))
        tms = timed(lambda: torch.nn.functional.scaled_dot_product_attention(
            q4, k4, v4, is_causal=w.causal, scale=scale), max(3, args.steps // 5), 2)
        comparators["torch_sdpa_fp32"] = {"tflops": w.flops / (tms * 1e-3) / 1e12,
                                          "ms_per_step": tms}
    kernel = "attention_d%d%s" % (w.D, "_causal" if w.causal else "")
    out = {
        "metric": "FP32 blockwise attention TFLOP/s (4 D flops per allowed query/key pair)",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_of_fp32_peak": 100.0 * tflops / PEAK_FP32_TFLOPS,
        "config": {"workload": w.describe(), "BH": w.BH, "Sq": w.Sq, "Skv": w.Skv, "D": w.D,
                   "causal": w.causal},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / PEAK_FP32_TFLOPS,
                     "traffic": (read_traffic(ATTN_TRAFFIC_FILE, ATTN_SOURCES)
                                 if args.workload == "attn_s2048_d128" else None),
                     "kernel": kernel, "event_ms_per_launch": ms},
        "cpu_baseline": (None if args.no_cpu_baseline
                         else attn_cpu_baseline(w, q_cpu, k_cpu, v_cpu, scale)),
        "comparators": comparators,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(out), flush=True)
    return 0


def general_cpu_baseline(w, A, B, C0, target_s: float = 12.0, keep=None):
    """The oracle's general form, untouched, on the leading rows of C (for A
    stored K x M the first rows of C use the first columns of A)."""
    import oracle
    a, b, c = A.numpy(), B.numpy(), C0.numpy()

    def rows_of_c(rows):
        return oracle.sgemm_ex_f64(bool(w.transA), bool(w.transB), rows, w.N, w.K, w.alpha, a,
                                   w.lda, b, w.ldb, w.beta, c, w.ldc)

    rows0 = 16
    t0 = time.perf_counter()
    rows_of_c(rows0)
    dt0 = time.perf_counter() - t0
    rows = int(min(w.M, max(rows0, rows0 * target_s / max(dt0, 1e-6))))
    t0 = time.perf_counter()
    ref, mag, used = rows_of_c(rows)
    dt = time.perf_counter() - t0
    if keep is not None:
        keep.update(rows=rows, ref=ref, mag=mag)
    flops = 2.0 * rows * w.N * w.K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(used), "kind": "oracle",
            "sample": "rows 0..%d of C for %s (%dx%dx%d, %.3g GFLOP) in %.2f s, FP64 "
                      "accumulation, OpenMP over rows" % (rows - 1, w.name, rows, w.N, w.K,
                                                          flops / 1e9, dt),
            "seconds": dt}


def bench_general(args) -> int:
    """The general form C = alpha op(A) op(B) + beta C (sgemm_ex): TFLOP/s
    of the 2MNK product against the FP32 matrix peak; C is read and written."""
    import torch
    from workloads import GENERAL_WORKLOADS, general_operands
    import tiled_fp32_gemm_sgemm_amd as sg

    if args.path not in ("mfma", "splitk") or args.graph or args.cold or args.config is not None:
        print("the general-form workloads time sgemm_ex (--path mfma) or sgemm_ex_splitk (--path "
              "splitk) with their own tile choice, launched on a stream", file=sys.stderr)
        return 2
    splitk = args.path == "splitk"
    w = GENERAL_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    A_cpu, B_cpu, C0_cpu = general_operands(w, pad=0.0)
    A, B, C0 = A_cpu.to(dev), B_cpu.to(dev), C0_cpu.to(dev)
    C = C0.clone()
    stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream

    if splitk:
        sk_config, sk_splits, sk_bytes = sg.ex_splitk_plan(w.M, w.N, w.K, bool(w.transA),
                                                           bool(w.transB), args.splits)
        ws = torch.zeros(max(sk_bytes, 256), dtype=torch.uint8, device=dev)

    def step():
        if splitk:
            st = sg.sgemm_ex_splitk_raw(w.transA, w.transB, w.M, w.N, w.K, w.alpha, A.data_ptr(),
                                        w.lda, B.data_ptr(), w.ldb, w.beta, C.data_ptr(), w.ldc,
                                        ws.data_ptr(), ws.numel(), handle, args.splits)
        else:
            st = sg.sgemm_ex_raw(w.transA, w.transB, w.M, w.N, w.K, w.alpha, A.data_ptr(),
                                 w.lda, B.data_ptr(), w.ldb, w.beta, C.data_ptr(), w.ldc, handle)
        if st != 0:
            raise sg.SgemmError(st, "sgemm_ex_splitk" if splitk else "sgemm_ex")

    # op(A), op(B) and C as torch views for hipBLASLt's addmm beside it.
    ra, ca = (w.K, w.M) if w.transA else (w.M, w.K)
    rb, cb = (w.N, w.K) if w.transB else (w.K, w.N)
    opA = A.as_strided((ra, ca), (w.lda, 1))
    opA = opA.t() if w.transA else opA
    opB = B.as_strided((rb, cb), (w.ldb, 1))
    opB = opB.t() if w.transB else opB
    C2 = C0.clone().as_strided((w.M, w.N), (w.ldc, 1))

    def torch_step():
        C2.addmm_(opA, opB, beta=w.beta, alpha=w.alpha)

    def timed(fn, n_steps, n_warm):
        for _ in range(n_warm):
            fn()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(n_steps):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n_steps

    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # Clock settle, then warm-up and timed counts from the time of one step,
    # as for the plain product.
    t0 = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
        n_settle += 4
    settle = {"launches": n_settle, "seconds": round(time.perf_counter() - t0, 4)}
    t0 = time.perf_counter()
    for _ in range(5):
        step()
    torch.cuda.synchronize()
    n = max(1, int(GEMM_WORK_S / max((time.perf_counter() - t0) / 5, 1e-6)))
    args.warmup = args.warmup if args.warmup is not None else max(30, n)
    args.steps = args.steps if args.steps is not None else max(50, n)
    ms = timed(step, args.steps, args.warmup)
    pairs = []
    for _ in range(min(args.steps, 50)):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    single = sorted(e0.elapsed_time(e1) for e0, e1 in pairs)
    flops = float(w.flops)
    tflops = flops / (ms * 1e-3) / 1e12
    if splitk:
        tile = "%s_splits%d" % (sg.config_info(sk_config)["name"], sk_splits)
        traffic = read_traffic(gemm_traffic_file("ex_splitk", w.name), GEMM_SOURCES,
                               sg.config_info(sk_config)["name"], sk_splits)
    else:
        tile = sg.config_info(sg.select_general_config(w.M, w.N, w.K))["name"]
        traffic = read_traffic(gemm_traffic_file("ex", w.name), GEMM_SOURCES, tile)

    comparators = {}
    if not args.no_comparator and splitk:
        def plain_step():
            st = sg.sgemm_ex_raw(w.transA, w.transB, w.M, w.N, w.K, w.alpha, A.data_ptr(), w.lda,
                                 B.data_ptr(), w.ldb, w.beta, C.data_ptr(), w.ldc, handle)
            if st != 0:
                raise sg.SgemmError(st, "sgemm_ex")
        pms = timed(plain_step, max(5, args.steps // 2), 3)
        comparators["sgemm_ex"] = {"tflops": flops / (pms * 1e-3) / 1e12, "ms_per_step": pms,
                                   "note": "the unsplit general form, same timing"}
    if not args.no_comparator:
        tms = timed(torch_step, max(5, args.steps // 2), 3)
        comparators["torch_addmm"] = {"tflops": flops / (tms * 1e-3) / 1e12, "ms_per_step": tms,
                                      "note": "torch addmm_ (hipBLASLt) with the same layouts "
                                              "and scalars, same timing"}
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        keep = {}
        cpu = general_cpu_baseline(w, A_cpu, B_cpu, C0_cpu, keep=keep)
        # One launch from the initial C (the timed launches kept updating it).
        C.copy_(C0)
        step()
        torch.cuda.synchronize()
        rows = keep["rows"]
        C_rows = C[:rows * w.ldc].view(rows, w.ldc)[:, :w.N].cpu().numpy()
        parity = gemm_parity(C_rows, keep)
    out = {
        "metric": "FP32 GEMM, general form C = alpha op(A) op(B) + beta C, TFLOP/s at M=%d N=%d "
                  "K=%d on 1 MI355X; %% of FP32 peak" % (w.M, w.N, w.K),
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_of_fp32_peak": 100.0 * tflops / PEAK_FP32_TFLOPS,
        "cache": "warm",
        "clock_settle": settle,
        "launch": "stream",
        "single_launch": {"n": len(single), "median_ms": single[len(single) // 2],
                          "min_ms": single[0],
                          "median_tflops": flops / (single[len(single) // 2] * 1e-3) / 1e12,
                          "max_tflops": flops / (single[0] * 1e-3) / 1e12},
        "config": {"workload": w.describe(), "M": w.M, "N": w.N, "K": w.K,
                   "transA": w.transA, "transB": w.transB, "alpha": w.alpha, "beta": w.beta,
                   "path": args.path, "tile": tile},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / PEAK_FP32_TFLOPS,
                     "traffic": traffic, "kernel": tile, "event_ms_per_launch": ms},
        "cpu_baseline": cpu,
        "parity": parity,
        "comparators": comparators,
        "device": torch.cuda.get_device_name(dev),
        "host": host_info(),
    }
    print(json.dumps(out), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: GEMMs as many as fill 0.1 s, at least 50; "
                         "200 for the window and convolution; 50 for attention)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: GEMMs as many as fill 0.1 s, at least "
                         "30, so clocks have settled; 200 for the window and convolution; 30 "
                         "for attention)")
    ap.add_argument("--path", choices=["mfma", "valu", "splitk", "window"], default="mfma",
                    help="GEMM path: the matrix-core product (sgemm), the vector-ALU comparator, "
                         "or the split-K entry point at --splits; for a convolution workload, "
                         "conv2d_nhwc (mfma) or conv2d_nhwc_splitk (splitk) (window: counter "
                         "summaries of the window kernel only)")
    ap.add_argument("--workload", default="square4096")
    ap.add_argument("--config", type=int, default=None, help="force a matrix-core tile config")
    ap.add_argument("--splits", type=int, default=0,
                    help="split-K comparator: k chunks per output tile (0: the time model's "
                         "plan, which may be the plain kernel)")
    ap.add_argument("--graph", action="store_true",
                    help="GEMM: capture the timed launches in one HIP graph (torch.cuda.CUDAGraph) and "
                         "time its replay, so host-side launch cost drops out")
    ap.add_argument("--cold", action="store_true",
                    help="GEMM: before every timed launch, write a 512 MiB buffer (more than the "
                         "256 MB last-level cache) so the operands come from HBM; each launch is "
                         "timed by its own event pair")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-comparator", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain copy kernel of known size (counter scaling)")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                    help="write a text summary of a rocprofv3 kernel-stats csv to --out")
    ap.add_argument("--trace-csv", help="kernel_trace.csv for --summarize-trace")
    ap.add_argument("--after-timed", type=int, default=0,
                    help="dispatches of the kernel after the timed ones (--summarize-trace; a "
                         "GEMM run launches min(steps, 50) single timed launches after them)")
    ap.add_argument("--timed", type=int, default=0,
                    help="timed dispatches at the end of the trace (--summarize-trace)")
    ap.add_argument("--summarize-counters", action="store_true",
                    help="write a counter summary from --fetch-csv/--write-csv/--sq-csv to --out")
    ap.add_argument("--fetch-csv")
    ap.add_argument("--write-csv")
    ap.add_argument("--sq-csv", action="append", default=[])
    ap.add_argument("--trace-summary",
                    help="committed kernel-trace summary whose timed average is the duration "
                         "the counter summary's utilisation is taken over")
    ap.add_argument("--kernel-part", default="sgemm_mfma")
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--out")
    args = ap.parse_args(argv)

    if args.summarize_trace or args.summarize_counters:
        # The summary's own invocation, without the --command annotations
        # (they name the profiler runs and change no figure).
        import shlex
        raw = list(sys.argv[1:] if argv is None else argv)
        own = []
        i = 0
        while i < len(raw):
            if raw[i] == "--command":
                i += 2
                continue
            if not raw[i].startswith("--command="):
                own.append(raw[i])
            i += 1
        own_cmd = "python3 bench.py " + " ".join(shlex.quote(a) for a in own)
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, " ".join(args.command), args.trace_csv,
                        args.timed, own_cmd, args.after_timed)
        return 0
    if args.summarize_counters:
        summarize_counters(args.out, args.workload, args.path, args.kernel_part, args.fetch_csv,
                           args.write_csv, args.sq_csv, args.command + [own_cmd], args.config,
                           args.trace_summary, args.splits)
        return 0

    if args.gpus != 1:
        print("bench.py measures one GPU: the library runs each call on a single MI355X and "
              "has no multi-GPU path (asked for --gpus %d)" % args.gpus, file=sys.stderr)
        return 2

    from workloads import ATTN_WORKLOADS, CONV_WORKLOADS, GENERAL_WORKLOADS, WINDOW_WORKLOADS
    short = args.workload in WINDOW_WORKLOADS or args.workload in CONV_WORKLOADS
    gemm = not (short or args.workload in ATTN_WORKLOADS)
    # GEMM defaults are set from the measured time of one step (at least
    # GEMM_WORK_S of launches for each phase, and 30 / 50 launches).
    if args.steps is None and not gemm:
        args.steps = 200 if short else 50
    if args.warmup is None and not gemm:
        args.warmup = 200 if short else 30
    if args.cold and (args.workload in ATTN_WORKLOADS or args.workload in WINDOW_WORKLOADS
                      or args.workload in CONV_WORKLOADS):
        print("--cold applies to the GEMM workloads", file=sys.stderr)
        return 2
    if args.workload in ATTN_WORKLOADS:
        return bench_attention(args)
    if args.workload in GENERAL_WORKLOADS:
        return bench_general(args)
    if args.workload in WINDOW_WORKLOADS:
        return bench_window(args)
    if args.workload in CONV_WORKLOADS:
        if args.path not in ("mfma", "splitk"):
            print("a convolution runs on --path mfma (conv2d_nhwc) or splitk "
                  "(conv2d_nhwc_splitk)", file=sys.stderr)
            return 2
        return bench_conv(args)

    if args.path == "window":
        print("--path window names the window kernel in counter summaries; run "
              "--workload window5 to time it", file=sys.stderr)
        return 2

    import torch
    from workloads import WORKLOADS, workload_operands
    import tiled_fp32_gemm_sgemm_amd as sg
    from tiled_fp32_gemm_sgemm_amd import _native

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    A_cpu, B_cpu = workload_operands(w, pad=0.0)
    A = A_cpu.to(dev)
    B = B_cpu.to(dev)
    c_len = (w.batch - 1) * w.strideC + w.M * w.ldc
    C = torch.empty(c_len, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream

    if w.batch == 1:
        sk_config, sk_splits, sk_bytes = sg.splitk_plan(w.M, w.N, w.K, args.splits)
        sk_ws = torch.zeros(max(sk_bytes, 256), dtype=torch.uint8, device=dev)

    def step(path=args.path, config=args.config):
        if path == "splitk":
            st = _native.lib().sgemm_splitk(-1, w.M, w.N, w.K, A.data_ptr(), w.lda,
                                            B.data_ptr(), w.ldb, C.data_ptr(), w.ldc,
                                            args.splits, sk_ws.data_ptr(), sk_ws.numel(), handle)
            if st != 0:
                raise sg.SgemmError(st, "sgemm_splitk")
            return
        if path == "torch":
            # hipBLASLt / rocBLAS through torch on the same operands (the
            # result goes to a fresh output; C is not touched).
            if w.batch == 1:
                torch.mm(A.as_strided((w.M, w.K), (w.lda, 1)),
                         B.as_strided((w.K, w.N), (w.ldb, 1)))
            else:
                torch.bmm(A.as_strided((w.batch, w.M, w.K), (w.strideA, w.lda, 1)),
                          B.as_strided((w.batch, w.K, w.N), (w.strideB, w.ldb, 1)))
            return
        if w.batch == 1 and config is None:
            st = sg.sgemm_raw(w.M, w.N, w.K, A.data_ptr(), w.lda, B.data_ptr(), w.ldb,
                              C.data_ptr(), w.ldc, handle, path)
        else:
            st = sg.sgemm_strided_batched_raw(w.M, w.N, w.K, A.data_ptr(), w.lda, w.strideA,
                                              B.data_ptr(), w.ldb, w.strideB, C.data_ptr(),
                                              w.ldc, w.strideC, w.batch, handle, path, config)
        if st != 0:
            raise sg.SgemmError(st, "sgemm")

    def timed(n_steps, n_warm, path=args.path, config=args.config):
        for _ in range(n_warm):
            step(path, config)
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(n_steps):
            step(path, config)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n_steps  # ms per step

    if args.calibrate_copy:
        # Elementwise copy kernel: reads and writes exactly COPY_BYTES each.
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def per_launch(n_steps, cold):
        """Each launch between its own event pair (the scrub, if any, outside
        it): the spread of single-launch times."""
        scrub = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev) if cold else None
        pairs = []
        for i in range(n_steps):
            if scrub is not None:
                scrub.fill_(float(i))
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        return sorted(e0.elapsed_time(e1) for e0, e1 in pairs)

    # Time-based defaults: short launches need many more of them before the
    # clocks settle (at 30 warm-up launches a 45 us batch ran 20 % slow).
    def counts(path=args.path, config=args.config):
        for _ in range(3):
            step(path, config)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(5):
            step(path, config)
        torch.cuda.synchronize()
        est = (time.perf_counter() - t0) / 5
        n = max(1, int(GEMM_WORK_S / max(est, 1e-6)))
        warm = args.warmup if args.warmup is not None else max(30, n)
        steps = args.steps if args.steps is not None else max(50, n)
        return warm, steps

    def graph_timed(n_steps, n_warm):
        """The n_steps launches captured once and replayed: GPU time per
        launch without the host's launch cost."""
        for _ in range(n_warm):
            step()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gh = torch.cuda.current_stream().cuda_stream
            for _ in range(n_steps):
                if w.batch == 1:
                    st = sg.sgemm_raw(w.M, w.N, w.K, A.data_ptr(), w.lda, B.data_ptr(), w.ldb,
                                      C.data_ptr(), w.ldc, gh, args.path)
                else:
                    st = sg.sgemm_strided_batched_raw(w.M, w.N, w.K, A.data_ptr(), w.lda,
                                                      w.strideA, B.data_ptr(), w.ldb, w.strideB,
                                                      C.data_ptr(), w.ldc, w.strideC, w.batch, gh,
                                                      args.path, args.config)
                if st != 0:
                    raise sg.SgemmError(st, "sgemm (graph capture)")
        g.replay()  # first replay uploads the graph
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n_steps

    if args.path == "splitk" and (args.graph or w.batch != 1):
        print("--path splitk times single products, launched on a stream", file=sys.stderr)
        return 2
    # Clock settle: the workload's own launches, back to back, for
    # SETTLE_S before the warm-up steps.  After an idle spell (loading the
    # operands, the oracle) the first ~25 ms of launches run 10-20 % slow
    # while the clock ramps up; the timed steps measure the settled clock.
    t0 = time.perf_counter()
    n_settle = 0
    batch = 4
    while time.perf_counter() - t0 < SETTLE_S:
        tb = time.perf_counter()
        for _ in range(batch):
            step()
        torch.cuda.synchronize()
        n_settle += batch
        # about 10 ms of launches between synchronisations
        batch = max(4, min(4096, int(0.01 * batch / max(time.perf_counter() - tb, 1e-6))))
    settle = {"launches": n_settle, "seconds": round(time.perf_counter() - t0, 4)}
    args.warmup, args.steps = counts()
    if args.graph and args.cold:
        print("--graph and --cold exclude each other", file=sys.stderr)
        return 2
    if args.graph:
        ms = graph_timed(args.steps, args.warmup)
        single = per_launch(min(args.steps, 50), False)
    elif args.cold:
        for _ in range(args.warmup):
            step()
        single = per_launch(args.steps, True)
        ms = sum(single) / len(single)
    else:
        ms = timed(args.steps, args.warmup)
        single = per_launch(min(args.steps, 50), False)
    flops = float(w.flops)
    tflops = flops / (ms * 1e-3) / 1e12

    if args.path == "splitk":
        tile = "%s_splits%d" % (sg.config_info(sk_config)["name"], sk_splits)
    elif args.config is not None:
        tile = sg.config_info(args.config)["name"]
    elif args.path == "mfma":
        tile = sg.config_info(sg.select_config(w.M, w.N, w.K, w.batch))["name"]
    else:
        tile = "valu_128x128x8_t8x8"

    # Each workload's counter summary was taken with warm caches on the tile
    # the time model chooses; it counts only for that tile (and chunk count).
    traffic = None
    if not args.cold:
        f = gemm_traffic_file(args.path, args.workload)
        if args.path == "splitk":
            traffic = read_traffic(f, GEMM_SOURCES, sg.config_info(sk_config)["name"], sk_splits)
        elif args.path == "mfma":
            traffic = read_traffic(f, GEMM_SOURCES, tile)
        else:
            traffic = read_traffic(f, GEMM_SOURCES)
    roofline = {"bound": "alu" if args.path == "valu" else "mfma",
                "achieved": tflops,
                "peak": PEAK_FP32_TFLOPS,
                "unit": "TFLOP/s",
                "frac": None,
                "traffic": traffic,
                "kernel": tile,
                "event_ms_per_launch": ms}
    roofline["frac"] = roofline["achieved"] / roofline["peak"]

    comparators = {}
    if not args.no_comparator and w.batch == 1 and args.path != "splitk":
        other = "valu" if args.path == "mfma" else "mfma"
        oms = timed(max(5, args.steps // 5), 3, other, None)
        comparators[other] = {"tflops": flops / (oms * 1e-3) / 1e12, "ms_per_step": oms}
        if args.path == "mfma" and not args.cold:
            s_warm, s_steps = counts("splitk", None)
            sms = timed(s_steps, s_warm, "splitk", None)
            comparators["splitk"] = {"tflops": flops / (sms * 1e-3) / 1e12, "ms_per_step": sms,
                                     "tile": sg.config_info(sk_config)["name"],
                                     "splits": sk_splits,
                                     "note": "sgemm_splitk (k chunks joined in the launch), "
                                             "same timing"}
    if not args.no_comparator and not args.cold:
        t_warm, t_steps = counts("torch", None)
        tms = timed(t_steps, t_warm, "torch", None)
        comparators["torch_matmul"] = {"tflops": flops / (tms * 1e-3) / 1e12, "ms_per_step": tms,
                                       "note": "torch.mm / torch.bmm (hipBLASLt) on the same "
                                               "operands, same timing"}

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        keep = {}
        cpu = cpu_baseline(w, A_cpu, B_cpu, keep=keep)
        if w.batch == 1 and not args.graph:
            # One more launch of the timed path (the comparators wrote C too).
            step()
            torch.cuda.synchronize()
            rows = keep["rows"]
            C_rows = C[:rows * w.ldc].view(rows, w.ldc)[:, :w.N].cpu().numpy()
            parity = gemm_parity(C_rows, keep)

    out = {
        "metric": gemm_metric(w),
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_of_fp32_peak": 100.0 * tflops / PEAK_FP32_TFLOPS,
        "cache": "cold" if args.cold else "warm",
        "clock_settle": settle,
        "launch": "hip_graph" if args.graph else "stream",
        "single_launch": {"n": len(single),
                          "median_ms": single[len(single) // 2],
                          "min_ms": single[0],
                          "median_tflops": flops / (single[len(single) // 2] * 1e-3) / 1e12,
                          "max_tflops": flops / (single[0] * 1e-3) / 1e12},
        "config": {"workload": w.describe(), "M": w.M, "N": w.N, "K": w.K, "batch": w.batch,
                   "path": args.path, "tile": tile},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "comparators": comparators,
        "device": torch.cuda.get_device_name(dev),
        "host": host_info(),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
