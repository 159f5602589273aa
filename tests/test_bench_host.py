"""Host-side logic of bench.py, on the CPU: argument refusals, the counter
summary it reads `traffic` from, and the rocprofv3 trace summary."""
import csv

import bench


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_window_path_is_not_a_gemm_timing(capsys):
    assert bench.main(["--path", "window", "--no-cpu-baseline"]) == 2
    assert "--workload window5" in capsys.readouterr().err


def _summary(tmp_path, source_hash, tile, hbm="123456.0"):
    p = tmp_path / "counters.txt"
    p.write_text("# counters\nkernel_source_sha256_16: %s\n"
                 "mfma_instructions_closed_form: 33554432 (tile %s)\n"
                 "beyond_l2_bytes_per_launch: %s\n" % (source_hash, tile, hbm))
    return str(p)


def test_traffic_only_for_the_same_kernel_source_and_tile(tmp_path):
    h = bench.kernel_source_hash()
    tile = "dl32_256x256x32_w2x4"
    good = _summary(tmp_path, h, tile)
    assert bench.read_traffic(good, tile=tile) == 123456.0
    assert bench.read_traffic(good, tile="dl32_128x128x32_w2x2") is None
    stale = _summary(tmp_path, "0" * 16, tile)
    assert bench.read_traffic(stale, tile=tile) is None
    assert bench.read_traffic(str(tmp_path / "missing.txt")) is None


def test_traffic_of_a_split_needs_the_same_chunk_count(tmp_path):
    h = bench.kernel_source_hash()
    tile = "dl32_64x64x128_w2x1_s2_k4"
    p = tmp_path / "counters.txt"
    p.write_text("kernel_source_sha256_16: %s\n"
                 "splitk_chunks: 4\n"
                 "mfma_instructions_closed_form: 1048576 (tile %s)\n"
                 "beyond_l2_bytes_per_launch: 59909651\n" % (h, tile))
    assert bench.read_traffic(str(p), tile=tile, chunks=4) == 59909651.0
    assert bench.read_traffic(str(p), tile=tile, chunks=8) is None


def test_every_committed_gemm_summary_is_found_by_its_workload():
    import os
    for path, workload in [("mfma", "square4096"), ("mfma", "square1024"), ("mfma", "tall"),
                           ("mfma", "ragged"), ("mfma", "shard512"), ("mfma", "batched128"),
                           ("splitk", "longk512"), ("valu", "square4096"), ("ex", "atb4096")]:
        f = bench.gemm_traffic_file(path, workload)
        assert os.path.exists(f), f
        with open(f) as fh:
            text = fh.read()
        assert "beyond_l2_bytes_per_launch:" in text and "kernel_source_sha256_16:" in text, f


def test_conv_summaries_are_named_by_entry_point():
    import os
    assert bench.conv_traffic_file("mfma", "conv3x3_c256").endswith(
        os.path.join("profiles", "conv2d_conv3x3_c256_counters.txt"))
    assert bench.conv_traffic_file("splitk", "conv3x3_c256").endswith(
        os.path.join("profiles", "conv2d_splitk_conv3x3_c256_counters.txt"))
    for path in ("mfma", "splitk"):
        f = bench.conv_traffic_file(path, "conv3x3_c256")
        assert os.path.exists(f), f
        with open(f) as fh:
            text = fh.read()
        assert "beyond_l2_bytes_per_launch:" in text and "kernel_source_sha256_16:" in text, f


def test_conv_rejects_gemm_only_paths(capsys):
    assert bench.main(["--workload", "conv3x3_c256", "--path", "valu"]) == 2
    assert "conv2d_nhwc" in capsys.readouterr().err


def test_source_hash_depends_on_every_listed_file(tmp_path, monkeypatch):
    for name in ("a.hpp", "b.hpp"):
        (tmp_path / name).write_text("int %s;\n" % name[0])
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    h0 = bench.kernel_source_hash(("a.hpp", "b.hpp"))
    (tmp_path / "b.hpp").write_text("int b2;\n")
    assert bench.kernel_source_hash(("a.hpp", "b.hpp")) != h0
    assert bench.kernel_source_hash(("b.hpp", "a.hpp")) == bench.kernel_source_hash(
        ("a.hpp", "b.hpp"))


def test_trace_summary_averages_the_timed_dispatches(tmp_path):
    stats = tmp_path / "stats.csv"
    with open(stats, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                    "MaxNs"])
        w.writerow(["gemm_kernel", 5, 5000, 1000, 100.0, 500, 1500])
    trace = tmp_path / "trace.csv"
    with open(trace, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        # two warm-up dispatches (1.5 us, 1.2 us), then three timed (0.5, 0.9, 1.0 us)
        for i, dur in enumerate([1500, 1200, 500, 900, 1000]):
            w.writerow([i + 1, "gemm_kernel", 10000 * i, 10000 * i + dur])
    out = tmp_path / "summary.txt"
    bench.summarize_trace(str(stats), str(out), "rocprofv3 ... -- python3 bench.py",
                          str(trace), timed=3)
    text = out.read_text()
    assert "# command: rocprofv3 ... -- python3 bench.py" in text
    assert "calls: 5  average_us: 1.00  min_us: 0.50  max_us: 1.50" in text
    assert "timed_average_us (last 3 dispatches): 0.80" in text


def test_cold_is_for_gemms_only(capsys):
    assert bench.main(["--workload", "window5", "--cold"]) == 2
    assert "GEMM" in capsys.readouterr().err


def test_gemm_parity_ratio():
    """The bench's parity field: largest |C - C_ref| / sum |A||B|, the bound
    check, and exact equality of the FP32-rounded oracle."""
    import numpy as np
    ref = np.array([[1.0, 2.0], [3.0, 0.0]])
    mag = np.array([[4.0, 2.0], [6.0, 0.0]])
    keep = {"rows": 2, "ref": ref, "mag": mag}
    same = bench.gemm_parity(ref.astype(np.float32), keep)
    assert same["max_err_over_abs_products"] == 0.0 and same["within_bound"]
    assert same["bitwise_equal_to_rounded_oracle"]
    off = ref.astype(np.float32).copy()
    off[1, 0] += 6.0 * 1e-3
    got = bench.gemm_parity(off, keep)
    assert abs(got["max_err_over_abs_products"] - 1e-3) < 1e-6
    assert not got["within_bound"] and not got["bitwise_equal_to_rounded_oracle"]
    # A nonzero error where the magnitude sum is zero is unbounded.
    bad = ref.astype(np.float32).copy()
    bad[1, 1] = 1e-30
    assert not bench.gemm_parity(bad, keep)["within_bound"]


def test_trace_average_and_metric_strings(tmp_path):
    from workloads import WORKLOADS
    p = tmp_path / "t.txt"
    p.write_text("kernel: k\n  calls: 9  average_us: 12.50  min_us: 1\n"
                 "  timed_average_us (100 dispatches before the last 50): 11.25\n")
    assert bench.trace_average_us(str(p)) == 11.25
    p.write_text("kernel: k\n  calls: 9  average_us: 12.50  min_us: 1\n")
    assert bench.trace_average_us(str(p)) == 12.5
    assert bench.trace_average_us(str(tmp_path / "none.txt")) is None
    assert bench.gemm_metric(WORKLOADS["square4096"]) == bench.METRIC
    assert "batch 1024 x M=128 N=128 K=128" in bench.gemm_metric(WORKLOADS["batched128"])
    assert "M=1024 N=1024 K=1024" in bench.gemm_metric(WORKLOADS["square1024"])
    assert "(1/sqrt(K))" in WORKLOADS["square4096"].describe()


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        for r in rows:
            w.writerow(r)


def test_counter_summary_derivations(tmp_path):
    """Utilisation over the trace duration at 2.4 GHz; the GRBM clock shown
    only when it is at most 2.4 GHz; beyond-L2 bytes scaled by the copy
    kernel and checked against the request sizes."""
    k = "sgemm_dev::sgemm_mfma_dl_kernel<x>"
    cp = "MulFunctor<float>"
    trace = tmp_path / "trace.txt"
    trace.write_text("kernel: %s\n  calls: 3  average_us: 20.00\n"
                     "  timed_average_us (last 3 dispatches): 20.00\n" % k)
    copy_kib = bench.COPY_BYTES / 1024.0
    _counter_csv(tmp_path / "f.csv", [(1, cp, "FETCH_SIZE", copy_kib / 2, 0, 1000),
                                      (2, k, "FETCH_SIZE", 1000.0, 0, 25000)])
    _counter_csv(tmp_path / "w.csv", [(1, cp, "WRITE_SIZE", copy_kib, 0, 1000),
                                      (2, k, "WRITE_SIZE", 4096.0, 0, 25000)])
    busy = 0.5 * 1024 * 2.4e9 * 20e-6
    # 25 us dispatch: 2.0 GHz would be 50000 cycles per XCD; 3.0 GHz 75000.
    _counter_csv(tmp_path / "s1.csv", [(2, k, "SQ_VALU_MFMA_BUSY_CYCLES", busy, 0, 25000),
                                       (2, k, "SQ_INSTS_VALU_MFMA_F32", busy / 64, 0, 25000),
                                       (2, k, "GRBM_GUI_ACTIVE", 8 * 50000, 0, 25000)])
    _counter_csv(tmp_path / "s2.csv", [(2, k, "TCC_EA0_RDREQ_32B_sum", 0, 0, 25000),
                                       (2, k, "TCC_EA0_RDREQ_64B_sum", 0, 0, 25000),
                                       (2, k, "TCC_EA0_RDREQ_128B_sum", 16000, 0, 25000),
                                       (2, k, "TCC_EA0_RDREQ_sum", 16000, 0, 25000),
                                       (2, k, "GRBM_GUI_ACTIVE", 8 * 75000, 0, 25000)])
    out = tmp_path / "c.txt"

    def summary(sq):
        bench.summarize_counters(str(out), "square1024", "mfma", "sgemm_", str(tmp_path / "f.csv"),
                                 str(tmp_path / "w.csv"), sq, ["cmd"], None, str(trace))
        return dict(l.split(": ", 1) for l in out.read_text().splitlines()
                    if ": " in l and not l.startswith("#"))

    v = summary([str(tmp_path / "s1.csv")])
    assert v["mfma_busy_fraction_at_2.4GHz"].startswith("0.5000")
    assert v["mfma_busy_cycles_per_instruction"].startswith("64.00")
    assert v["grbm_clock_ghz_counter_run"].startswith("2.000")
    assert v["beyond_l2_read_bytes_per_launch"].startswith("2048000")
    assert v["beyond_l2_write_bytes_per_launch"].startswith("4194304")
    v = summary([str(tmp_path / "s2.csv")])
    assert v["grbm_clock_ghz_counter_run"].startswith("omitted")
    assert v["fetch_scale_check"].startswith("1.0000")
    # L1 -> L2 read requests against the line model of the chosen tile
    import tiled_fp32_gemm_sgemm_amd as sg
    from tiled_fp32_gemm_sgemm_amd import model
    info = sg.config_info(sg.select_config(1024, 1024, 1024, 1))
    nreq = model.l2_read_requests(1024, 1024, 1024, info["bm"], info["bn"], info["bk"])
    _counter_csv(tmp_path / "s3.csv", [(2, k, "TCP_TCC_READ_REQ_sum", 1.5 * nreq, 0, 25000)])
    v = summary([str(tmp_path / "s3.csv")])
    assert v["l2_read_requests_model"].startswith("%d " % nreq)
    assert v["l2_read_requests_over_model"].startswith("1.5000")


def test_general_form_counter_summary(tmp_path):
    """The general-form workload's summary: compulsory bytes with C read and
    written, the general tile's closed form, and reads against the per-XCD
    panel model plus one read of C."""
    import tiled_fp32_gemm_sgemm_amd as sg
    from tiled_fp32_gemm_sgemm_amd import model
    from workloads import GENERAL_WORKLOADS
    w = GENERAL_WORKLOADS["atb4096"]
    k = "sgemm_dev::sgemm_mfma_dl_kernel<x>"
    cp = "MulFunctor<float>"
    copy_kib = bench.COPY_BYTES / 1024.0
    cfg = sg.select_general_config(w.M, w.N, w.K)
    info = sg.config_info(cfg)
    panels = model.per_xcd_operand_bytes(w.M, w.N, w.K, info["bm"], info["bn"], 1,
                                         resident=32 * sg.workgroups_per_cu(cfg))
    c_read = 4 * w.M * w.N
    # FETCH_SIZE scaled by 2 (the copy's 512 MiB read as 256 MiB): reads equal the model.
    _counter_csv(tmp_path / "f.csv", [(1, cp, "FETCH_SIZE", copy_kib / 2, 0, 1000),
                                      (2, k, "FETCH_SIZE", (panels + c_read) / 2048.0, 0, 900000)])
    _counter_csv(tmp_path / "w.csv", [(1, cp, "WRITE_SIZE", copy_kib, 0, 1000),
                                      (2, k, "WRITE_SIZE", c_read / 1024.0, 0, 900000)])
    out = tmp_path / "c.txt"
    bench.summarize_counters(str(out), "atb4096", "mfma", "sgemm_", str(tmp_path / "f.csv"),
                             str(tmp_path / "w.csv"), [], ["cmd"])
    v = dict(l.split(": ", 1) for l in out.read_text().splitlines()
             if ": " in l and not l.startswith("#"))
    assert v["compulsory_bytes"] == str(4 * (2 * w.M * w.K + 2 * w.M * w.N))
    assert v["mfma_instructions_closed_form"].endswith("(tile %s)" % info["name"])
    assert v["c_read_bytes"].startswith("%d " % c_read)
    assert v["beyond_l2_read_over_panel_model_plus_c"].startswith("1.0000")
    assert bench.gemm_traffic_file("ex", "atb4096").endswith("sgemm_ex_atb4096_counters.txt")


def test_general_form_bench_takes_its_own_tile(capsys):
    assert bench.main(["--workload", "atb4096", "--path", "valu"]) == 2
    assert bench.main(["--workload", "atb4096", "--config", "3"]) == 2
    assert "sgemm_ex" in capsys.readouterr().err
