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
                 "hbm_bytes_per_launch: %s\n" % (source_hash, tile, hbm))
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
