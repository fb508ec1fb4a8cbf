"""Host logic of the rocprofv3 summaries (no GPU): kernel-name parsing and the
copy-kernel calibration of the FETCH_SIZE / WRITE_SIZE counters."""
import csv

import pytest

from cg_streaming_vector_amd import profiling


def test_short_name():
    f = profiling.short_name
    assert f("void (anonymous namespace)::k_dot<2, true>((anonymous namespace)::Split, double const*)") == \
        "k_dot<2, true>"
    assert f("(anonymous namespace)::k_scatter(long, int const*, double const*, double*)") == "k_scatter"
    assert f("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)


def test_calibrated_traffic(tmp_path):
    n = 1000
    # the read counter reports half, the write counter all of a copy's bytes
    fetch = [("void (anonymous namespace)::k_copy<1>(x)", "FETCH_SIZE", 8 * n / 2 / 1024)] * 3
    fetch += [("(anonymous namespace)::k_scatter(y)", "FETCH_SIZE", 30.0)]
    write = [("void (anonymous namespace)::k_copy<1>(x)", "WRITE_SIZE", 8 * n / 1024)] * 3
    write += [("(anonymous namespace)::k_scatter(y)", "WRITE_SIZE", 20.0)]
    write_counters(tmp_path / "f.csv", fetch)
    write_counters(tmp_path / "w.csv", write)
    with open(tmp_path / "s.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "AverageNs"])
        w.writerow(["(anonymous namespace)::k_scatter(y)", 7, 1500.0])
    s = profiling.summarize(tmp_path / "s.csv", tmp_path / "f.csv", tmp_path / "w.csv", "k_copy<1>", n)
    assert s["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert s["calibration"]["write_scale"] == pytest.approx(1.0)
    assert s["kernels"]["k_copy<1>"]["hbm_bytes_per_launch"] == pytest.approx(16 * n)
    k = s["kernels"]["k_scatter"]
    assert k["hbm_bytes_per_launch"] == pytest.approx(30 * 1024 * 2 + 20 * 1024)
    assert k["calls"] == 7 and k["avg_ns"] == 1500.0
    md = profiling.to_markdown(s, "t", ["rocprofv3 ..."])
    assert "k_scatter" in md and "rocprofv3 ..." in md
