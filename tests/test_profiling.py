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
    # a wrong copy size (the run copied n doubles, the caller says 8 n) is refused
    with pytest.raises(ValueError, match="copy-doubles"):
        profiling.summarize(tmp_path / "s.csv", tmp_path / "f.csv", tmp_path / "w.csv", "k_copy<1>", 8 * n)
    md = profiling.to_markdown(s, "t", ["rocprofv3 ..."])
    assert "k_scatter" in md and "rocprofv3 ..." in md


def test_resources_from_trace(tmp_path):
    hdr = ["Kernel_Name", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "LDS_Block_Size", "Scratch_Size",
           "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    with open(tmp_path / "t.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(hdr)
        w.writerow(["(anonymous namespace)::k_scatter(y)", 92, 0, 24, 0, 0, 256, 1, 1, 256 * 1024, 1, 1])
        w.writerow(["(anonymous namespace)::k_scatter(y)", 92, 0, 24, 0, 0, 256, 1, 1, 256 * 4096, 1, 1])
        w.writerow(["void (anonymous namespace)::k_gather_plan<false>(z)", 8, 0, 30, 12800, 0, 256, 1, 1, 2560, 1,
                    1])
    r = profiling.load_resources(tmp_path / "t.csv")
    assert r["k_scatter"]["max_workgroups"] == 4096 and r["k_scatter"]["workgroup"] == 256
    assert r["k_gather_plan<false>"]["lds_bytes"] == 12800 and r["k_gather_plan<false>"]["max_workgroups"] == 10


def test_compiler_remarks(tmp_path):
    text = """x.hip:1:1: remark: Function Name: _Z1kv [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     TotalSGPRs: 28 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     VGPRs: 46 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     Occupancy [waves/SIMD]: 2 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     LDS Size [bytes/block]: 32 [-Rpass-analysis=kernel-resource-usage]
"""
    (tmp_path / "r.txt").write_text(text)
    r = profiling.load_remarks(tmp_path / "r.txt", demangle=lambda n: "void (anonymous namespace)::k_dot<4, false>()")
    k = r["k_dot<4, false>"]
    assert k["vgpr"] == 46 and k["sgpr"] == 28 and k["occupancy"] == 2 and k["vgpr_spill"] == 0
    assert k["lds_static"] == 32 and k["scratch_per_lane"] == 0
    s = profiling.summarize(None, None, None, "k_copy<1>", 1, remarks=None)
    s["kernels"]["k_dot<4, false>"] = {"compiler": k}
    md = profiling.to_markdown(s, "t", [])
    assert "| `k_dot<4, false>` | 46 | 0 | 28 | 0/ | 2 |" in md


def test_reused_calibration(tmp_path):
    fetch = [("(anonymous namespace)::k_scatter(y)", "FETCH_SIZE", 30.0)]
    write = [("(anonymous namespace)::k_scatter(y)", "WRITE_SIZE", 20.0)]
    write_counters(tmp_path / "f.csv", fetch)
    write_counters(tmp_path / "w.csv", write)
    s = profiling.summarize(None, tmp_path / "f.csv", tmp_path / "w.csv", "k_copy<1>", 1000, calibration=(2.0, 1.0))
    assert s["calibration"]["reused"]
    assert s["kernels"]["k_scatter"]["hbm_bytes_per_launch"] == pytest.approx(30 * 1024 * 2 + 20 * 1024)
    assert "reused" in profiling.to_markdown(s, "t", [])


def test_in_step_launches(tmp_path):
    """Only the launches between the step's neighbours are averaged; the
    per-operation loop's back-to-back launches of the same kernel are not."""
    rows = []
    t = 0

    def launch(name, dur, queue=1):
        nonlocal t
        rows.append([queue, t, t + dur, f"void (anonymous namespace)::{name}(x)"])
        t += dur + 10

    for _ in range(3):          # the per-operation loop: the kernel back to back
        launch("k_cg_update<4>", 1000)
    for d in (1200, 1400):      # two steps: dot, update, scatter
        launch("k_dot<4, false>", 500)
        launch("k_cg_update<4>", d)
        launch("k_scatter", 700)
    launch("k_dot<4, false>", 500, queue=2)  # a neighbour on another queue does not count
    launch("k_cg_update<4>", 9999)
    launch("k_scatter", 700)
    with open(tmp_path / "trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Queue_Id", "Start_Timestamp", "End_Timestamp", "Kernel_Name"])
        w.writerows(rows)
    d = profiling.load_in_step(tmp_path / "trace.csv", "k_dot<4, false>", "k_cg_update<4>", "k_scatter")
    assert d == [1200, 1400]


def test_counter_averages(tmp_path):
    """--pmc: plain per-kernel averages per dispatch over several counter
    files, filtered to the kernels asked for."""
    write_counters(tmp_path / "a.csv", [
        ("void (anonymous namespace)::k_gather_plan<false>(x)", "SQ_WAVES", 8.0),
        ("void (anonymous namespace)::k_gather_plan<false>(x)", "SQ_WAVES", 12.0),
        ("(anonymous namespace)::k_scatter(y)", "SQ_WAVES", 4.0),
        ("__amd_rocclr_copyBuffer", "SQ_WAVES", 99.0)])
    write_counters(tmp_path / "b.csv", [
        ("void (anonymous namespace)::k_gather_plan<false>(x)", "TCC_HIT_sum", 3.0)])
    t = profiling.load_counters([tmp_path / "a.csv", tmp_path / "b.csv"], {"k_gather_plan<false>", "k_scatter"})
    assert set(t) == {"k_gather_plan<false>", "k_scatter"}
    assert t["k_gather_plan<false>"]["SQ_WAVES"] == [8.0, 12.0]
    assert t["k_gather_plan<false>"]["TCC_HIT_sum"] == [3.0]
    md_path = tmp_path / "c.md"
    profiling.main(["--pmc", str(tmp_path / "a.csv"), "--pmc", str(tmp_path / "b.csv"), "--kernel",
                    "k_gather_plan<false>", "--title", "t", "--command", "rocprofv3 --pmc ...", "--md", str(md_path)])
    md = md_path.read_text()
    assert "| SQ_WAVES | 2 | 10 |" in md and "| TCC_HIT_sum | 1 | 3 |" in md
    assert "k_scatter" not in md and "rocprofv3 --pmc ..." in md
