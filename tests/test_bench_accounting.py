"""The byte accounting behind every bandwidth figure the benchmark prints.

Algorithmic bytes count each array an operation touches once, index tables
included ("Portable high-order finite element kernels I: Streaming
Operations", arXiv 2009.10917, the performance model: bandwidth is bytes
moved over time). The totals below are worked out by hand for the 32^3
order-7 box (N_G = 225^3, N_L = 32^3 * 8^3) from the arrays each operation
reads and writes, so an edit of the formulas in bench.py shows up here."""
import pytest

import bench

NG = 225 ** 3           # global nodes of the 32^3 order-7 box
NL = 32 ** 3 * 8 ** 3   # local entries
F64, I32 = 8, 4


def arrays_touched(op):
    """(element count, bytes per element) of every array op reads or writes."""
    return {
        "copy": [(NG, F64), (NG, F64)],                                  # read x, write y
        "axpy": [(NG, F64), (NG, F64), (NG, F64)],                       # read x, read y, write y
        "norm": [(NG, F64)],                                             # read x
        "dot": [(NG, F64), (NG, F64)],                                   # read x, y
        "cg_update": [(NG, F64)] * 6,                                    # read p q x r, write x r
        "scatter": [(NL, I32), (NG, F64), (NL, F64)],                    # read l2g, v_G once, write v_L
        "gather": [(NG + 1, I32), (NL, I32), (NL, F64), (NG, F64)],      # read off, ids, v_L; write v_G
    }[op]


@pytest.mark.parametrize("op", bench.OPS)
def test_op_bytes_at_the_box32_order7_mesh(op):
    want = sum(n * b for n, b in arrays_touched(op))
    assert bench.op_bytes(op, NG, NL, NG) == want


def test_printed_totals():
    got = {op: bench.op_bytes(op, NG, NL, NG) for op in bench.OPS}
    assert got == {"copy": 182_250_000, "axpy": 273_375_000, "norm": 91_125_000, "dot": 182_250_000,
                   "cg_update": 546_750_000, "scatter": 292_451_592, "gather": 338_014_096}
    assert sum(got.values()) == 1_906_215_688  # one step of all seven operations


def test_metric_names_the_peak():
    assert bench.PEAK_GBPS == 8000.0
    assert "GB/s" in bench.METRIC and "fp64" in bench.METRIC


def test_sweep_fit_on_synthetic_timings():
    """The sweep's post-processing on timings generated from known T0 and
    W_max: the fit recovers them, the residuals vanish, B_0.8 = 4 T0 W_max
    (eq. 10), and the plateau is the median rate of the points of >= 0.5 GB."""
    T0, W = 3e-6, 6.5e12
    B = [16 * 2 ** k for k in range(10, 29)]
    f = bench.sweep_fit([(b, T0 + b / W) for b in B])
    assert f["T0_s"] == pytest.approx(T0, rel=1e-9)
    assert f["W_max"] == pytest.approx(W, rel=1e-9)
    assert f["B_08_bytes"] == pytest.approx(4 * T0 * W, rel=1e-9)
    assert max(abs(r) for r in f["rel_residuals"]) < 1e-6 and f["r2_bandwidth"] == pytest.approx(1.0)
    big = [b / (T0 + b / W) for b in B if b >= 0.5e9]  # 2^25 .. 2^28 doubles
    assert len(big) == 4
    assert f["plateau_GBps"] == pytest.approx((sorted(big)[1] + sorted(big)[2]) / 2 / 1e9, abs=0.05)
    # a point measured 10% slow shows up as a residual of about -10% at its size
    pts = [(b, (T0 + b / W) * (1.1 if b == B[-1] else 1.0)) for b in B]
    g = bench.sweep_fit(pts)
    assert g["rel_residuals"][-1] < -0.05


def test_line_summaries():
    fits = {"copy": bench.sweep_fit([(16 * 2 ** k, 3e-6 + 16 * 2 ** k / 6.5e12) for k in range(10, 29)])}
    row = bench.sweep_summary(fits)["copy"]
    assert len(row) == len(bench.SWEEP_FIELDS)
    assert row[0] == pytest.approx(3.0, abs=0.01) and row[1] == pytest.approx(6500.0, abs=1)
    wl = {"box24_N15_mesh": {"n_local": 1}, "box24_N15": {"copy": {"us": 115.0, "pct_peak": 81.8}},
          "tetsplit11_N7_curve": {"scatter": {"us": 1.0, "pct_peak": 1.0}},
          "slab32x32x4_N7": {"copy": {"us": 6.0, "pct_peak": 48.0}},
          "cg_sequence_box24_N15": {"device_cg_us_per_iter": 1028.6, "fixed_scalars_us_per_iter": 1048.8,
                                    "true_cg_us_per_iter": 1090.7, "device_cg_GBps_moved": 5894.7},
          "cg_sequence_cg_box32_N7": {"device_cg_us_per_iter": 252.2, "fixed_scalars_us_per_iter": 269.8,
                                      "true_cg_us_per_iter": 307.3, "device_cg_GBps_moved": 6112.4}}
    out = bench.workload_summary(wl)
    assert out["box24_N15"] == {"copy": [115.0, 81.8]}
    assert out["cg_box24_N15"] == [1028.6, 1048.8, 1090.7, 5894.7]
    assert out["cg_box32_N7"][0] == 252.2
    # the mesh records, the slab and the secondary element orders stay out of the line
    assert not any(k.endswith("_mesh") or "slab" in k or k.endswith("_curve") for k in out)
