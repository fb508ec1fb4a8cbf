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
