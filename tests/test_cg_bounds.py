"""CPU pins of the CG drift bounds (tests/cg_bounds.py) that the GPU CG
tests use as their tolerance.

The bounds are first-order sensitivities of CG on A = Z^T Z = diag(m) to
every rounding, computed in the class space of the multiplicities. They are
pinned here against things that do not come from the bound code itself:
  - a closed form: exact CG makes r_1 orthogonal to r_0, so a relative change
    d of alpha_0 changes rr_1 by exactly 2 d rr_1 to first order, and beta_0
    does not touch rr_1;
  - a second floating-point CG whose reductions are summed differently (numpy
    pairwise sums instead of the oracle's Dot2) stays inside the bounds;
  - the bounds have teeth: a CG whose reductions are off by much more than
    the assumed bound fails them;
  - one multiplicity class: CG converges in one step, so rr_1 is rounding
    noise and is held to the floor.
"""
from decimal import Decimal, localcontext

import numpy as np
import pytest

import bs_inputs
import cg_bounds as cb


def numpy_cg(orc, l2g, ng, b, iters, pq_scale=None):
    """CG on Z^T Z with the oracle's elementwise operations but numpy's
    summation for r.r and p.q; pq_scale[k] multiplies the p.q of step k."""
    x = np.zeros_like(b)
    r, p = b.copy(), b.copy()
    rr = float(np.sum(r * r))
    hist = [rr]
    for k in range(iters):
        q = orc.gather(l2g, orc.scatter(l2g, p), ng)
        pq = float(np.sum(p * q))
        if pq_scale is not None:
            pq *= pq_scale[k]
        a = rr / pq
        x, r, _ = orc.cg_update(a, p, q, x, r)
        rn = float(np.sum(r * r))
        p = orc.axpy(1.0, r, rn / rr, p)
        rr = rn
        hist.append(rr)
    return x, hist


def box(bs, E, N):
    l2g = bs.bs_mesh_box_l2g(E, E, E, N)
    ng = bs.bs_mesh_box_count(E, E, E, N)[1]
    return l2g, ng


@pytest.fixture(scope="module")
def lib():
    import cg_streaming_vector_amd as bs
    bs._lib()
    return bs


def test_first_step_sensitivity_closed_form():
    lam, S = [1.0, 2.0, 4.0, 8.0], [3.0, 5.0, 7.0, 11.0]
    h = Decimal("1e-40")
    with localcontext() as ctx:
        ctx.prec = 80
        base = cb._run(lam, S, 2)
        da = cb._run(lam, S, 2, ("alpha", 0, None, h))
        db = cb._run(lam, S, 2, ("beta", 0, None, h))
        rel_a = (da[0][1] - base[0][1]) / h / base[0][1]
        rel_b = (db[0][1] - base[0][1]) / h / base[0][1]
        assert abs(rel_a - 2) < Decimal("1e-30")
        assert rel_b == 0
        # r_1 is orthogonal to r_0 in the class-space inner product
        dotp = sum(base[1][1][c] * base[1][0][c] * Decimal(S[c]) for c in range(4))
        assert abs(dotp) < Decimal("1e-60")


def test_exact_cg_converges_in_one_step_per_class():
    lam, S = [1.0, 3.0, 4.0], [2.0, 1.0, 0.5]
    B = cb.CgBounds(lam, S, 3)
    assert B.rr_exact[3] < 1e-60 * B.rr_exact[0]
    assert np.allclose(B.xi_exact, [1.0, 1 / 3, 0.25], rtol=1e-14)
    assert B.significant(2) and not B.significant(3)


@pytest.mark.parametrize("case", ["box8_N3", "tet_split"])
def test_a_differently_summed_cg_stays_inside_the_bounds(lib, orc, case):
    if case == "box8_N3":
        l2g, ng = box(lib, 8, 3)
        b = bs_inputs.uniform_pm1(1001, ng)
    else:
        ev, nv, _ = bs_inputs.hex_tet_split(6, 5, 6)
        ev, _ = bs_inputs.hex_orient(ev, 701)
        l2g, ng = lib.bs_mesh_hex_l2g(ev, 5, nv)
        b = bs_inputs.uniform_pm1(721, ng)
    off, _ = lib.bs_index_g2l(l2g, ng)
    m = np.diff(off)
    iters = len(np.unique(m))
    ox, _, ohist = orc.cg_sequence(l2g, ng, b, iters)
    x, hist = numpy_cg(orc, l2g, ng, b, iters)
    bounds = cb.check_cg(hist, ohist, x, ox, m, b, iters, case)
    # the bounds are tight enough to mean something: every compared step at
    # most a few 1e-12 relative
    assert max(bounds.rel_tol[k] for k in range(iters)) < 1e-11


def test_a_cg_with_worse_reductions_fails_the_bounds(lib, orc):
    l2g, ng = box(lib, 8, 3)
    b = bs_inputs.uniform_pm1(1001, ng)
    off, _ = lib.bs_index_g2l(l2g, ng)
    m = np.diff(off)
    ox, _, ohist = orc.cg_sequence(l2g, ng, b, 4)
    # p.q off by 1e-13 relative (inside the assumed reduction bound): passes
    x, hist = numpy_cg(orc, l2g, ng, b, 4, pq_scale=[1 + 1e-13] * 4)
    cb.check_cg(hist, ohist, x, ox, m, b, 4, "1e-13")
    # off by 1e-10: far outside what rounding explains
    x, hist = numpy_cg(orc, l2g, ng, b, 4, pq_scale=[1.0, 1 + 1e-10, 1.0, 1.0])
    with pytest.raises(AssertionError):
        cb.check_cg(hist, ohist, x, ox, m, b, 4, "1e-10")


def test_single_class_is_held_to_the_floor(lib, orc):
    # one element: every node has multiplicity 1, A = I, CG is exact after one step
    l2g, ng = box(lib, 1, 3)
    b = bs_inputs.uniform_pm1(1002, ng)
    off, _ = lib.bs_index_g2l(l2g, ng)
    m = np.diff(off)
    ox, _, ohist = orc.cg_sequence(l2g, ng, b, 1)
    x, hist = numpy_cg(orc, l2g, ng, b, 1)
    bounds = cb.check_cg(hist, ohist, x, ox, m, b, 1, "one class")
    assert not bounds.significant(1)
    # the floor is set by alpha's assumed error (2 eta + u, about 2.3e-13):
    # a relative residual of that order
    assert bounds.floor[1] <= (4 * cb.ETA_GPU) ** 2 * hist[0]
    assert hist[1] <= 1e-30 * hist[0] and ohist[1] <= 1e-30 * hist[0]
