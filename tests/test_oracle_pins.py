"""Pins of the CPU oracle against what the pages and mathematics fix.

Nothing here compares the oracle with itself: every expected value comes from
exact integer/rational arithmetic, a closed form, a brute force over positions,
or a textbook routine (numpy's Legendre polynomials), so a dropped term, a
wrong sign or index, or a transposed operand in the oracle fails a test.
Pages: "Portable high-order finite element kernels I: Streaming Operations"
(arXiv 2009.10917; eqs. 1-3, the CG vector-operation list, the BS test list)
and "GPU accelerated spectral finite elements on all-hex meshes" (arXiv
1506.05996; the local-to-global and global-to-local tables).
"""
import math
import struct
from fractions import Fraction
from itertools import product

import numpy as np
import pytest

import bs_inputs

SCALE = 2 ** 52  # generated values are integer multiples of 2**-52


def as_int(v):
    """Exact integer X with v = X * 2**-52 (generated inputs only)."""
    X = v * SCALE
    assert X == int(X)
    return int(X)


def rn(fr):
    """Round an exact rational to the nearest binary64 (ties to even)."""
    return float(fr)


def bits(a):
    return np.asarray(a, dtype=np.float64).view(np.uint64)


# -------------------------------------------------------------- BS1 copy --

def test_copy_is_bitwise(orc):
    specials = [0.0, -0.0, float("inf"), -float("inf"), 5e-324, -2.2250738585072014e-308,
                1.0, -1.5]
    nan_payload = struct.unpack("<d", struct.pack("<Q", 0x7FF8_0000_DEAD_BEEF))[0]
    x = np.array(specials + [nan_payload] + list(bs_inputs.uniform_pm1(11, 1001)))
    y = orc.copy(x)
    assert y.tobytes() == x.tobytes()
    assert orc.copy(np.empty(0)).size == 0


# -------------------------------------------------------------- BS2 AXPY --

def test_axpy_matches_exact_rounding(orc):
    """y = RN(RN(a x) + RN(b y)): each product rounded, then the sum; no FMA."""
    n = 4000
    x = bs_inputs.uniform_pm1(21, n)
    y = bs_inputs.uniform_pm1(22, n)
    for a, b in [(0.37, 1.0), (-1.25, 0.7), (1.0, -0.3), (0.1, 0.0), (0.0, 0.9)]:
        out = orc.axpy(a, x, b, y)
        for i in range(n):
            t1 = rn(Fraction(a) * Fraction(x[i]))
            t2 = rn(Fraction(b) * Fraction(y[i]))
            want = rn(Fraction(t1) + Fraction(t2))
            assert out[i] == want, (a, b, i)
    # a fused multiply-add would round a*x + RN(b*y) once: find an input where
    # the two differ and check the oracle takes the separately rounded one
    a, b = 0.37, 1.0
    seen = False
    for i in range(n):
        fused = rn(Fraction(a) * Fraction(x[i]) + Fraction(y[i]))
        sep = rn(Fraction(rn(Fraction(a) * Fraction(x[i]))) + Fraction(y[i]))
        if fused != sep:
            seen = True
            assert orc.axpy(a, x[i:i + 1], b, y[i:i + 1])[0] == sep
    assert seen


def test_axpy_dyadic_closed_form(orc):
    x = bs_inputs.small_ints(31, 5000, -1000, 1000)
    y = bs_inputs.small_ints(32, 5000, -1000, 1000)
    assert np.array_equal(orc.axpy(0.5, x, 1.0, y), y + x / 2)
    assert np.array_equal(orc.axpy(1.0, x, -2.0, y), x - 2 * y)
    # beta = 0 still reads y: 0 * inf = NaN propagates
    yy = y.copy()
    yy[3] = np.inf
    out = orc.axpy(2.0, x, 0.0, yy)
    assert np.isnan(out[3]) and np.array_equal(np.delete(out, 3), np.delete(2 * x, 3))


# ------------------------------------------------------- BS3/BS4 reductions --

def exact_dot(x, y):
    S = sum(as_int(a) * as_int(b) for a, b in zip(x.tolist(), y.tolist()))
    return Fraction(S, SCALE * SCALE)


@pytest.mark.parametrize("n", [1, 2, 3, 1000, 65535, 65536, 65537, 150001])
def test_dot_exact_rational(orc, n):
    x = bs_inputs.uniform_pm1(41, n)
    y = bs_inputs.uniform_pm1(42, n)
    want = exact_dot(x, y)
    got = orc.dot(x, y)
    # Dot2 is accurate to about one rounding of the exact value
    assert abs(Fraction(got) - want) <= Fraction(2) * abs(want) * Fraction(1, 2 ** 53) + Fraction(1, 2 ** 150)


@pytest.mark.parametrize("n", [1000, 70001])
def test_dot_ill_conditioned(orc, n):
    """Random x, y plus one last pair (-RN(S), 1) with S the exact dot of the
    rest: the exact result S - RN(S) is below one ulp of S while sum |x y| is
    of order n, a condition number near 1e16. Dot2 (error-free products and
    sums) still returns it to high relative accuracy; a plain or half-
    compensated sum does not."""
    x = bs_inputs.uniform_pm1(48, n)
    y = bs_inputs.uniform_pm1(49, n)
    S = exact_dot(x, y)
    x = np.append(x, -float(S))
    y = np.append(y, 1.0)
    want = S - Fraction(float(S))
    assert want != 0
    got = orc.dot(x, y)
    assert abs(Fraction(got) - want) <= abs(want) * Fraction(1, 10 ** 6)


def test_dot_integer_vectors_exact(orc):
    n = 300_000
    x = bs_inputs.small_ints(43, n, -50, 50)
    y = bs_inputs.small_ints(44, n, -50, 50)
    want = int(np.dot(x.astype(np.int64), y.astype(np.int64)))
    assert orc.dot(x, y) == float(want)


def test_dot_unit_vectors_and_symmetry(orc):
    x = bs_inputs.uniform_pm1(45, 777)
    for k in [0, 1, 400, 776]:
        e = np.zeros(777)
        e[k] = 1.0
        assert orc.dot(x, e) == x[k]
        assert orc.dot(e, x) == x[k]
    y = bs_inputs.uniform_pm1(46, 777)
    assert orc.dot(x, y) == orc.dot(y, x)
    assert orc.dot(np.empty(0), np.empty(0)) == 0.0


def test_norm_closed_forms(orc):
    # sum of ones is exact, the square root correctly rounded
    for n in [1, 2, 3, 4, 9, 65536, 65537, 1 << 20, 1000003]:
        assert orc.norm(np.ones(n)) == math.sqrt(n)
    assert orc.norm(np.ones(1 << 20)) == 1024.0
    assert orc.norm(np.array([3.0, 4.0])) == 5.0
    assert orc.norm(np.array([-3.0, 0.0, 4.0])) == 5.0
    e = np.zeros(100)
    e[57] = -1.0
    assert orc.norm(e) == 1.0
    assert orc.norm(np.empty(0)) == 0.0


@pytest.mark.parametrize("n", [17, 70000])
def test_norm_exact_rational(orc, n):
    x = bs_inputs.uniform_pm1(47, n)
    s = exact_dot(x, x)
    want = math.sqrt(float(s))  # two roundings: within 1 ulp
    got = orc.norm(x)
    assert abs(got - want) <= 2 * np.spacing(want)
    # dot(x, x) = norm^2 to rounding
    assert abs(orc.dot(x, x) - got * got) <= 4 * np.spacing(got * got)


# ---------------------------------------------------- BS5 fused CG update --

def test_cg_update_exact(orc):
    n = 3000
    p = bs_inputs.uniform_pm1(51, n)
    q = bs_inputs.uniform_pm1(52, n)
    x = bs_inputs.uniform_pm1(53, n)
    r = bs_inputs.uniform_pm1(54, n)
    a = 0.37
    xo, ro, rr = orc.cg_update(a, p, q, x, r)
    for i in range(n):
        wx = rn(Fraction(x[i]) + Fraction(rn(Fraction(a) * Fraction(p[i]))))
        wr = rn(Fraction(r[i]) - Fraction(rn(Fraction(a) * Fraction(q[i]))))
        assert xo[i] == wx and ro[i] == wr, i
    # rr is the norm squared of the updated r, evaluated exactly here
    S = sum(Fraction(v) * Fraction(v) for v in ro.tolist())
    assert abs(Fraction(rr) - S) <= 2 * S / 2 ** 53


def test_cg_update_dyadic(orc):
    n = 4096
    p = bs_inputs.small_ints(55, n, -9, 9)
    q = bs_inputs.small_ints(56, n, -9, 9)
    x = bs_inputs.small_ints(57, n, -9, 9)
    r = bs_inputs.small_ints(58, n, -9, 9)
    xo, ro, rr = orc.cg_update(0.5, p, q, x, r)
    assert np.array_equal(xo, x + p / 2)
    assert np.array_equal(ro, r - q / 2)
    assert rr == float(np.sum((2 * r - q) ** 2)) / 4


# --------------------------------------------------------- GLL nodes ------

def test_gll_nodes_closed_forms(orc):
    assert np.array_equal(orc.gll_nodes(1), [-1.0, 1.0])
    assert np.array_equal(orc.gll_nodes(2), [-1.0, 0.0, 1.0])
    r3 = orc.gll_nodes(3)
    assert np.allclose(r3, [-1, -1 / math.sqrt(5), 1 / math.sqrt(5), 1], atol=1e-15, rtol=0)
    r4 = orc.gll_nodes(4)
    s = math.sqrt(3 / 7)
    assert np.allclose(r4, [-1, -s, 0, s, 1], atol=1e-15, rtol=0)


@pytest.mark.parametrize("p", [5, 7, 15])
def test_gll_nodes_are_roots_of_legendre_derivative(orc, p):
    r = orc.gll_nodes(p)
    want = np.sort(np.polynomial.legendre.Legendre.basis(p).deriv().roots().real)
    assert r[0] == -1.0 and r[-1] == 1.0
    assert np.all(np.diff(r) > 0)
    assert np.allclose(r[1:-1], want, atol=1e-12, rtol=0)


# ------------------------------------------------------------ mesh tables --

def mult_histogram(E, N):
    """Closed form: nodes of multiplicity 2^k number C(3,k) a^k b^(3-k)."""
    a, b = E - 1, E * (N - 1) + 2
    return {2 ** k: math.comb(3, k) * a ** k * b ** (3 - k) for k in range(4)}


@pytest.mark.parametrize("E,N", [(1, 1), (1, 4), (2, 2), (3, 1), (4, 3), (8, 3), (5, 5)])
def test_box_counts_and_multiplicities(orc, E, N):
    l2g, ng = orc.mesh_box(E, E, E, N)
    G = E * N + 1
    assert ng == G ** 3
    assert l2g.size == E ** 3 * (N + 1) ** 3
    assert l2g.min() == 0 and l2g.max() == ng - 1
    m = np.bincount(l2g, minlength=ng)
    hist = dict(zip(*np.unique(m, return_counts=True)))
    want = {k: v for k, v in mult_histogram(E, N).items() if v}
    assert {int(k): int(v) for k, v in hist.items()} == want
    # per-node multiplicity is the product of per-axis ones (2 on interior
    # element boundaries, 1 elsewhere)
    m1 = np.ones(G, dtype=np.int64)
    m1[N:G - 1:N] = 2
    want_m = (m1[None, None, :] * m1[None, :, None] * m1[:, None, None]).ravel()
    assert np.array_equal(m, want_m)


@pytest.mark.parametrize("E,N", [(2, 2), (2, 3), (3, 1)])
def test_box_bruteforce_positions(orc, E, N):
    """Two local nodes share an id iff their physical positions coincide, and
    ids follow the lexicographic order of positions (x fastest)."""
    l2g, ng = orc.mesh_box(E, E, E, N)
    r = np.sort(np.polynomial.legendre.Legendre.basis(N).deriv().roots().real) if N > 1 else np.array([])
    t = np.concatenate([[-1.0], r, [1.0]])
    pos = []
    for ez, ey, ex in product(range(E), repeat=3):
        for k, j, i in product(range(N + 1), repeat=3):
            pos.append((ex + (1 + t[i]) / 2, ey + (1 + t[j]) / 2, ez + (1 + t[k]) / 2))
    pos = np.array(pos)
    d = np.abs(pos[:, None, :] - pos[None, :, :]).max(axis=2)
    same = d < 1e-9
    assert np.array_equal(same, l2g[:, None] == l2g[None, :])
    # lexicographic (z, y, x) order of positions is the id order
    first = np.full(ng, -1)
    for L in range(l2g.size):
        if first[l2g[L]] < 0:
            first[l2g[L]] = L
    P = pos[first]
    key = [tuple(v) for v in P[:, ::-1]]
    assert key == sorted(key)


def test_box_anisotropic(orc):
    l2g, ng = orc.mesh_box(3, 2, 1, 2)
    assert ng == 7 * 5 * 3
    m = np.bincount(l2g, minlength=ng)
    assert m.sum() == 6 * 27
    # element (0,0,0) node (2,0,0) is shared with element (1,0,0) node (0,0,0)
    Np = 27
    assert l2g[0 * Np + 2] == l2g[1 * Np + 0]
    assert l2g[0 * Np + 2 + 3 * 2] == l2g[3 * Np + 2]  # (2,2,0) of e0 = (2,0,0) of e3


def test_box_shuffled_relation(orc):
    """Slot s holds element elem_perm[s]; lexicographic id g becomes node_perm[g]."""
    E, N = 4, 3
    Np = (N + 1) ** 3
    ep = bs_inputs.permutation(61, E ** 3)
    G = E * N + 1
    npm = bs_inputs.permutation(62, G ** 3)
    lex, ng = orc.mesh_box(E, E, E, N)
    shf, ng2 = orc.mesh_box(E, E, E, N, ep, npm)
    assert ng == ng2
    want = npm[lex.reshape(E ** 3, Np)[ep]].ravel()
    assert np.array_equal(shf, want)


def test_g2l_structure(orc):
    l2g, ng = orc.mesh_box(4, 4, 4, 3)
    off, ids = orc.g2l(l2g, ng)
    assert off[0] == 0 and off[-1] == l2g.size and np.all(np.diff(off) >= 1)
    assert np.array_equal(np.sort(ids), np.arange(l2g.size))
    for g in range(0, ng, 7):
        row = ids[off[g]:off[g + 1]]
        assert np.all(np.diff(row) > 0)
        assert np.all(l2g[row] == g)
        assert set(row.tolist()) == set(np.nonzero(l2g == g)[0].tolist())


def test_g2l_masked(orc):
    l2g, ng = orc.mesh_box(2, 2, 2, 2)
    l2g = l2g.copy()
    l2g[::5] = -1
    off, ids = orc.g2l(l2g, ng)
    assert off[-1] == np.count_nonzero(l2g >= 0)
    assert np.all(l2g[ids] >= 0)


# ----------------------------------------------------- BS6/BS7 gather/scatter --

def dense_Z(l2g, ng):
    Z = np.zeros((l2g.size, ng))
    for i, g in enumerate(l2g):
        if g >= 0:
            Z[i, g] = 1.0
    return Z


@pytest.mark.parametrize("E,N", [(2, 2), (3, 1), (2, 3)])
def test_scatter_gather_dense_bruteforce(orc, E, N):
    """Z is Boolean with one nonzero per row (eq. 3); its column sums are the
    multiplicities; Z v and Z^T v match dense products on integer data."""
    l2g, ng = orc.mesh_box(E, E, E, N)
    Z = dense_Z(l2g, ng)
    assert np.all(Z.sum(axis=1) == 1)
    vg = bs_inputs.small_ints(71, ng, -100, 100)
    vl = bs_inputs.small_ints(72, l2g.size, -100, 100)
    assert np.array_equal(orc.scatter(l2g, vg), Z @ vg)
    assert np.array_equal(orc.gather(l2g, vl, ng), Z.T @ vl)
    assert np.array_equal(orc.gather(l2g, np.ones(l2g.size), ng), Z.sum(axis=0))


def test_scatter_identity_values(orc):
    l2g, ng = orc.mesh_box(5, 5, 5, 4)
    vg = np.arange(ng, dtype=np.float64)
    assert np.array_equal(orc.scatter(l2g, vg), l2g.astype(np.float64))


def test_scatter_masked_is_positive_zero(orc):
    l2g = np.array([2, -1, 0, -7, 1], dtype=np.int32)
    vg = np.array([-0.0, 5.0, -3.0])
    out = orc.scatter(l2g, vg)
    assert out[0] == -3.0 and out[2] == -0.0 and np.signbit(out[2])
    assert out[1] == 0.0 and not np.signbit(out[1]) and not np.signbit(out[3])


def test_gather_ascending_local_order(orc):
    """Left-to-right summation from +0.0 in ascending local index.

    With v = (2^53, 1, 1, -2^53) mapping to one node: 2^53 + 1 is halfway
    between 2^53 and 2^53 + 2 and rounds to the even 2^53, twice, so the
    ascending sum is 0; the descending sum is 2 (every partial exact) and the
    pairwise tree (2^53+1) + (1-2^53) gives 1."""
    l2g = np.array([0, 0, 0, 0], dtype=np.int32)
    v = np.array([2.0 ** 53, 1.0, 1.0, -2.0 ** 53])
    assert orc.gather(l2g, v, 1)[0] == 0.0
    # positions interleaved with another node must not change that order
    l2g2 = np.array([1, 0, 1, 0, 1, 0, 0], dtype=np.int32)
    v2 = np.array([7.0, 2.0 ** 53, 8.0, 1.0, 9.0, 1.0, -2.0 ** 53])
    out = orc.gather(l2g2, v2, 3)
    assert out[0] == 0.0 and out[1] == 24.0 and out[2] == 0.0 and not np.signbit(out[2])


def test_gather_signed_zero_and_empty_rows(orc):
    l2g = np.array([0, 0, 2, -1], dtype=np.int32)
    v = np.array([-0.0, -0.0, -0.0, 5.0])
    out = orc.gather(l2g, v, 4)
    assert list(out) == [0.0, 0.0, 0.0, 0.0]
    assert not np.any(np.signbit(out))


def test_gather_scatter_multiplicity(orc):
    """Z^T Z v = m v exactly for small integers; sum of gather = sum of input."""
    E, N = 6, 4
    l2g, ng = orc.mesh_box(E, E, E, N)
    m = np.bincount(l2g, minlength=ng).astype(np.float64)
    v = bs_inputs.small_ints(81, ng, -1000, 1000)
    assert np.array_equal(orc.gather(l2g, orc.scatter(l2g, v), ng), m * v)
    vl = bs_inputs.small_ints(82, l2g.size, -1000, 1000)
    assert orc.gather(l2g, vl, ng).sum() == vl.sum()
    assert np.array_equal(orc.gather(l2g, np.ones(l2g.size), ng), m)


def test_gather_scatter_random_bound(orc):
    E, N = 4, 5
    l2g, ng = orc.mesh_box(E, E, E, N)
    m = np.bincount(l2g, minlength=ng).astype(np.float64)
    v = bs_inputs.uniform_pm1(83, ng)
    got = orc.gather(l2g, orc.scatter(l2g, v), ng)
    # repeated addition of the same value: within (m-1) roundings of m v
    assert np.all(np.abs(got - m * v) <= (m - 1) * np.spacing(m * np.abs(v)))


# ------------------------------------------------ lumped mass, 1/m scale ----

def test_gll_weights_closed_forms(orc):
    assert np.allclose(orc.gll_weights(1), [1, 1], rtol=0, atol=1e-15)
    assert np.allclose(orc.gll_weights(2), [1 / 3, 4 / 3, 1 / 3], rtol=0, atol=1e-15)
    assert np.allclose(orc.gll_weights(3), [1 / 6, 5 / 6, 5 / 6, 1 / 6], rtol=0, atol=1e-15)
    assert np.allclose(orc.gll_weights(4), [1 / 10, 49 / 90, 32 / 45, 49 / 90, 1 / 10], rtol=0, atol=1e-15)


@pytest.mark.parametrize("p", [1, 2, 5, 7, 15])
def test_gll_quadrature_exactness(orc, p):
    """GLL with p+1 points integrates every polynomial of degree <= 2p-1
    exactly: sum_i w_i r_i^k = 2/(k+1) for even k, 0 for odd k; and it fails
    for degree 2p (the end-point rule is not Gauss)."""
    r, w = orc.gll_nodes(p), orc.gll_weights(p)
    for k in range(2 * p):
        want = 2.0 / (k + 1) if k % 2 == 0 else 0.0
        assert abs(np.dot(w, r ** k) - want) < 1e-13, k
    assert abs(np.dot(w, r ** (2 * p)) - 2.0 / (2 * p + 1)) > 1e-11


@pytest.mark.parametrize("E,N", [(1, 3), (3, 2), (4, 7)])
def test_lumped_mass(orc, E, N):
    """m = Z^T w_L: positive, sums to the box volume E^3, and on one element
    is the tensor product of the GLL weights over 8."""
    l2g, ng = orc.mesh_box(E, E, E, N)
    wl = orc.mesh_box_mass(E, E, E, N)
    m = orc.gather(l2g, wl, ng)
    assert np.all(m > 0)
    assert abs(m.sum() - E ** 3) <= 1e-12 * E ** 3
    if E == 1:
        w = orc.gll_weights(N)
        want = (w[None, None, :] * w[None, :, None] * w[:, None, None]).ravel() / 8
        assert np.allclose(m, want, rtol=1e-15, atol=0)
    # a node shared by two elements gets both elements' weights
    w = orc.gll_weights(N)
    if E > 1:
        g = l2g[N]  # node (N,0,0) of element 0 is node (0,0,0) of element 1
        assert m[g] == (w[N] * w[0] * w[0] / 8.0) + (w[0] * w[0] * w[0] / 8.0)


def test_scale_exact_rounding(orc):
    x = bs_inputs.uniform_pm1(201, 3000)
    d = bs_inputs.uniform_pm1(202, 3000) + 2.0
    y = orc.scale(x, d)
    for i in range(3000):
        assert y[i] == rn(Fraction(x[i]) / Fraction(d[i]))
    assert np.array_equal(orc.scale(x, np.ones(3000)), x)


# ------------------------------------------------------- CG on Z^T Z ------

def test_cg_sequence_converges_in_four(orc):
    """A = Z^T Z = diag(m), m in {1,2,4,8}: CG ends in at most 4 steps, x = b/m."""
    E, N = 4, 3
    l2g, ng = orc.mesh_box(E, E, E, N)
    m = np.bincount(l2g, minlength=ng).astype(np.float64)
    b = bs_inputs.uniform_pm1(91, ng)
    x, r, hist = orc.cg_sequence(l2g, ng, b, 4)
    assert math.sqrt(hist[-1] / hist[0]) < 1e-13
    assert np.allclose(x, b / m, rtol=1e-12, atol=1e-14)
    # one distinct multiplicity in the support: a single step suffices
    b1 = np.where(m == 2.0, b, 0.0)
    x1, _, h1 = orc.cg_sequence(l2g, ng, b1, 1)
    assert math.sqrt(h1[-1] / h1[0]) < 1e-15
    assert np.allclose(x1, b1 / m, rtol=1e-15, atol=0)


# ------------------------------------------- unstructured hex meshes ------
# A global numbering is fixed only up to renaming; the oracle numbers nodes by
# first appearance, so every expected partition below is renamed the same way
# before the arrays are compared.

def first_touch(keys):
    """Rename equal keys 0, 1, 2, ... in order of first appearance."""
    keys = np.asarray(keys)
    _, first, inv = np.unique(keys, return_index=True, return_inverse=True)
    rank = np.empty(len(first), dtype=np.int64)
    rank[np.argsort(first, kind="stable")] = np.arange(len(first))
    return rank[inv.ravel()].astype(np.int32)


def unrotate(l2g, sym, N):
    """Undo bs_inputs.hex_orient on a local array: element e was presented in
    the corner order of cube symmetry sym[e]; return the array in the
    element's original node order."""
    nq = N + 1
    loc = np.asarray(l2g).reshape(-1, nq, nq, nq)  # [e, k, j, i]
    out = np.empty_like(loc)
    q = np.stack(np.meshgrid(np.arange(nq), np.arange(nq), np.arange(nq), indexing="ij"), -1)  # [k,j,i,(k,j,i)]
    q = q[..., ::-1]  # (i, j, k)
    for e in range(loc.shape[0]):
        perm, flip, _ = bs_inputs.cube_symmetry(int(sym[e]))
        o = np.empty_like(q)
        for a in range(3):
            o[..., perm[a]] = np.where((flip >> a) & 1, N - q[..., a], q[..., a])
        out[e, o[..., 2], o[..., 1], o[..., 0]] = loc[e]
    return out.ravel()


def entity_count(ev, N):
    """Global node count from the mesh's entities: vertices, then N-1 nodes
    per edge, (N-1)^2 per face and (N-1)^3 per element."""
    edges, faces = set(), set()
    for h in ev:
        for c in range(8):
            for a in range(3):
                if not (c >> a) & 1:
                    edges.add(frozenset((h[c], h[c | 1 << a])))
        for a in range(3):
            for side in (0, 1):
                faces.add(frozenset(h[c] for c in range(8) if (c >> a) & 1 == side))
    V = len(set(np.asarray(ev).ravel()))
    return V + (N - 1) * len(edges) + (N - 1) ** 2 * len(faces) + (N - 1) ** 3 * len(ev)


@pytest.mark.parametrize("dims,N", [((1, 1, 1), 1), ((2, 3, 2), 3), ((4, 3, 2), 4), ((3, 3, 3), 7)])
def test_hex_box_equals_box_positions(orc, dims, N):
    """On the box lattice the corner-connectivity oracle finds exactly the
    partition of the position-based box oracle, and the lattice count."""
    ev, nv = bs_inputs.hex_box(*dims)
    l2g, ng = orc.mesh_hex(ev, N, nv)
    box, bng = orc.mesh_box(*dims, N)
    assert ng == bng == math.prod(d * N + 1 for d in dims)
    assert np.array_equal(l2g, first_touch(box))


@pytest.mark.parametrize("N", [1, 2, 5])
def test_hex_orientation_invariant(orc, N):
    """Presenting every element in a random one of the 48 corner orders of the
    cube renames its local nodes only: undoing the renaming gives the box's
    partition back."""
    ev, nv = bs_inputs.hex_box(3, 2, 3)
    rot, sym = bs_inputs.hex_orient(ev, 501)
    assert len(set(sym.tolist())) > 10
    l2g, ng = orc.mesh_hex(rot, N, nv)
    box, bng = orc.mesh_box(3, 2, 3, N)
    assert ng == bng
    assert np.array_equal(first_touch(unrotate(l2g, sym, N)), first_touch(box))


def test_hex_vertex_names_do_not_matter(orc):
    ev, nv = bs_inputs.hex_box(3, 3, 2)
    rot, _ = bs_inputs.hex_orient(ev, 502)
    ref, ng = orc.mesh_hex(rot, 4, nv)
    ev2, nv2 = bs_inputs.hex_relabel(rot, nv, 503, spare=17)
    l2g, ng2 = orc.mesh_hex(ev2, 4, nv2)
    assert ng2 == ng and np.array_equal(l2g, ref)


def lattice_keys(dims, N, periodic, twist):
    """Brute force: node (i,j,k) of cell (cx,cy,cz) is the lattice point
    (cx N + i, ...), wrapped on periodic axes (and reflected in y where the
    twisted x axis wraps)."""
    nx, ny, nz = dims
    G = [d * N for d in dims]
    keys = []
    for cz in range(nz):
        for cy in range(ny):
            for cx in range(nx):
                for k in range(N + 1):
                    for j in range(N + 1):
                        for i in range(N + 1):
                            X, Y, Z = cx * N + i, cy * N + j, cz * N + k
                            if periodic[0] and X == G[0]:
                                X = 0
                                if twist:
                                    Y = G[1] - Y
                            if periodic[1]:
                                Y %= G[1]
                            if periodic[2]:
                                Z %= G[2]
                            keys.append((Z * (G[1] + 1) + Y) * (G[0] + 1) + X)
    return np.array(keys)


@pytest.mark.parametrize("periodic,twist", [((True, False, False), False), ((True, True, True), False),
                                            ((True, False, True), True)])
@pytest.mark.parametrize("N", [2, 3])
def test_hex_periodic_and_twisted(orc, periodic, twist, N):
    dims = (3, 3, 4)
    ev, nv = bs_inputs.hex_box(*dims, periodic=periodic, twist=twist)
    rot, sym = bs_inputs.hex_orient(ev, 504)
    l2g, ng = orc.mesh_hex(rot, N, nv)
    want = first_touch(lattice_keys(dims, N, periodic, twist))
    assert ng == want.max() + 1
    assert ng == math.prod(d * N + (0 if p else 1) for d, p in zip(dims, periodic))
    assert np.array_equal(first_touch(unrotate(l2g, sym, N)), want)


def gll_points(N):
    """GLL points from numpy's Legendre class: -1, the roots of P_N', +1."""
    inner = np.polynomial.legendre.Legendre.basis(N).deriv().roots() if N > 1 else np.array([])
    return np.concatenate([[-1.0], np.sort(inner.real), [1.0]])


@pytest.mark.parametrize("N", [1, 3, 6])
def test_hex_tet_split_by_physical_positions(orc, N):
    """Unstructured mesh: maps every local node through its element's
    trilinear map and clusters the physical points (distance < 1e-9); the
    clusters are the oracle's global nodes. The count also matches the
    entity formula."""
    from scipy.sparse import coo_matrix
    from scipy.sparse.csgraph import connected_components
    from scipy.spatial import cKDTree

    ev, nv, X = bs_inputs.hex_tet_split(2, 1, 2)
    l2g, ng = orc.mesh_hex(ev, N, nv)
    assert ng == entity_count(ev, N)
    r = gll_points(N)
    t = (1 + r) / 2
    phi = np.stack([1 - t, t])  # [bit, node]
    nq = N + 1
    pts = np.zeros((len(ev), nq, nq, nq, 3))
    for c in range(8):
        a, b, d = c & 1, (c >> 1) & 1, (c >> 2) & 1
        w = phi[d][:, None, None] * phi[b][None, :, None] * phi[a][None, None, :]  # [k, j, i]
        pts += w[None, :, :, :, None] * X[ev[:, c]][:, None, None, None, :]
    pts = pts.reshape(-1, 3)
    pairs = cKDTree(pts).query_pairs(1e-9, output_type="ndarray")
    n = len(pts)
    g = coo_matrix((np.ones(len(pairs)), (pairs[:, 0], pairs[:, 1])), shape=(n, n))
    ncomp, lab = connected_components(g, directed=False)
    assert ncomp == ng
    assert np.array_equal(l2g, first_touch(lab))


def test_hex_rejects_bad_elements(orc):
    ev, nv = bs_inputs.hex_box(2, 1, 1)
    bad = ev.copy()
    bad[1, 3] = bad[1, 0]
    with pytest.raises(ValueError):
        orc.mesh_hex(bad, 2, nv)
    with pytest.raises(ValueError):
        orc.mesh_hex(ev, 2, int(ev.max()))
    l2g, ng = orc.mesh_hex(np.zeros((0, 8), np.int32), 3, 0)
    assert l2g.size == 0 and ng == 0


# ------------------------------------------- unstructured lumped mass ------

def gll_rule(N):
    """GLL points and weights from numpy's Legendre class (independent of the
    oracle): -1, the roots of P_N', +1; w = 2 / (N (N+1) P_N(r)^2)."""
    r = gll_points(N)
    P = np.polynomial.legendre.Legendre.basis(N)(r)
    return r, 2.0 / (N * (N + 1) * P * P)


@pytest.mark.parametrize("N", [1, 3, 7])
def test_hexmass_unit_box(orc, N):
    xe = bs_inputs.hex_box_coords(3, 2, 2)
    w = orc.mesh_hex_mass(xe, N)
    assert np.allclose(w, orc.mesh_box_mass(3, 2, 2, N), rtol=1e-14, atol=0)


@pytest.mark.parametrize("N", [1, 2, 5])
def test_hexmass_affine_elements(orc, N):
    """An affine image A x + b of the unit cubes has the constant Jacobian
    det A / 8 on the reference cube: every weight is w_i w_j w_k |det A| / 8
    and every element holds |det A|."""
    A = np.array([[1.3, 0.2, -0.1], [0.05, 0.9, 0.3], [-0.2, 0.1, 1.1]])
    xe = bs_inputs.hex_box_coords(2, 2, 1) @ A.T + np.array([0.5, -1.0, 2.0])
    w = orc.mesh_hex_mass(xe, N).reshape(4, -1)
    r, g = gll_rule(N)
    want = (g[None, None, :] * g[None, :, None] * g[:, None, None]).ravel() * abs(np.linalg.det(A)) / 8
    for e in range(4):
        assert np.allclose(w[e], want, rtol=1e-13, atol=0)
        assert w[e].sum() == pytest.approx(abs(np.linalg.det(A)), rel=1e-13)


@pytest.mark.parametrize("N", [2, 4, 6])
def test_hexmass_trilinear_frustum(orc, N):
    """Bottom face the unit square, top face [0, s]^2 at height 1: with
    u, v, w = (1 + xi)/2 ... the map is x = u h, y = v h, z = w, h = 1 + (s-1) w,
    so det J = h^2 / 8 pointwise and the volume (1 + s + s^2) / 3, which GLL
    integrates exactly from N = 2 (degree 2 in w)."""
    s = 1.7
    xe = np.array([[[0, 0, 0], [1, 0, 0], [0, 1, 0], [1, 1, 0],
                    [0, 0, 1], [s, 0, 1], [0, s, 1], [s, s, 1]]], dtype=np.float64)
    w = orc.mesh_hex_mass(xe, N)
    r, g = gll_rule(N)
    h = 1 + (s - 1) * (1 + r) / 2
    want = (g[:, None, None] * h[:, None, None] ** 2 * g[None, :, None] * g[None, None, :]).ravel() / 8
    assert np.allclose(w, want, rtol=1e-13, atol=0)
    assert w.sum() == pytest.approx((1 + s + s * s) / 3, rel=1e-13)


@pytest.mark.parametrize("N", [2, 5])
def test_hexmass_tet_split_volumes(orc, N):
    """Each of the four hexahedra of a tetrahedron is its barycentric quarter:
    in a unit cube's Kuhn split every hexahedron has volume 1/24, and their
    Jacobians are of degree 2 per variable, so GLL from N = 2 is exact."""
    ev, nv, X = bs_inputs.hex_tet_split(2, 1, 2)
    w = orc.mesh_hex_mass(X[ev], N).reshape(len(ev), -1)
    assert np.allclose(w.sum(axis=1), 1.0 / 24, rtol=1e-13, atol=0)
    assert np.all(w > 0)


def test_hexmass_orientation(orc):
    """Any of the 48 corner orders (reflections give det J < 0) renames the
    element's nodes and leaves the weight of each physical node alone."""
    N = 4
    ev, nv, X = bs_inputs.hex_tet_split(1, 1, 1)
    xe = X[ev]
    sym = (bs_inputs.splitmix64(601, len(ev)) % np.uint64(48)).astype(np.int64)
    w0 = orc.mesh_hex_mass(xe, N)
    w1 = orc.mesh_hex_mass(bs_inputs.reorder_corners(xe, sym), N)
    assert np.allclose(unrotate(w1, sym, N), w0, rtol=1e-14, atol=0)
