"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Bar (arXiv 2009.10917 defines the operations; the tolerances are this
library's contract): bit-exact for copy, AXPY, the fused update's x and r,
scatter and both gather kernels; relative 1e-12 for norm, dot and the fused
update's |r|^2. Sizes span several tiles with ragged tails, the empty and
one-element cases, misaligned operands, and the full workloads: the 32^3
order-7 box, the shuffled 40^3 order-5 box, the 24^3 order-15 box, and the
2^10 .. 2^28 vector sweep, launched exactly as the benchmark launches them.
"""
import math

import numpy as np
import pytest

import bs_inputs
from cg_bounds import check_cg

pytestmark = pytest.mark.gpu

RTOL = 1e-12


@pytest.fixture(scope="module")
def env():
    import torch
    import cg_streaming_vector_amd as bs
    import oracle
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device")
    oracle.lib()
    return bs, oracle, torch, torch.device("cuda:0")


def dev(torch, device, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t):
    return t.cpu().numpy()


def assert_bits(got, want, what=""):
    g = np.asarray(got, dtype=np.float64).view(np.uint64)
    w = np.asarray(want, dtype=np.float64).view(np.uint64)
    assert g.shape == w.shape, what
    bad = np.nonzero(g != w)[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}"


def assert_rel(got, want, what=""):
    assert abs(got - want) <= RTOL * abs(want) or got == want, f"{what}: {got!r} vs {want!r}"


# -------------------------------------------------------- vector ops ------

SIZES = [1, 2, 3, 4, 5, 7, 8, 255, 256, 257, 1023, 1024, 1025, 4099, 65537, 262147, 1 << 20, (1 << 20) + 5,
         3_000_001]


def run_vector_ops(env, n, seed, offset=(0, 0, 0, 0)):
    """All five vector ops at length n; offset[k] shifts operand k by elements
    inside a larger buffer (to test 8- but not 16-byte aligned pointers)."""
    bs, orc, torch, d = env
    v = {k: bs_inputs.uniform_pm1(seed + i, n) for i, k in enumerate("xpqr")}

    def place(a, o):
        buf = torch.empty(n + 2, dtype=torch.float64, device=d)
        t = buf[o:o + n]
        t.copy_(torch.from_numpy(a))
        return t

    x, p, q, r = (place(v[k], offset[i]) for i, k in enumerate("xpqr"))
    # copy
    y = place(np.zeros(n), offset[1])
    bs.bs_copy(x, y)
    assert_bits(host(y), v["x"], f"copy n={n}")
    # axpy with the benchmark's coefficients and a general pair
    for a, b in [(0.37, 1.0), (-1.5, 0.25)]:
        y = place(v["p"], offset[1])
        bs.bs_axpy(a, x, b, y)
        assert_bits(host(y), orc.axpy(a, v["x"], b, v["p"]), f"axpy n={n} a={a} b={b}")
    # norm, dot
    assert_rel(bs.bs_norm(x).item(), orc.norm(v["x"]), f"norm n={n}")
    assert_rel(bs.bs_dot(x, p).item(), orc.dot(v["x"], v["p"]), f"dot n={n}")
    # fused update
    rr = bs.bs_cg_update(0.37, p, q, x, r).item()
    ox, orr_, orr = orc.cg_update(0.37, v["p"], v["q"], v["x"], v["r"])
    assert_bits(host(x), ox, f"cg x n={n}")
    assert_bits(host(r), orr_, f"cg r n={n}")
    assert_rel(rr, orr, f"cg rr n={n}")


@pytest.mark.parametrize("n", SIZES)
def test_vector_ops_sizes(env, n):
    run_vector_ops(env, n, 100 + n % 97)


@pytest.mark.parametrize("offset", [(1, 1, 1, 1), (1, 0, 1, 0), (0, 1, 1, 1), (1, 1, 0, 0)])
@pytest.mark.parametrize("n", [1, 2, 9, 4097, 100_003])
def test_vector_ops_alignment(env, n, offset):
    run_vector_ops(env, n, 300, offset)


def test_vector_ops_empty(env):
    bs, orc, torch, d = env
    e = torch.empty(0, dtype=torch.float64, device=d)
    out = torch.full((1,), 7.0, dtype=torch.float64, device=d)
    bs.bs_copy(e, e)
    bs.bs_axpy(1.0, e, 1.0, e)
    assert bs.bs_norm(e, out).item() == 0.0
    out.fill_(7.0)
    assert bs.bs_dot(e, e, out).item() == 0.0
    out.fill_(7.0)
    assert bs.bs_cg_update(0.5, e, e, e, e, out).item() == 0.0
    assert not math.copysign(1.0, out.item()) < 0


def test_copy_special_values(env):
    bs, orc, torch, d = env
    raw = np.array([0x7FF8_0000_DEAD_BEEF, 0x8000_0000_0000_0000, 0x7FF0_0000_0000_0000, 1, 0xFFF4_0000_0000_0001],
                   dtype=np.uint64)
    a = np.tile(raw, 1001).view(np.float64)
    y = torch.empty(a.size, dtype=torch.float64, device=d)
    bs.bs_copy(dev(torch, d, a), y)
    assert host(y).tobytes() == a.tobytes()


def test_copy_and_axpy_in_place(env):
    """x == y is allowed for copy (no change) and AXPY (y = (a y) + (b y))."""
    bs, orc, torch, d = env
    v = bs_inputs.uniform_pm1(12, 100_003)
    t = dev(torch, d, v)
    bs.bs_copy(t, t)
    assert_bits(host(t), v, "copy in place")
    bs.bs_axpy(0.37, t, 1.5, t)
    assert_bits(host(t), orc.axpy(0.37, v, 1.5, v), "axpy in place")


def test_axpy_beta_zero_reads_y(env):
    bs, orc, torch, d = env
    n = 5000
    x = bs_inputs.uniform_pm1(5, n)
    yv = bs_inputs.uniform_pm1(6, n)
    yv[[0, 17, 4999]] = [np.inf, np.nan, -np.inf]
    y = dev(torch, d, yv)
    bs.bs_axpy(2.0, dev(torch, d, x), 0.0, y)
    assert_bits(host(y), orc.axpy(2.0, x, 0.0, yv), "axpy beta=0")


def test_reductions_integer_data_bit_exact(env):
    """Integer-valued data sum exactly in any order: the GPU must match bits."""
    bs, orc, torch, d = env
    n = 5_000_011
    x = bs_inputs.small_ints(7, n, -30, 30)
    y = bs_inputs.small_ints(8, n, -30, 30)
    assert bs.bs_dot(dev(torch, d, x), dev(torch, d, y)).item() == float(
        np.dot(x.astype(np.int64), y.astype(np.int64)))
    s = int(np.dot(x.astype(np.int64), x.astype(np.int64)))
    assert bs.bs_norm(dev(torch, d, x)).item() == math.sqrt(s)
    assert bs.bs_norm(dev(torch, d, np.ones(1 << 22))).item() == 2048.0


def test_reductions_deterministic(env):
    bs, orc, torch, d = env
    n = 11_390_625
    x = dev(torch, d, bs_inputs.uniform_pm1(9, n))
    y = dev(torch, d, bs_inputs.uniform_pm1(10, n))
    a = [bs.bs_dot(x, y).item() for _ in range(3)]
    b = [bs.bs_norm(x).item() for _ in range(3)]
    assert len(set(a)) == 1 and len(set(b)) == 1


def test_one_kernel_reductions_back_to_back(env):
    """The reductions finish in the last block to arrive (an atomic ticket,
    partials through coherent agent-scope accesses). Queue many calls back to
    back with no synchronisation between them: six input sets of different
    values, grids of 1 to 512 blocks (one counter, and counters per group of
    blocks) interleaved so that every call follows one of another size and
    other values, each result in its own slot. Every result must match the
    oracle to 1e-12 and repeat bit for bit per input, which fails if a finish
    read a stale partial (of an earlier call, or from its own XCD's cache) or
    if a ticket counter was left nonzero."""
    bs, orc, torch, d = env
    sizes = [11_390_625, 3_000_001, 700_001, 9_000, 513, 3]
    vals = [{k: bs_inputs.uniform_pm1(4000 + 8 * i + j, n) for j, k in enumerate("xy")}
            for i, n in enumerate(sizes)]
    ref = [{"dot": orc.dot(v["x"], v["y"]), "norm": orc.norm(v["x"])} for v in vals]
    t = [{k: dev(torch, d, a) for k, a in v.items()} for v in vals]
    order = [(5 * i + i // 4) % len(sizes) for i in range(240)]
    out = torch.full((2 * len(order),), float("nan"), dtype=torch.float64, device=d)
    for i, s in enumerate(order):
        bs.bs_dot(t[s]["x"], t[s]["y"], out[2 * i:2 * i + 1])
        bs.bs_norm(t[s]["x"], out[2 * i + 1:2 * i + 2])
    torch.cuda.synchronize()
    got = host(out)
    first = {}
    for i, s in enumerate(order):
        for j, k in enumerate(("dot", "norm")):
            g = got[2 * i + j]
            assert_rel(g, ref[s][k], f"{k} call {i} size {sizes[s]}")
            assert first.setdefault((s, k), g) == g, f"{k} call {i} size {sizes[s]} not repeatable"


def test_one_kernel_cg_update_back_to_back(env):
    """As above for the fused update: alpha = 0 keeps x and r, so each call on
    a set returns that set's r.r; p and q are distinct arrays per set."""
    bs, orc, torch, d = env
    sizes = [11_390_625, 2_000_003, 9_000, 3]
    sets = []
    for i, n in enumerate(sizes):
        v = [bs_inputs.uniform_pm1(5000 + 8 * i + j, n) for j in range(4)]
        sets.append(([dev(torch, d, a) for a in v], orc.dot(v[3], v[3]), v))
    order = [(3 * i + i // 5) % len(sizes) for i in range(160)]
    out = torch.full((len(order),), float("nan"), dtype=torch.float64, device=d)
    for i, s in enumerate(order):
        p, q, x, r = sets[s][0]
        bs.bs_cg_update(0.0, p, q, x, r, out[i:i + 1])
    torch.cuda.synchronize()
    got = host(out)
    first = {}
    for i, s in enumerate(order):
        assert_rel(got[i], sets[s][1], f"rr call {i} size {sizes[s]}")
        assert first.setdefault(s, got[i]) == got[i], f"rr call {i} size {sizes[s]} not repeatable"
    for (tv, _, v) in sets:
        assert_bits(host(tv[2]), v[2], "x unchanged at alpha 0")
        assert_bits(host(tv[3]), v[3], "r unchanged at alpha 0")


@pytest.mark.parametrize("k", list(range(10, 29)))
def test_sweep_sizes(env, k):
    """The 2^10 .. 2^28 sweep: every op, whole vectors against the oracle."""
    bs, orc, torch, d = env
    n = 1 << k
    name = "sweep"
    v = bs_inputs.vectors(name, n, "xpqr")
    x, p, q, r = (dev(torch, d, v[c]) for c in "xpqr")
    y = torch.empty_like(x)
    bs.bs_copy(x, y)
    assert torch.equal(y, x)
    del y
    assert_rel(bs.bs_norm(x).item(), orc.norm(v["x"]), f"norm 2^{k}")
    assert_rel(bs.bs_dot(x, p).item(), orc.dot(v["x"], v["p"]), f"dot 2^{k}")
    rr = bs.bs_cg_update(0.37, p, q, x, r).item()
    ox, orr_, orr = orc.cg_update(0.37, v["p"], v["q"], v["x"], v["r"])
    assert_bits(host(x), ox, f"cg x 2^{k}")
    assert_bits(host(r), orr_, f"cg r 2^{k}")
    assert_rel(rr, orr, f"cg rr 2^{k}")
    bs.bs_axpy(0.37, p, 1.0, q)
    assert_bits(host(q), orc.axpy(0.37, v["p"], 1.0, v["q"]), f"axpy 2^{k}")


# ----------------------------------------------------- scatter / gather ----

MESHES = {
    "box8_N3": (8, 3),
    "box32_N7": (32, 7),
    "shuffled40_N5": (40, 5),
    "box24_N15": (24, 15),
}


def mesh_case(env, name):
    bs, orc, torch, d = env
    E, N = MESHES[name]
    ep, npm = bs_inputs.mesh_perms(name, E, N)
    l2g = bs.bs_mesh_box_l2g(E, E, E, N, ep, npm)
    ng = bs.bs_mesh_box_count(E, E, E, N)[1]
    off, ids = bs.bs_index_g2l(l2g, ng)
    ol2g, ong = orc.mesh_box(E, E, E, N, ep, npm)
    assert ong == ng
    return l2g, off, ids, ol2g, ng


@pytest.mark.parametrize("name", list(MESHES))
def test_scatter_gather_mesh(env, name):
    bs, orc, torch, d = env
    l2g, off, ids, ol2g, ng = mesh_case(env, name)
    nl = l2g.size
    b = bs_inputs.base_seed(name)
    vgv = bs_inputs.uniform_pm1(b + 1, ng)
    vlv = bs_inputs.uniform_pm1(b + 9, nl)
    # scatter
    vl = torch.empty(nl, dtype=torch.float64, device=d)
    bs.bs_scatter(dev(torch, d, l2g), dev(torch, d, vgv), vl)
    assert_bits(host(vl), orc.scatter(ol2g, vgv), f"scatter {name}")
    # gather, both kernels
    want = orc.gather(ol2g, vlv, ng)
    doff, dids, dvl = dev(torch, d, off), dev(torch, d, ids), dev(torch, d, vlv)
    vg = torch.full((ng,), np.nan, dtype=torch.float64, device=d)
    bs.bs_gather(doff, dids, dvl, vg)
    assert_bits(host(vg), want, f"gather rows {name}")
    for npb in (256, 512, 1024):
        plan = bs.bs_gather_plan(off, npb)
        vg.fill_(np.nan)
        bs.bs_gather(doff, dids, dvl, vg, dev(torch, d, plan))
        assert_bits(host(vg), want, f"gather lds {name} npb={npb}")


def test_gather_multiplicity_and_identity(env):
    """gather(1_L) is the node multiplicity; scatter(g) returns l2g."""
    bs, orc, torch, d = env
    l2g, off, ids, ol2g, ng = mesh_case(env, "box32_N7")
    m = np.diff(off).astype(np.float64)
    vg = torch.empty(ng, dtype=torch.float64, device=d)
    bs.bs_gather(dev(torch, d, off), dev(torch, d, ids), torch.ones(l2g.size, dtype=torch.float64, device=d), vg)
    assert_bits(host(vg), m, "gather(ones)")
    vl = torch.empty(l2g.size, dtype=torch.float64, device=d)
    bs.bs_scatter(dev(torch, d, l2g), torch.arange(ng, dtype=torch.float64, device=d), vl)
    assert_bits(host(vl), l2g.astype(np.float64), "scatter(arange)")


def test_masked_scatter_gather(env):
    bs, orc, torch, d = env
    E, N = 6, 4
    l2g = bs.bs_mesh_box_l2g(E, E, E, N).copy()
    ng = bs.bs_mesh_box_count(E, E, E, N)[1]
    ol2g, _ = orc.mesh_box(E, E, E, N)
    mask = bs_inputs.splitmix64(77, l2g.size) % np.uint64(5) == 0
    l2g[mask] = -1
    ol2g = ol2g.copy()
    ol2g[mask] = -3
    off, ids = bs.bs_index_g2l(l2g, ng)
    vgv = bs_inputs.uniform_pm1(78, ng)
    vl = torch.full((l2g.size,), np.nan, dtype=torch.float64, device=d)
    bs.bs_scatter(dev(torch, d, l2g), dev(torch, d, vgv), vl)
    got = host(vl)
    assert_bits(got, orc.scatter(ol2g, vgv), "masked scatter")
    assert not np.any(np.signbit(got[mask]))
    vlv = bs_inputs.uniform_pm1(79, l2g.size)
    want = orc.gather(ol2g, vlv, ng)
    for plan in (None, bs.bs_gather_plan(off, 1024)):
        vg = torch.full((ng,), np.nan, dtype=torch.float64, device=d)
        bs.bs_gather(dev(torch, d, off), dev(torch, d, ids), dev(torch, d, vlv), vg,
                     None if plan is None else dev(torch, d, plan))
        assert_bits(host(vg), want, "masked gather")


def test_gather_order_and_signed_zero(env):
    """Ascending local order from +0.0: (2^53, 1, 1, -2^53) sums to 0 (ties to
    even twice), rows of -0.0 give +0.0, empty rows give +0.0."""
    bs, orc, torch, d = env
    l2g = np.array([0, 2, 0, 2, 0, 0, 3, 3], dtype=np.int32)
    vlv = np.array([2.0 ** 53, -0.0, 1.0, -0.0, 1.0, -2.0 ** 53, 5.0, -5.0])
    ng = 5
    off, ids = bs.bs_index_g2l(l2g, ng)
    want = orc.gather(l2g, vlv, ng)
    assert list(want) == [0.0, 0.0, 0.0, 0.0, 0.0]
    for plan in (None, bs.bs_gather_plan(off, 3), bs.bs_gather_plan(off, 1024)):
        vg = torch.full((ng,), np.nan, dtype=torch.float64, device=d)
        bs.bs_gather(dev(torch, d, off), dev(torch, d, ids), dev(torch, d, vlv), vg,
                     None if plan is None else dev(torch, d, plan))
        assert_bits(host(vg), want, "order witness")


def test_gather_long_row_fallback(env):
    """A node with more entries than the LDS stage holds takes the direct path."""
    bs, orc, torch, d = env
    nl = 10_000
    l2g = np.zeros(nl, dtype=np.int32)
    l2g[::3] = 1
    l2g[1::7] = 2
    ng = 3
    vlv = bs_inputs.uniform_pm1(80, nl)
    off, ids = bs.bs_index_g2l(l2g, ng)
    want = orc.gather(l2g, vlv, ng)
    for plan in (None, bs.bs_gather_plan(off, 1024), bs.bs_gather_plan(off, 1)):
        vg = torch.empty(ng, dtype=torch.float64, device=d)
        bs.bs_gather(dev(torch, d, off), dev(torch, d, ids), dev(torch, d, vlv), vg,
                     None if plan is None else dev(torch, d, plan))
        assert_bits(host(vg), want, "long rows")


def test_gather_spans_at_and_over_capacity(env):
    """Without a plan the rows go in spans of 512: spans of exactly 2048
    entries are staged, spans of more take the global-memory path, and the
    spans are launched out of row order (runs per XCD over the whole rounds,
    the rest in order); every row gets the oracle's bits, also in the folded
    dot."""
    bs, orc, torch, d = env
    span, rows = 512, 79 * 512 + 300  # 80 spans: one round of 64 remapped, 16 in order
    length = np.empty(rows, dtype=np.int64)
    for s in range(80):
        length[s * span:(s + 1) * span] = [4, 5, 1, 8, 0, 3][s % 6]  # 2048, 2560, 512, 4096, 0, 1536
    l2g = np.repeat(np.arange(rows, dtype=np.int32), length)
    vlv = bs_inputs.uniform_pm1(86, l2g.size)
    wv = bs_inputs.uniform_pm1(87, rows)
    off, ids = bs.bs_index_g2l(l2g, rows)
    assert off[span] - off[0] == 2048 and off[2 * span] - off[span] == 2560
    want = orc.gather(l2g, vlv, rows)
    vg = torch.full((rows,), np.nan, dtype=torch.float64, device=d)
    doff, dids, dvl = dev(torch, d, off), dev(torch, d, ids), dev(torch, d, vlv)
    bs.bs_gather(doff, dids, dvl, vg)
    assert_bits(host(vg), want, "spans at and over capacity")
    vg.fill_(np.nan)
    got = bs.bs_gather_dot(doff, dids, dvl, vg, dev(torch, d, wv)).item()
    assert_bits(host(vg), want, "spans at and over capacity, folded dot")
    assert_rel(got, orc.dot(want, wv), "span gather dot")


def test_gather_span_over_capacity_on_a_long_box(env):
    """An 80 x 2 x 2 box at order 7: its interior line of element corners is
    561 rows long, so one 512-row span holds more entries than the span
    kernel stages (2120 > 2048) and goes through global memory, between
    spans that are staged; with and without a plan, the oracle's bits."""
    bs, orc, torch, d = env
    l2g = bs.bs_mesh_box_l2g(80, 2, 2, 7)
    ng = bs.bs_mesh_box_count(80, 2, 2, 7)[1]
    off, ids = bs.bs_index_g2l(l2g, ng)
    spans = np.diff(off[np.minimum(np.arange(0, ng + 512, 512), ng)])
    assert spans.max() > 2048 and (spans <= 2048).sum() > 200
    ol2g, _ = orc.mesh_box(80, 2, 2, 7)
    vlv = bs_inputs.uniform_pm1(88, l2g.size)
    want = orc.gather(ol2g, vlv, ng)
    for plan in (None, bs.bs_gather_plan(off, 1024)):
        vg = torch.full((ng,), np.nan, dtype=torch.float64, device=d)
        bs.bs_gather(dev(torch, d, off), dev(torch, d, ids), dev(torch, d, vlv), vg,
                     None if plan is None else dev(torch, d, plan))
        assert_bits(host(vg), want, f"long box, plan={plan is not None}")


def test_gather_plan_over_capacity_blocks(env):
    """A hand-made plan whose blocks exceed the LDS capacity (rows or
    entries) takes the global-memory path, with the same bits."""
    bs, orc, torch, d = env
    l2g = bs.bs_mesh_box_l2g(6, 6, 6, 3)
    ng = bs.bs_mesh_box_count(6, 6, 6, 3)[1]
    off, ids = bs.bs_index_g2l(l2g, ng)
    ol2g, _ = orc.mesh_box(6, 6, 6, 3)
    vlv = bs_inputs.uniform_pm1(85, l2g.size)
    want = orc.gather(ol2g, vlv, ng)
    starts = [np.array([0, ng], dtype=np.int32),
              np.array([0, 700, 2100, 2101, ng], dtype=np.int32),
              np.arange(0, ng + 1, dtype=np.int32)]
    for rows in starts:
        # blocks (first row, end row, first entry, end entry) in row order
        plan = np.stack([rows[:-1], rows[1:], off[rows[:-1]], off[rows[1:]]], axis=1).astype(np.int32)
        bs.bs_validate_plan(plan, off)
        vg = torch.full((ng,), np.nan, dtype=torch.float64, device=d)
        bs.bs_gather(dev(torch, d, off), dev(torch, d, ids), dev(torch, d, vlv), vg, dev(torch, d, plan))
        assert_bits(host(vg), want, f"plan with {rows.size - 1} blocks")


def test_scatter_ragged_and_misaligned(env):
    bs, orc, torch, d = env
    for nl in [1, 3, 5, 1023, 1025, 4097, 8191, 8193, 16383, 16384, 16385, 3 * 16384 + 77, 5 * 16384 - 1]:
        ng = 50
        l2g = (bs_inputs.splitmix64(81, nl) % np.uint64(ng)).astype(np.int32)
        vgv = bs_inputs.uniform_pm1(82, ng)
        want = orc.scatter(l2g, vgv)
        for o in (0, 1):
            ibuf = torch.zeros(nl + 4, dtype=torch.int32, device=d)
            ibuf[o:o + nl] = dev(torch, d, l2g)
            obuf = torch.zeros(nl + 4, dtype=torch.float64, device=d)
            bs.bs_scatter(ibuf[o:o + nl], dev(torch, d, vgv), obuf[o:o + nl])
            assert_bits(host(obuf[o:o + nl]), want, f"scatter nl={nl} o={o}")


def test_errors_enqueue_nothing(env):
    bs, orc, torch, d = env
    L, h = bs._lib(), bs.context().handle
    x = torch.zeros(10, dtype=torch.float64, device=d)
    raw = x.data_ptr()
    assert L.bs_copy(h, -1, raw, raw, None) == bs.BS_EINVAL
    assert L.bs_copy(h, 4, raw + 4, raw, None) == bs.BS_EALIGN
    assert L.bs_axpy(h, 4, 1.0, raw, 1.0, None, None) == bs.BS_EINVAL
    assert L.bs_scatter(h, 1 << 31, raw, raw, raw, None) == bs.BS_ERANGE
    assert L.bs_dot(h, 4, raw, raw, None, None) == bs.BS_EINVAL
    assert L.bs_gather(h, 4, raw, raw, raw, raw, raw, 0, None) == bs.BS_EINVAL
    with pytest.raises(TypeError):
        bs.bs_copy(x.float(), x.float())
    # operands that overlap where the call does not allow it (8 bytes a double)
    assert L.bs_copy(h, 4, raw, raw + 8, None) == bs.BS_EINVAL
    assert L.bs_axpy(h, 4, 1.0, raw + 16, 1.0, raw, None) == bs.BS_EINVAL
    assert L.bs_scale(h, 4, raw, raw + 40, raw + 32, None) == bs.BS_EINVAL
    o = raw + 72  # a device double for the residual, apart from the vectors
    assert L.bs_cg_update(h, 2, 1.0, raw, raw + 16, raw + 32, raw + 32, o, None) == bs.BS_EINVAL  # x == r
    assert L.bs_cg_update(h, 2, 1.0, raw, raw + 16, raw + 8, raw + 32, o, None) == bs.BS_EINVAL   # x meets p
    assert L.bs_cg_update(h, 2, 1.0, raw, raw + 16, raw + 32, raw + 24, o, None) == bs.BS_EINVAL  # r meets q
    torch.cuda.synchronize()
    assert torch.count_nonzero(x).item() == 0


def test_overlap_rules_of_the_iteration(env):
    """The CG iteration rejects overlapping vectors before it enqueues
    anything; the fused update takes p and q as one array."""
    bs, orc, torch, d = env
    L, h = bs._lib(), bs.context().handle
    E, N = 2, 2
    l2g = bs.bs_mesh_box_l2g(E, E, E, N)
    ng = bs.bs_mesh_box_count(E, E, E, N)[1]
    nl = l2g.size
    off, ids = bs.bs_index_g2l(l2g, ng)
    dl2g, doff, dids = dev(torch, d, l2g), dev(torch, d, off), dev(torch, d, ids)
    s = ng + (ng & 1)  # doubles per vector slot, keeping every slot 16-byte aligned
    buf = torch.zeros(4 * s + nl, dtype=torch.float64, device=d)  # x, r, p, q, p_local back to back
    base, hist = buf.data_ptr(), torch.zeros(4, dtype=torch.float64, device=d)
    x, r, p, q, pl = (base + 8 * s * k for k in range(5))

    def solve(*vecs):
        return L.bs_cg_solve(h, ng, nl, dl2g.data_ptr(), doff.data_ptr(), dids.data_ptr(), None, 0, *vecs, 3,
                             0.0, hist.data_ptr(), None)

    assert solve(x, r, p, q, q) == bs.BS_EINVAL       # p_local on q
    assert solve(x, x, p, q, pl) == bs.BS_EINVAL      # x == r
    assert solve(x, r, p, p + 16, pl) == bs.BS_EINVAL  # q shifted into p
    torch.cuda.synchronize()
    assert torch.count_nonzero(buf).item() == 0 and torch.count_nonzero(hist).item() == 0
    # p == q is allowed: both are only read
    v = bs_inputs.vectors("box8_N3", 4099)
    pp, xx, rr_ = dev(torch, d, v["p"]), dev(torch, d, v["x"]), dev(torch, d, v["r"])
    got = bs.bs_cg_update(0.37, pp, pp, xx, rr_).item()
    wx, wr, wrr = orc.cg_update(0.37, v["p"], v["p"], v["x"], v["r"])
    assert_bits(host(xx), wx, "x with p == q")
    assert_bits(host(rr_), wr, "r with p == q")
    assert_rel(got, wrr, "rr with p == q")


# ------------------------------------------------- CG streaming sequence ----

def test_cg_sequence_matches_oracle(env):
    """Four CG iterations on Z^T Z through the library vs the oracle."""
    bs, orc, torch, d = env
    E, N = 8, 3
    l2g = bs.bs_mesh_box_l2g(E, E, E, N)
    ng = bs.bs_mesh_box_count(E, E, E, N)[1]
    off, ids = bs.bs_index_g2l(l2g, ng)
    ol2g, _ = orc.mesh_box(E, E, E, N)
    b = bs_inputs.uniform_pm1(1001, ng)
    ox, orr_, ohist = orc.cg_sequence(ol2g, ng, b, 4)
    dl2g, doff, dids = dev(torch, d, l2g), dev(torch, d, off), dev(torch, d, ids)
    x = torch.zeros(ng, dtype=torch.float64, device=d)
    r = dev(torch, d, b)
    p = dev(torch, d, b)
    q = torch.empty_like(p)
    pl = torch.empty(l2g.size, dtype=torch.float64, device=d)
    rr = bs.bs_dot(r, r).item()
    hist = [rr]
    for _ in range(4):
        bs.bs_scatter(dl2g, p, pl)
        bs.bs_gather(doff, dids, pl, q)
        alpha = rr / bs.bs_dot(p, q).item()
        rr_new = bs.bs_cg_update(alpha, p, q, x, r).item()
        bs.bs_axpy(1.0, r, rr_new / rr, p)
        rr = rr_new
        hist.append(rr)
    check_cg(hist, ohist, host(x), ox, np.diff(off), b, 4, "host-driven CG")


# ----------------------------------------- gather + dot, device-resident CG ----

@pytest.mark.parametrize("name", ["box8_N3", "box32_N7"])
def test_gather_dot(env, name):
    """bs_gather_dot: the gather's bits unchanged, w . v_G to 1e-12."""
    bs, orc, torch, d = env
    l2g, off, ids, ol2g, ng = mesh_case(env, name)
    vlv = bs_inputs.uniform_pm1(86, l2g.size)
    wv = bs_inputs.uniform_pm1(87, ng)
    want = orc.gather(ol2g, vlv, ng)
    want_dot = orc.dot(want, wv)
    doff, dids, dvl, dw = dev(torch, d, off), dev(torch, d, ids), dev(torch, d, vlv), dev(torch, d, wv)
    for plan in (None, bs.bs_gather_plan(off, 1024)):
        vg = torch.full((ng,), np.nan, dtype=torch.float64, device=d)
        got = bs.bs_gather_dot(doff, dids, dvl, vg, dw, None if plan is None else dev(torch, d, plan)).item()
        assert_bits(host(vg), want, f"gather_dot values {name}")
        assert_rel(got, want_dot, f"gather_dot {name}")


@pytest.mark.parametrize("n", [1, 2, 3, 1000, 4097, 1_000_003, 11_390_625])
def test_scale_bit_exact(env, n):
    """bs_scale: y = x / d, one correctly rounded division per entry."""
    bs, orc, torch, d = env
    x = bs_inputs.uniform_pm1(211, n)
    dv = bs_inputs.uniform_pm1(212, n) + 1.5
    y = torch.empty(n, dtype=torch.float64, device=d)
    bs.bs_scale(dev(torch, d, x), dev(torch, d, dv), y)
    assert_bits(host(y), orc.scale(x, dv), f"scale n={n}")
    xt = dev(torch, d, x)
    bs.bs_scale(xt, dev(torch, d, dv), xt)  # in place
    assert_bits(host(xt), orc.scale(x, dv), f"scale in place n={n}")


@pytest.mark.parametrize("name", ["box8_N3", "box32_N7"])
def test_lumped_mass_and_inverse_scale(env, name):
    """m = Z^T w_L through bs_gather, then y = r / m through bs_scale, bit for
    bit against the oracle on the same weights; the library's own weights
    agree with the oracle's to rounding and sum to the box volume."""
    bs, orc, torch, d = env
    l2g, off, ids, ol2g, ng = mesh_case(env, name)
    E, N = MESHES[name]
    ow = orc.mesh_box_mass(E, E, E, N)
    lw = bs.bs_mesh_box_mass(E, E, E, N)
    assert np.allclose(lw, ow, rtol=1e-14, atol=0)
    want_m = orc.gather(ol2g, ow, ng)
    m = torch.empty(ng, dtype=torch.float64, device=d)
    bs.bs_gather(dev(torch, d, off), dev(torch, d, ids), dev(torch, d, ow), m,
                 dev(torch, d, bs.bs_gather_plan(off, 1024)))
    assert_bits(host(m), want_m, "lumped mass")
    assert abs(host(m).sum() - E ** 3) <= 1e-11 * E ** 3
    r = bs_inputs.uniform_pm1(213, ng)
    y = torch.empty(ng, dtype=torch.float64, device=d)
    bs.bs_scale(dev(torch, d, r), m, y)
    assert_bits(host(y), orc.scale(r, want_m), "r / m")


def cg_setup(env, name):
    bs, orc, torch, d = env
    l2g, off, ids, ol2g, ng = mesh_case(env, name)
    b = bs_inputs.uniform_pm1(bs_inputs.base_seed(name) + 3, ng)
    t = {"l2g": dev(torch, d, l2g), "off": dev(torch, d, off), "ids": dev(torch, d, ids),
         "plan": dev(torch, d, bs.bs_gather_plan(off, 1024)),
         "x": torch.zeros(ng, dtype=torch.float64, device=d), "r": dev(torch, d, b), "p": dev(torch, d, b),
         "q": torch.empty(ng, dtype=torch.float64, device=d),
         "pl": torch.empty(l2g.size, dtype=torch.float64, device=d)}
    return t, ol2g, ng, b


@pytest.mark.parametrize("name", ["box8_N3", "box32_N7"])
def test_cg_solve_matches_oracle(env, name):
    """Four device-resident CG iterations on Z^T Z against the oracle's CG
    (A = diag(m), m in {1,2,4,8}: exact CG converges in 4 steps): each
    residual within the first-order rounding bound of its own size, the
    converged one below the rounding floor, x per class (cg_bounds)."""
    bs, orc, torch, d = env
    t, ol2g, ng, b = cg_setup(env, name)
    ox, orr_, ohist = orc.cg_sequence(ol2g, ng, b, 4)
    m = np.diff(host(t["off"]))
    for plan in (None, t["plan"]):
        x, r, p = t["x"].clone(), t["r"].clone(), t["p"].clone()
        hist = bs.bs_cg_solve(t["l2g"], t["off"], t["ids"], x, r, p, t["q"], t["pl"], 4, 0.0, plan)
        check_cg(host(hist), ohist, host(x), ox, m, b, 4, f"{name} plan={plan is not None}")


def test_cg_solve_cache_resident_slab(env):
    """The CG iteration on one GPU's share of the 32^3 order-7 box (a
    32 x 32 x 4-element slab, 1.47M nodes): its vectors and tables, about
    87 MB, fit in the last-level cache, so the iteration runs the
    cache-keeping kernels, at full tiles and some two thousand gather blocks.
    Residual history and x against the oracle's CG, as for the boxes."""
    bs, orc, torch, d = env
    E, N = 32, 7
    l2g = bs.bs_mesh_box_l2g(E, E, 4, N)
    ng = bs.bs_mesh_box_count(E, E, 4, N)[1]
    off, ids = bs.bs_index_g2l(l2g, ng)
    ol2g, ong = orc.mesh_box(E, E, 4, N)
    assert ong == ng and np.array_equal(l2g, ol2g)
    working_set = 8 * (4 * ng + l2g.size) + 4 * (2 * l2g.size + ng + 1)
    assert working_set < 256 << 20
    b = bs_inputs.uniform_pm1(bs_inputs.base_seed("slab32x32x4_N7") + 3, ng)
    ox, _, ohist = orc.cg_sequence(ol2g, ng, b, 4)
    plan = dev(torch, d, bs.bs_gather_plan(off, 1024))
    dl2g, doff, dids = dev(torch, d, l2g), dev(torch, d, off), dev(torch, d, ids)
    x = torch.zeros(ng, dtype=torch.float64, device=d)
    r, p = dev(torch, d, b), dev(torch, d, b)
    q = torch.empty(ng, dtype=torch.float64, device=d)
    pl = torch.empty(l2g.size, dtype=torch.float64, device=d)
    h = host(bs.bs_cg_solve(dl2g, doff, dids, x, r, p, q, pl, 4, 0.0, plan))
    check_cg(h, ohist, host(x), ox, np.diff(off), b, 4, "slab")


@pytest.mark.parametrize("ex,ey,ez,N", [(1, 1, 1, 1), (3, 2, 5, 2), (7, 4, 3, 5), (10, 11, 9, 4), (13, 9, 12, 6),
                                         (24, 24, 24, 7), (24, 24, 24, 10)])
def test_cg_solve_boxes(env, ex, ey, ez, N):
    """The device CG on boxes of several shapes and orders, in all three of
    its cache regimes: the first boxes fit the 256 MB last-level cache whole;
    at 24^3 order 7 only r and p fit (77 MB), which the update hands to the
    direction update through the cache; at 24^3 order 10 (14.0M global
    nodes) r and p take 224 MB and every stream is non-temporal. Residual
    history and x against the oracle's CG, with and without a gather plan."""
    bs, orc, torch, d = env
    l2g = bs.bs_mesh_box_l2g(ex, ey, ez, N)
    ng = bs.bs_mesh_box_count(ex, ey, ez, N)[1]
    off, ids = bs.bs_index_g2l(l2g, ng)
    ol2g, _ = orc.mesh_box(ex, ey, ez, N)
    b = bs_inputs.uniform_pm1(9000 + ex * 1000 + ey * 100 + ez * 10 + N, ng)
    m = np.diff(off)
    iters = len(np.unique(m))
    ox, _, ohist = orc.cg_sequence(ol2g, ng, b, iters)
    dl2g, doff, dids = dev(torch, d, l2g), dev(torch, d, off), dev(torch, d, ids)
    q = torch.empty(ng, dtype=torch.float64, device=d)
    pl = torch.empty(l2g.size, dtype=torch.float64, device=d)
    for plan in (None, dev(torch, d, bs.bs_gather_plan(off, 1024))):
        x = torch.zeros(ng, dtype=torch.float64, device=d)
        r, p = dev(torch, d, b), dev(torch, d, b)
        h = host(bs.bs_cg_solve(dl2g, doff, dids, x, r, p, q, pl, iters, 0.0, plan))
        check_cg(h, ohist, host(x), ox, m, b, iters, f"box {ex}x{ey}x{ez} order {N} plan={plan is not None}")


def test_cg_solve_box24_N15(env):
    """The device CG on the 24^3 order-15 box (47.0M global nodes, 56.6M local
    entries), the mesh on which the benchmark times the CG iteration, in the
    benchmark's launch configuration (plan of 1024 entries per block; only
    r and p would not fit the last-level cache, so every stream is
    non-temporal). Four iterations against the oracle's CG within the derived
    bounds."""
    bs, orc, torch, d = env
    l2g, off, ids, ol2g, ng = mesh_case(env, "box24_N15")
    m = np.diff(off)
    assert sorted(set(m.tolist())) == [1, 2, 4, 8]
    b = bs_inputs.uniform_pm1(bs_inputs.base_seed("box24_N15") + 3, ng)
    print(f"box24_N15 CG: oracle ({ng} nodes)", flush=True)
    ox, _, ohist = orc.cg_sequence(ol2g, ng, b, 4)
    del ol2g
    dl2g, doff, dids = dev(torch, d, l2g), dev(torch, d, off), dev(torch, d, ids)
    plan = dev(torch, d, bs.bs_gather_plan(off, 1024))
    x = torch.zeros(ng, dtype=torch.float64, device=d)
    r, p = dev(torch, d, b), dev(torch, d, b)
    q = torch.empty(ng, dtype=torch.float64, device=d)
    pl = torch.empty(l2g.size, dtype=torch.float64, device=d)
    print("box24_N15 CG: device", flush=True)
    h = host(bs.bs_cg_solve(dl2g, doff, dids, x, r, p, q, pl, 4, 0.0, plan))
    check_cg(h, ohist, host(x), ox, m, b, 4, "box24_N15")


def test_cg_solve_early_exit_and_zero_iterations(env):
    """A tolerance stops the iteration on the device: later history entries
    stay -1 and x no longer changes; iters = 0 only measures rr0."""
    bs, orc, torch, d = env
    t, ol2g, ng, b = cg_setup(env, "box8_N3")
    x, r, p = t["x"].clone(), t["r"].clone(), t["p"].clone()
    hist = host(bs.bs_cg_solve(t["l2g"], t["off"], t["ids"], x, r, p, t["q"], t["pl"], 12, 1e-10, t["plan"]))
    done = [i for i in range(1, 13) if hist[i] >= 0]
    assert 1 <= len(done) <= 5 and done == list(range(1, len(done) + 1))
    assert np.all(hist[len(done) + 1:] == -1.0)
    assert math.sqrt(hist[len(done)] / hist[0]) <= 1e-10
    x2, r2, p2 = t["x"].clone(), t["r"].clone(), t["p"].clone()
    h0 = host(bs.bs_cg_solve(t["l2g"], t["off"], t["ids"], x2, r2, p2, t["q"], t["pl"], 0, 0.0, t["plan"]))
    assert h0.size == 1 and abs(h0[0] - orc.dot(b, b)) <= 1e-12 * orc.dot(b, b)
    assert torch.count_nonzero(x2).item() == 0
    # a zero right-hand side is converged before the first step
    z = torch.zeros_like(t["r"])
    hz = host(bs.bs_cg_solve(t["l2g"], t["off"], t["ids"], z.clone(), z.clone(), z.clone(), t["q"], t["pl"], 3,
                             0.0, t["plan"]))
    assert list(hz) == [0.0, -1.0, -1.0, -1.0]


# ------------------------------------------------ unstructured hex meshes ----

def unstructured_case(env, kind):
    """A mesh with arbitrary element orientation: the library builds the
    tables it runs on, the oracle builds its own from the same corners."""
    bs, orc, torch, d = env
    if kind.startswith("tet_split"):
        ev, nv, coords = bs_inputs.hex_tet_split(6, 5, 6)  # 4320 hexahedra, not a lattice
        N = 5
    else:
        ev, nv = bs_inputs.hex_box(16, 16, 12, periodic=(True, True, True))
        N = 7
    ev, _ = bs_inputs.hex_orient(ev, 701)
    if kind == "tet_split_curve":
        # stored along the library's Hilbert curve; both builders get the same corners
        ev = np.ascontiguousarray(ev[bs.bs_mesh_hex_order(coords[ev])])
    ev, nv = bs_inputs.hex_relabel(ev, nv, 702, spare=5)
    if kind == "tet_split_xcd":
        # eight regions of the generator's order interleaved in runs of 16 elements
        ev = np.ascontiguousarray(ev[bs.bs_mesh_xcd_interleave(len(ev), 16)])
    elif kind != "tet_split_curve":
        ev = ev[bs_inputs.permutation(703, len(ev))]
    l2g, ng = bs.bs_mesh_hex_l2g(ev, N, nv)
    off, ids = bs.bs_index_g2l(l2g, ng)
    ol2g, ong = orc.mesh_hex(ev, N, nv)
    assert ong == ng
    return l2g, off, ids, ol2g, ng


@pytest.mark.parametrize("kind", ["tet_split", "tet_split_curve", "tet_split_xcd", "torus"])
def test_unstructured_scatter_gather(env, kind):
    bs, orc, torch, d = env
    l2g, off, ids, ol2g, ng = unstructured_case(env, kind)
    vgv = bs_inputs.uniform_pm1(711, ng)
    vlv = bs_inputs.uniform_pm1(712, l2g.size)
    wv = bs_inputs.uniform_pm1(713, ng)
    vl = torch.empty(l2g.size, dtype=torch.float64, device=d)
    bs.bs_scatter(dev(torch, d, l2g), dev(torch, d, vgv), vl)
    assert_bits(host(vl), orc.scatter(ol2g, vgv), f"scatter {kind}")
    want = orc.gather(ol2g, vlv, ng)
    doff, dids, dvl = dev(torch, d, off), dev(torch, d, ids), dev(torch, d, vlv)
    plans = [None, bs.bs_gather_plan(off, 1024), bs.bs_gather_plan(off, 300)]
    if kind == "tet_split_xcd":  # blocks placed on the XCDs by region
        plans += [bs.bs_gather_plan(off, 1024, ids, 16 * 6 ** 3), bs.bs_gather_plan(off, 300, ids, 16 * 6 ** 3)]
    for plan in plans:
        dplan = None if plan is None else dev(torch, d, plan)
        vg = torch.full((ng,), np.nan, dtype=torch.float64, device=d)
        bs.bs_gather(doff, dids, dvl, vg, dplan)
        assert_bits(host(vg), want, f"gather {kind}")
        vg.fill_(np.nan)
        got = bs.bs_gather_dot(doff, dids, dvl, vg, dev(torch, d, wv), dplan).item()
        assert_bits(host(vg), want, f"gather_dot values {kind}")
        assert_rel(got, orc.dot(want, wv), f"gather_dot {kind}")


def test_unstructured_cg_solve(env):
    """Device-resident CG on Z^T Z = diag(m) of the tet-split mesh, whose
    multiplicities take many values: the residual history follows the
    oracle's CG while it is significant, and the iteration reaches b / m
    within one step per distinct multiplicity."""
    bs, orc, torch, d = env
    l2g, off, ids, ol2g, ng = unstructured_case(env, "tet_split")
    m = np.diff(off)
    iters = len(np.unique(m))
    b = bs_inputs.uniform_pm1(721, ng)
    ox, _, ohist = orc.cg_sequence(ol2g, ng, b, iters)
    t = {k: dev(torch, d, v) for k, v in (("l2g", l2g), ("off", off), ("ids", ids),
                                           ("plan", bs.bs_gather_plan(off, 1024)))}
    x = torch.zeros(ng, dtype=torch.float64, device=d)
    r, p = dev(torch, d, b), dev(torch, d, b)
    q = torch.empty(ng, dtype=torch.float64, device=d)
    pl = torch.empty(l2g.size, dtype=torch.float64, device=d)
    h = host(bs.bs_cg_solve(t["l2g"], t["off"], t["ids"], x, r, p, q, pl, iters, 0.0, t["plan"]))
    check_cg(h, ohist, host(x), ox, m, b, iters, "tet-split")


@pytest.mark.parametrize("order", ["gen", "curve", "xcd"])
def test_unstructured_cg_solve_handoff(env, order):
    """The device CG on the benchmark's tet-split mesh (11^3 cubes, 31944
    randomly oriented hexahedra, order 7: 11.1M global nodes). Its vectors and
    tables exceed the 256 MB last-level cache while r and p (177 MB) fit, so
    the update hands them to the direction update through the cache. Library
    and oracle build their own tables from the same corners; the residual
    history follows the oracle's CG and x reaches b / m. Elements in the
    generator's order, along the Hilbert curve, or interleaved by region for
    the XCDs with the gather plan placed by region (the benchmark's element
    orders)."""
    bs, orc, torch, d = env
    ev, nv, coords = bs_inputs.hex_tet_split(11, 11, 11)
    ev, _ = bs_inputs.hex_orient(ev, 731)
    N = 7
    region = 0
    if order == "curve":
        ev = np.ascontiguousarray(ev[bs.bs_mesh_hex_order(coords[ev])])
    elif order == "xcd":
        ev = np.ascontiguousarray(ev[bs.bs_mesh_xcd_interleave(len(ev), 64)])
        region = 64 * (N + 1) ** 3
    l2g, ng = bs.bs_mesh_hex_l2g(ev, N, nv)
    ol2g, ong = orc.mesh_hex(ev, N, nv)
    assert ong == ng and 16 * ng <= 210 << 20
    off, ids = bs.bs_index_g2l(l2g, ng)
    m = np.diff(off)
    iters = len(np.unique(m))
    b = bs_inputs.uniform_pm1(732, ng)
    ox, _, ohist = orc.cg_sequence(ol2g, ng, b, iters)
    t = {k: dev(torch, d, v) for k, v in (("l2g", l2g), ("off", off), ("ids", ids),
                                           ("plan", bs.bs_gather_plan(off, 1024, ids, region)))}
    x = torch.zeros(ng, dtype=torch.float64, device=d)
    r, p = dev(torch, d, b), dev(torch, d, b)
    q = torch.empty(ng, dtype=torch.float64, device=d)
    pl = torch.empty(l2g.size, dtype=torch.float64, device=d)
    h = host(bs.bs_cg_solve(t["l2g"], t["off"], t["ids"], x, r, p, q, pl, iters, 0.0, t["plan"]))
    check_cg(h, ohist, host(x), ox, m, b, iters, f"tet-split 11^3 order={order}")
    # scatter and gather on the same tables, as the benchmark launches them
    vgv = bs_inputs.uniform_pm1(733, ng)
    vl = torch.empty(l2g.size, dtype=torch.float64, device=d)
    bs.bs_scatter(t["l2g"], dev(torch, d, vgv), vl)
    assert_bits(host(vl), orc.scatter(ol2g, vgv), "scatter")
    vlv = bs_inputs.uniform_pm1(734, l2g.size)
    vg = torch.full((ng,), np.nan, dtype=torch.float64, device=d)
    bs.bs_gather(t["off"], t["ids"], dev(torch, d, vlv), vg, t["plan"])
    assert_bits(host(vg), orc.gather(ol2g, vlv, ng), "gather")


# -------------------------------------------------------- launch loop -----

def test_kernel_timing_events(env):
    """bs_ctx_time_next: the next kernel records the two events at its own
    start and end. Its duration lies inside what events recorded on the stream
    around the call measure; an operation that enqueues nothing leaves the
    context armed; the launch after the timed one does not touch the events;
    the timed launch computes the same result."""
    bs, orc, torch, d = env
    n = 11_390_625
    v = [bs_inputs.uniform_pm1(6100 + k, n) for k in range(4)]
    p, q, x, r = (dev(torch, d, a) for a in v)
    ctx = bs.context()
    st = torch.cuda.current_stream()
    k0, k1, s0, s1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    for e in (k0, k1):
        e.record(st)
    torch.cuda.synchronize()
    ctx.time_next(k0, k1)
    empty = torch.empty(0, dtype=torch.float64, device=d)
    bs.bs_copy(empty, empty)  # enqueues nothing: still armed
    s0.record(st)
    rr = bs.bs_cg_update(0.37, p, q, x, r)
    s1.record(st)
    torch.cuda.synchronize()
    kernel_ms, call_ms = k0.elapsed_time(k1), s0.elapsed_time(s1)
    assert 0.0 < kernel_ms <= call_ms * 1.02 + 1e-3, (kernel_ms, call_ms)
    ox, orr_, orr = orc.cg_update(0.37, v[0], v[1], v[2], v[3])
    assert_bits(host(x), ox, "timed cg x")
    assert_rel(rr.item(), orr, "timed cg rr")
    # disarmed: a later launch leaves the events as they were
    bs.bs_dot(p, q)
    torch.cuda.synchronize()
    assert k0.elapsed_time(k1) == kernel_ms
    ctx.time_next(k0, k1)
    ctx.time_next()  # disarm
    bs.bs_dot(p, q)
    torch.cuda.synchronize()
    assert k0.elapsed_time(k1) == kernel_ms


def test_bench_loop_runs_the_operations(env):
    """bs_bench_loop issues the real operations: after a loop over two sets
    the outputs are those of the last call on each set."""
    bs, orc, torch, d = env
    n = 100_003
    xs = [dev(torch, d, bs_inputs.uniform_pm1(731 + k, n)) for k in range(2)]
    ys = [dev(torch, d, bs_inputs.uniform_pm1(741 + k, n)) for k in range(2)]
    out = torch.zeros(1, dtype=torch.float64, device=d)
    t = bs.bs_bench_loop("norm", n, [(xs[0],), (xs[1],)], 5, out)
    assert t > 0
    assert_rel(out.item(), orc.norm(host(xs[0])), "norm via loop")  # call 4 used set 0
    ycopy = [torch.empty_like(x) for x in xs]
    bs.bs_bench_loop("copy", n, [(xs[0], ycopy[0]), (xs[1], ycopy[1])], 2)
    assert_bits(host(ycopy[0]), host(xs[0]), "copy via loop set 0")
    assert_bits(host(ycopy[1]), host(xs[1]), "copy via loop set 1")
    y0 = host(ys[0])
    bs.bs_bench_loop("axpy", n, [(xs[0], ys[0])], 1, alpha=0.37, beta=1.0)
    assert_bits(host(ys[0]), orc.axpy(0.37, host(xs[0]), 1.0, y0), "axpy via loop")
    with pytest.raises(bs.BSError):
        bs._check(bs._lib().bs_bench_loop(bs.context().handle, 9, n, 1.0, 1.0, 0, 1, None, None, 1, None,
                                           None), "bad op")
    with pytest.raises(ValueError):
        bs.bs_bench_loop("dot", n + 1, [(xs[0], ys[0])], 1, out)


def test_bench_loop_scatter_gather(env):
    """Scatter and gather through bs_bench_loop write what the direct calls
    write (both gather kernels), on the 8^3 order-3 box."""
    bs, orc, torch, d = env
    l2g, off, ids, ol2g, ng = mesh_case(env, "box8_N3")
    vgv = bs_inputs.uniform_pm1(751, ng)
    vlv = bs_inputs.uniform_pm1(752, l2g.size)
    vl = torch.empty(l2g.size, dtype=torch.float64, device=d)
    bs.bs_bench_loop("scatter", l2g.size, [(dev(torch, d, l2g), dev(torch, d, vgv), vl)], 3)
    assert_bits(host(vl), orc.scatter(ol2g, vgv), "scatter via loop")
    plan = bs.bs_gather_plan(off, 1024)
    want = orc.gather(ol2g, vlv, ng)
    for p in (None, dev(torch, d, plan)):
        vg = torch.full((ng,), np.nan, dtype=torch.float64, device=d)
        bs.bs_bench_loop("gather", ng, [(dev(torch, d, off), dev(torch, d, ids), dev(torch, d, vlv), vg, p)], 2,
                         n_blocks=0 if p is None else plan.shape[0])
        assert_bits(host(vg), want, "gather via loop")


# ------------------------------------------------- seeded random cases -----

def _draw(seed, k, lo, hi):
    """k integers in [lo, hi] from the seeded stream (inputs only)."""
    return [int(v) for v in (bs_inputs.splitmix64(seed, k) % np.uint64(hi - lo + 1)).astype(np.int64) + lo]


@pytest.mark.parametrize("case", range(24))
def test_random_vector_ops(env, case):
    """Lengths log-uniform in [1, 4M] and random 8-byte phases per operand."""
    w = _draw(900 + case, 6, 0, 2 ** 31)
    n = max(1, int(2 ** (22 * (w[0] / 2 ** 31))))
    offset = tuple(v % 2 for v in w[1:5])
    run_vector_ops(env, n, 1000 + case, offset)


@pytest.mark.parametrize("case", range(16))
def test_random_meshes(env, case):
    """Random box dimensions and orders, optional element and node
    permutations, optional Dirichlet masks, random blockStarts capacities:
    scatter, both gathers and the folded dot against the oracle."""
    bs, orc, torch, d = env
    ex, ey, ez, N, shuffle, masked, npb = _draw(950 + case, 7, 1, 1 << 30)
    ex, ey, ez = 1 + ex % 7, 1 + ey % 6, 1 + ez % 5
    N = 1 + N % 9
    G = (ex * N + 1) * (ey * N + 1) * (ez * N + 1)
    ep = bs_inputs.permutation(960 + case, ex * ey * ez) if shuffle % 2 else None
    npm = bs_inputs.permutation(970 + case, G) if shuffle % 3 == 0 else None
    l2g = bs.bs_mesh_box_l2g(ex, ey, ez, N, ep, npm).copy()
    ol2g, ng = orc.mesh_box(ex, ey, ez, N, ep, npm)
    assert np.array_equal(l2g, ol2g) and ng == G
    if masked % 2:
        m = bs_inputs.splitmix64(980 + case, l2g.size) % np.uint64(7) == 0
        l2g[m] = -1
        ol2g = ol2g.copy()
        ol2g[m] = -1
    off, ids = bs.bs_index_g2l(l2g, ng)
    vgv = bs_inputs.uniform_pm1(990 + case, ng)
    vlv = bs_inputs.uniform_pm1(995 + case, l2g.size)
    wv = bs_inputs.uniform_pm1(999 + case, ng)
    vl = torch.full((l2g.size,), np.nan, dtype=torch.float64, device=d)
    bs.bs_scatter(dev(torch, d, l2g), dev(torch, d, vgv), vl)
    assert_bits(host(vl), orc.scatter(ol2g, vgv), f"scatter case {case}")
    want = orc.gather(ol2g, vlv, ng)
    doff, dids, dvl, dw = dev(torch, d, off), dev(torch, d, ids), dev(torch, d, vlv), dev(torch, d, wv)
    # plans of several capacities, and one whose blocks launch in the
    # region order (any block order must give the same bits)
    region = 1 + (npb >> 10) % 5000
    plans = {None: None, 1 + npb % 1024: None, 1024: None, "region": bs.bs_gather_plan(off, 1024, ids, region)}
    for cap in plans:
        host_plan = plans[cap] if cap == "region" else None if cap is None else bs.bs_gather_plan(off, cap)
        if host_plan is not None:
            bs.bs_validate_plan(host_plan, off)
        plan = None if host_plan is None else dev(torch, d, host_plan)
        vg = torch.full((ng,), np.nan, dtype=torch.float64, device=d)
        bs.bs_gather(doff, dids, dvl, vg, plan)
        assert_bits(host(vg), want, f"gather case {case} cap {cap}")
        vg.fill_(np.nan)
        got = bs.bs_gather_dot(doff, dids, dvl, vg, dw, plan).item()
        assert_bits(host(vg), want, f"gather_dot values case {case} cap {cap}")
        assert_rel(got, orc.dot(want, wv), f"gather_dot case {case} cap {cap}")


@pytest.mark.parametrize("case", range(6))
def test_random_unstructured(env, case):
    """Tet-split and periodic meshes with random orientation, vertex names and
    element order at random orders: the library's table runs the kernels, the
    oracle's table the reference, and the two tables must be equal."""
    bs, orc, torch, d = env
    a, b, c, N, kind = _draw(1100 + case, 5, 1, 1 << 30)
    N = 1 + N % 8
    if kind % 2:
        ev, nv, _ = bs_inputs.hex_tet_split(1 + a % 3, 1 + b % 3, 1 + c % 2)
    else:
        ev, nv = bs_inputs.hex_box(3 + a % 3, 3 + b % 3, 3 + c % 3, periodic=(True, kind % 3 == 0, True))
    ev, _ = bs_inputs.hex_orient(ev, 1110 + case)
    ev, nv = bs_inputs.hex_relabel(ev, nv, 1120 + case, spare=case)
    ev = ev[bs_inputs.permutation(1130 + case, len(ev))]
    l2g, ng = bs.bs_mesh_hex_l2g(ev, N, nv)
    ol2g, ong = orc.mesh_hex(ev, N, nv)
    assert ng == ong and np.array_equal(l2g, ol2g)
    off, ids = bs.bs_index_g2l(l2g, ng)
    vgv = bs_inputs.uniform_pm1(1140 + case, ng)
    vlv = bs_inputs.uniform_pm1(1150 + case, l2g.size)
    vl = torch.empty(l2g.size, dtype=torch.float64, device=d)
    bs.bs_scatter(dev(torch, d, l2g), dev(torch, d, vgv), vl)
    assert_bits(host(vl), orc.scatter(ol2g, vgv), f"scatter unstructured {case}")
    want = orc.gather(ol2g, vlv, ng)
    region = (N + 1) ** 3 * (1 + a % 4)  # runs of 1-4 elements
    for plan in (None, bs.bs_gather_plan(off, 1024), bs.bs_gather_plan(off, 1024, ids, region)):
        vg = torch.full((ng,), np.nan, dtype=torch.float64, device=d)
        bs.bs_gather(dev(torch, d, off), dev(torch, d, ids), dev(torch, d, vlv), vg,
                     None if plan is None else dev(torch, d, plan))
        assert_bits(host(vg), want, f"gather unstructured {case}")


def test_contexts_on_concurrent_streams(env):
    """One context per stream: reductions issued alternately on two streams
    (default priority) with their own contexts keep their own partials, and
    each result matches the oracle."""
    bs, orc, torch, d = env
    n = 3_000_001
    xs = [bs_inputs.uniform_pm1(761 + k, n) for k in range(2)]
    X = [dev(torch, d, x) for x in xs]
    ctxs = [bs.Context(0), bs.Context(0)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.zeros(8, dtype=torch.float64, device=d) for _ in range(2)]
    torch.cuda.synchronize()
    for rep in range(8):
        for k in range(2):
            bs.bs_norm(X[k], outs[k][rep:rep + 1], ctx=ctxs[k], stream=streams[k])
    torch.cuda.synchronize()
    for k in range(2):
        want = orc.norm(xs[k])
        got = host(outs[k])
        assert np.all(got == got[0])
        assert_rel(got[0], want, f"stream {k}")
    for c in ctxs:
        c.close()
    # without explicit contexts the binding gives each stream its own shared one
    outs = [torch.zeros(8, dtype=torch.float64, device=d) for _ in range(2)]
    torch.cuda.synchronize()
    for rep in range(8):
        for k in range(2):
            bs.bs_norm(X[k], outs[k][rep:rep + 1], stream=streams[k])
    torch.cuda.synchronize()
    assert bs.context(0, streams[0]) is not bs.context(0, streams[1])
    for k in range(2):
        got = host(outs[k])
        assert np.all(got == got[0])
        assert_rel(got[0], orc.norm(xs[k]), f"shared context, stream {k}")


def test_unstructured_lumped_mass(env):
    """Lumped mass of the tet-split mesh (randomly oriented): m = Z^T w_L
    through both gathers bit for bit against the oracle on the oracle's
    weights; sum(m) = the volume of the box; r / m bit for bit; and the
    library's weights agree with the oracle's to rounding."""
    bs, orc, torch, d = env
    ev, nv, X = bs_inputs.hex_tet_split(5, 4, 3)
    ev, sym = bs_inputs.hex_orient(ev, 771)
    xe = bs_inputs.reorder_corners(X[bs_inputs.hex_tet_split(5, 4, 3)[0]], sym)
    assert np.array_equal(xe, X[ev])
    N = 5
    l2g, ng = bs.bs_mesh_hex_l2g(ev, N, nv)
    ol2g, _ = orc.mesh_hex(ev, N, nv)
    off, ids = bs.bs_index_g2l(l2g, ng)
    ow = orc.mesh_hex_mass(xe, N)
    assert np.allclose(bs.bs_mesh_hex_mass(xe, N), ow, rtol=1e-13, atol=0)
    want = orc.gather(ol2g, ow, ng)
    for plan in (None, bs.bs_gather_plan(off, 1024)):
        m = torch.empty(ng, dtype=torch.float64, device=d)
        bs.bs_gather(dev(torch, d, off), dev(torch, d, ids), dev(torch, d, ow), m,
                     None if plan is None else dev(torch, d, plan))
        assert_bits(host(m), want, "unstructured lumped mass")
    assert abs(host(m).sum() - 5 * 4 * 3) <= 1e-11 * 60
    r = bs_inputs.uniform_pm1(772, ng)
    y = torch.empty(ng, dtype=torch.float64, device=d)
    bs.bs_scale(dev(torch, d, r), m, y)
    assert_bits(host(y), orc.scale(r, want), "r / m unstructured")
