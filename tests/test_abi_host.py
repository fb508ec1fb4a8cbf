"""CPU tests of libbs: the exported C ABI, argument checks that fail before
any HIP call, and the host-side tables against the oracle's independent
builder (exact equality).

The host tables follow "GPU accelerated spectral finite elements on all-hex
meshes" (arXiv 1506.05996, local-to-global and global-to-local tables) and
the blockStarts array of "Portable high-order finite element kernels I"
(arXiv 2009.10917, implementation section, BS6).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import bs_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="session")
def bs():
    import cg_streaming_vector_amd as m
    if not os.path.exists(m.LIB_PATH):
        from cg_streaming_vector_amd import _build
        _build.build()
    m._lib()
    return m


def header_symbols():
    src = open(os.path.join(ROOT, "include", "bs.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bs_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol(bs):
    syms = header_symbols()
    assert len(syms) >= 17
    L = ctypes.CDLL(bs.LIB_PATH)
    for s in syms:
        assert hasattr(L, s), s
    # the binding declares exactly the header's entry points
    assert sorted(bs.SIGNATURES) == syms


def test_strerror_and_version(bs):
    L = bs._lib()
    assert L.bs_strerror(0) == b"ok"
    for code in (-1, -2, -3, -4, -5):
        assert L.bs_strerror(code) not in (b"ok", b"unknown status")
    assert L.bs_strerror(-99) == b"unknown status"
    assert L.bs_version() >= 100


def test_null_context_is_einval_before_any_hip_call(bs):
    L = bs._lib()
    assert L.bs_copy(None, 10, None, None, None) == bs.BS_EINVAL
    assert L.bs_axpy(None, 10, 1.0, None, 1.0, None, None) == bs.BS_EINVAL
    assert L.bs_norm(None, 10, None, None, None) == bs.BS_EINVAL
    assert L.bs_dot(None, 10, None, None, None, None) == bs.BS_EINVAL
    assert L.bs_cg_update(None, 10, 1.0, None, None, None, None, None, None) == bs.BS_EINVAL
    assert L.bs_scatter(None, 10, None, None, None, None) == bs.BS_EINVAL
    assert L.bs_gather(None, 10, None, None, None, None, None, 0, None) == bs.BS_EINVAL
    assert L.bs_gather_dot(None, 10, None, None, None, None, None, 0, None, None, None) == bs.BS_EINVAL
    assert L.bs_cg_solve(None, 10, 10, None, None, None, None, 0, None, None, None, None, None, 4, 0.0, None,
                         None) == bs.BS_EINVAL
    assert L.bs_cg_solve_static(10, 10, None, None, None, None, 0, None, None, None, None, None, 4, 0.0, None,
                                None) == bs.BS_EINVAL
    assert L.bs_bench_loop(None, 0, 10, 1.0, 1.0, 0, 1, None, None, 1, None, None) == bs.BS_EINVAL
    assert L.bs_ctx_create(0, None) == bs.BS_EINVAL
    assert L.bs_ctx_info(None, None, None, None) == bs.BS_EINVAL
    L.bs_ctx_destroy(None)


# ------------------------------------------------------------- mesh sizes --

def test_box_counts(bs):
    assert bs.bs_mesh_box_count(8, 8, 8, 3) == (32768, 15625)
    assert bs.bs_mesh_box_count(32, 32, 32, 7) == (16777216, 11390625)
    assert bs.bs_mesh_box_count(40, 40, 40, 5) == (13824000, 8120601)
    assert bs.bs_mesh_box_count(24, 24, 24, 15) == (56623104, 47045881)
    assert bs.bs_mesh_box_count(3, 2, 1, 2) == (6 * 27, 7 * 5 * 3)
    for bad in [(0, 1, 1, 1), (1, 1, 1, 0), (1, -2, 1, 3)]:
        with pytest.raises(bs.BSError) as e:
            bs.bs_mesh_box_count(*bad)
        assert e.value.status == bs.BS_EINVAL
    with pytest.raises(bs.BSError) as e:
        bs.bs_mesh_box_count(1000, 1000, 1000, 7)
    assert e.value.status == bs.BS_ERANGE


@pytest.mark.parametrize("dims", [(2 ** 21, 2 ** 21, 2 ** 21, 1), (2 ** 31 - 1, 2 ** 31 - 1, 2 ** 31 - 1, 1),
                                  (2 ** 16, 2 ** 16, 2 ** 16, 1), (2 ** 31 - 1, 1, 1, 1), (1, 1, 1, 2048),
                                  (1, 1, 1, 2 ** 31 - 1), (2 ** 30, 1, 1, 3), (1, 46341, 46341, 1),
                                  (1, 1, 1, 1290)])
def test_box_count_products_that_would_overflow(bs, dims):
    """Sizes whose element, local or global counts pass int32 (or whose
    products would pass int64 if formed) are refused, with nothing written."""
    L = bs._lib()
    nl, ng = ctypes.c_int64(-7), ctypes.c_int64(-7)
    assert L.bs_mesh_box_count(*dims, ctypes.byref(nl), ctypes.byref(ng)) == bs.BS_ERANGE
    assert nl.value == -7 and ng.value == -7


def test_box_count_at_the_int32_edge(bs):
    # boxes at the edge of int32 counts still fit
    assert bs.bs_mesh_box_count(1, 1, 1, 1289) == (1290 ** 3, 1290 ** 3)
    assert bs.bs_mesh_box_count(268435455, 1, 1, 1) == (8 * 268435455, 2 * 2 * 268435456)
    assert bs.bs_mesh_box_count(16383, 16383, 1, 1) == (8 * 16383 ** 2, 2 * 16384 ** 2)


# ------------------------------------------- tables against the oracle ----

@pytest.mark.parametrize("dims,N", [((1, 1, 1), 1), ((2, 2, 2), 2), ((3, 2, 4), 3), ((8, 8, 8), 3),
                                    ((5, 5, 5), 6), ((2, 3, 2), 15)])
def test_box_l2g_matches_oracle(bs, orc, dims, N):
    l2g = bs.bs_mesh_box_l2g(*dims, N)
    ol2g, ng = orc.mesh_box(*dims, N)
    assert np.array_equal(l2g, ol2g)
    assert ng == bs.bs_mesh_box_count(*dims, N)[1]


def test_box_shuffled_matches_oracle(bs, orc):
    E, N = 6, 5
    G = E * N + 1
    ep = bs_inputs.permutation(71, E ** 3)
    npm = bs_inputs.permutation(72, G ** 3)
    l2g = bs.bs_mesh_box_l2g(E, E, E, N, ep, npm)
    ol2g, _ = orc.mesh_box(E, E, E, N, ep, npm)
    assert np.array_equal(l2g, ol2g)


def test_box_rejects_non_permutations(bs):
    ep = np.arange(8, dtype=np.int32)
    ep[3] = 2
    with pytest.raises(bs.BSError):
        bs.bs_mesh_box_l2g(2, 2, 2, 1, ep, None)
    npm = np.arange(27, dtype=np.int32)
    npm[0] = 27
    with pytest.raises(bs.BSError):
        bs.bs_mesh_box_l2g(2, 2, 2, 1, None, npm)


@pytest.mark.slow
def test_full_size_tables_match_oracle(bs, orc):
    """The 32^3 order-7 box and the shuffled 40^3 order-5 box, exactly."""
    l2g = bs.bs_mesh_box_l2g(32, 32, 32, 7)
    ol2g, ng = orc.mesh_box(32, 32, 32, 7)
    assert np.array_equal(l2g, ol2g)
    off, ids = bs.bs_index_g2l(l2g, ng)
    ooff, oids = orc.g2l(ol2g, ng)
    assert np.array_equal(off, ooff) and np.array_equal(ids, oids)
    ep, npm = bs_inputs.mesh_perms("shuffled40_N5", 40, 5)
    l2g = bs.bs_mesh_box_l2g(40, 40, 40, 5, ep, npm)
    ol2g, ng = orc.mesh_box(40, 40, 40, 5, ep, npm)
    assert np.array_equal(l2g, ol2g)


@pytest.mark.parametrize("masked", [False, True])
def test_g2l_matches_oracle(bs, orc, masked):
    E, N = 5, 4
    ep = bs_inputs.permutation(73, E ** 3)
    npm = bs_inputs.permutation(74, (E * N + 1) ** 3)
    l2g, ng = orc.mesh_box(E, E, E, N, ep, npm)
    if masked:
        l2g = l2g.copy()
        l2g[bs_inputs.splitmix64(75, l2g.size) % np.uint64(7) == 0] = -1
    off, ids = bs.bs_index_g2l(l2g, ng)
    ooff, oids = orc.g2l(l2g, ng)
    assert np.array_equal(off, ooff)
    assert np.array_equal(ids, oids)


def test_g2l_rejects_out_of_range(bs):
    l2g = np.array([0, 1, 5], dtype=np.int32)
    with pytest.raises(bs.BSError):
        bs.bs_index_g2l(l2g, 5)
    with pytest.raises(bs.BSError):
        bs.bs_validate_l2g(l2g, 5)
    bs.bs_validate_l2g(l2g, 6)
    bs.bs_validate_l2g(np.array([-1, 2], dtype=np.int32), 3)


def plan_rule(off, npb):
    """blockStarts by the documented rule, written out row by row: the
    greedy end under both caps, then, for every block but the last, rounded
    down to a multiple of 16 rows when that keeps the block non-empty."""
    ng = len(off) - 1
    starts, a = [0], 0
    while a < ng:
        b = a + 1
        while b < ng and b - a < npb and off[b + 1] - off[a] <= npb:
            b += 1
        if b < ng and (b // 16) * 16 > a:
            b = (b // 16) * 16
        starts.append(b)
        a = b
    return starts


def plan_tiling(plan, off):
    """Row starts of a plan's blocks in row order, after checking each block's
    entries against the offsets and that the row ranges tile [0, n_global)."""
    ng = len(off) - 1
    assert plan.ndim == 2 and plan.shape[1] == 4
    assert np.array_equal(plan[:, 2], off[plan[:, 0]]) and np.array_equal(plan[:, 3], off[plan[:, 1]])
    rows = plan[np.argsort(plan[:, 0], kind="stable"), :2]
    assert rows[0, 0] == 0 and rows[-1, 1] == ng and np.array_equal(rows[1:, 0], rows[:-1, 1])
    assert np.all(rows[:, 1] > rows[:, 0])
    return list(rows[:, 0]) + [ng]


def runs_slots(nb):
    """Block (in row order) launched at each slot with runs of 8 per XCD: in
    round r of 64 blocks, XCD x's k-th slot, 64r + 8k + x, takes block
    64r + 8x + k; slots past the last whole round keep their own block."""
    out = list(range(nb))
    for r in range(nb // 64):
        for x in range(8):
            for k in range(8):
                out[64 * r + 8 * k + x] = 64 * r + 8 * x + k
    return out


@pytest.mark.parametrize("npb", [1, 8, 256, 512, 1000, 1024])
def test_gather_plan(bs, npb):
    l2g = bs.bs_mesh_box_l2g(6, 5, 4, 3)
    ng = bs.bs_mesh_box_count(6, 5, 4, 3)[1]
    off, _ = bs.bs_index_g2l(l2g, ng)
    blocks = bs.bs_gather_plan(off, npb)
    plan = np.asarray(plan_tiling(blocks, off))
    ent = off[plan[1:]] - off[plan[:-1]]
    rows = np.diff(plan)
    # never above the target unless the block is one long row
    assert np.all((ent <= npb) | (rows == 1))
    assert np.all(rows <= npb)
    # every inner boundary on a multiple of 16 rows where the block reaches one
    inner = plan[1:-1]
    assert np.all((inner % 16 == 0) | (inner // 16 * 16 <= plan[:-2]))
    assert list(plan) == plan_rule(off, npb)
    # launch order: runs of 8 blocks per XCD
    assert list(blocks[:, 0]) == [plan[b] for b in runs_slots(len(plan) - 1)]


def test_gather_plan_caps_rows(bs):
    # empty rows (fully masked nodes) still count against the row cap
    off = np.zeros(3001, dtype=np.int32)
    plan = bs.bs_gather_plan(off, 1024)
    assert plan.tolist() == [[0, 1024, 0, 0], [1024, 2048, 0, 0], [2048, 3000, 0, 0]]


def test_xcd_interleave(bs):
    """Region x takes the slots s with (s // chunk) % 8 == x and holds the
    next consecutive run of the given order there, in order."""
    for E, chunk in [(0, 4), (1, 1), (7, 1), (100, 3), (513, 64), (31944, 64), (1000, 200)]:
        perm = bs.bs_mesh_xcd_interleave(E, chunk)
        assert sorted(perm.tolist()) == list(range(E))
        slots = np.arange(E)
        expect_next = 0
        for x in range(8):
            got = perm[(slots // chunk) % 8 == x]
            assert np.array_equal(got, np.arange(expect_next, expect_next + got.size))
            expect_next += got.size
    with pytest.raises(bs.BSError):
        bs.bs_mesh_xcd_interleave(10, 0)
    # a run as long as the mesh or longer is the identity, up to the largest chunk
    for chunk in (100, 101, 2 ** 40, 2 ** 62, 2 ** 63 - 1):
        assert np.array_equal(bs.bs_mesh_xcd_interleave(100, chunk), np.arange(100))


def test_gather_plan_rejects_bad_offsets(bs):
    """Offsets that are not a CSR's, and a negative id where region placement
    reads one, are refused before any block is written."""
    for off in ([0, 3, 2, 5], [-1, 0, 1], [0, 1, 0]):
        with pytest.raises(bs.BSError):
            bs.bs_gather_plan(np.array(off, dtype=np.int32), 16)
    off = np.array([0, 1, 2, 3], dtype=np.int32)
    assert bs.bs_gather_plan(off, 16, np.array([0, 1, 2], dtype=np.int32), 1).shape == (1, 4)
    with pytest.raises(bs.BSError):
        bs.bs_gather_plan(off, 16, np.array([-5, 1, 2], dtype=np.int32), 1)


@pytest.mark.parametrize("chunk", [1, 4, 64])
def test_gather_plan_by_region(bs, chunk):
    """With the local layout interleaved by region, XCD x (the slots s with
    s % 8 == x) takes the blocks of region x in row order, and only as many
    slots go elsewhere as the regions' block counts differ."""
    ev, nv, _ = bs_inputs.hex_tet_split(4, 4, 4)
    ev, _ = bs_inputs.hex_orient(ev, 77)
    N = 3
    ev = np.ascontiguousarray(ev[bs.bs_mesh_xcd_interleave(len(ev), chunk)])
    l2g, ng = bs.bs_mesh_hex_l2g(ev, N, nv)
    off, ids = bs.bs_index_g2l(l2g, ng)
    region = chunk * (N + 1) ** 3
    for npb in (64, 1024):
        blocks = bs.bs_gather_plan(off, npb, ids, region)
        starts = plan_tiling(blocks, off)
        assert starts == plan_rule(off, npb)
        bs.bs_validate_plan(blocks, off)
        nb = len(blocks)
        reg = (ids[blocks[:, 2]] // region) % 8
        counts = np.bincount(reg, minlength=8)
        on_own = reg == np.arange(nb) % 8
        # every region's blocks go to its own XCD until that XCD's slots or
        # the region's blocks run out
        slots = np.bincount(np.arange(nb) % 8, minlength=8)
        assert on_own.sum() >= sum(min(int(c), int(t)) for c, t in zip(counts, slots)) - 8
        for x in range(8):
            mine = blocks[(np.arange(nb) % 8 == x) & on_own, 0]
            assert np.all(np.diff(mine) > 0)
    with pytest.raises(ValueError):
        bs.bs_gather_plan(off, 1024, None, region)


@pytest.mark.parametrize("p", [1, 2, 3, 4, 5, 7, 10, 15])
def test_gll_matches_oracle(bs, orc, p):
    """The library's GLL rule (Newton on P_{p+1} - P_{p-1}) and the oracle's
    (Newton on P_p' itself) are written independently; they agree to a few
    units in the last place."""
    r, w = bs.bs_gll(p)
    assert np.allclose(r, orc.gll_nodes(p), rtol=0, atol=4e-16)
    assert np.allclose(w, orc.gll_weights(p), rtol=4e-15, atol=0)
    assert r[0] == -1.0 and r[-1] == 1.0
    with pytest.raises(bs.BSError):
        bs.bs_gll(0)


def test_box_mass_matches_oracle(bs, orc):
    for dims, N in [((1, 1, 1), 1), ((3, 2, 4), 3), ((5, 5, 5), 7)]:
        w = bs.bs_mesh_box_mass(*dims, N)
        assert np.allclose(w, orc.mesh_box_mass(*dims, N), rtol=1e-14, atol=0)


def test_gather_plan_long_rows(bs):
    # one node with 10 entries, the rest single
    off = np.array([0, 1, 11, 12, 13], dtype=np.int32)
    plan = bs.bs_gather_plan(off, 4)
    assert plan.tolist() == [[0, 1, 0, 1], [1, 2, 1, 11], [2, 4, 11, 13]]
    with pytest.raises(bs.BSError):
        bs.bs_gather_plan(off, 0)
    with pytest.raises(bs.BSError):
        bs.bs_gather_plan(off, 1025)


# ------------------------------------------- unstructured hex meshes ------

def hex_meshes():
    """(name, ev, n_vert) of every family the generators make."""
    out = []
    ev, nv = bs_inputs.hex_box(4, 3, 2)
    out.append(("box", ev, nv))
    out.append(("box_oriented", bs_inputs.hex_orient(ev, 601)[0], nv))
    ev, nv = bs_inputs.hex_box(3, 4, 3, periodic=(True, True, True))
    out.append(("torus_oriented", bs_inputs.hex_orient(ev, 602)[0], nv))
    ev, nv = bs_inputs.hex_box(3, 3, 3, periodic=(True, False, True), twist=True)
    out.append(("twisted_oriented", bs_inputs.hex_orient(ev, 603)[0], nv))
    ev, nv, _ = bs_inputs.hex_tet_split(2, 2, 1)
    ev, _ = bs_inputs.hex_orient(ev, 604)
    ev, nv = bs_inputs.hex_relabel(ev, nv, 605, spare=11)
    out.append(("tet_split_oriented_relabeled", ev, nv))
    return out


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("mesh", hex_meshes(), ids=lambda m: m[0])
def test_hex_l2g_matches_oracle(bs, orc, mesh, N):
    """The library's topological builder (entity frames) and the oracle's
    symbolic trilinear weights are independent; both number by first
    appearance, so the tables must be identical."""
    _, ev, nv = mesh
    l2g, ng = bs.bs_mesh_hex_l2g(ev, N, nv)
    ol2g, ong = orc.mesh_hex(ev, N, nv)
    assert ng == ong
    assert np.array_equal(l2g, ol2g)


def test_hex_l2g_shuffled_elements(bs, orc):
    ev, nv, _ = bs_inputs.hex_tet_split(2, 1, 2)
    ev = ev[bs_inputs.permutation(606, len(ev))]
    l2g, ng = bs.bs_mesh_hex_l2g(ev, 4, nv)
    ol2g, ong = orc.mesh_hex(ev, 4, nv)
    assert ng == ong and np.array_equal(l2g, ol2g)


def test_hex_l2g_box_equals_box_builder(bs):
    """Same partition as the closed-form box builder (renamed by first
    appearance)."""
    ev, nv = bs_inputs.hex_box(5, 4, 3)
    l2g, ng = bs.bs_mesh_hex_l2g(ev, 4, nv)
    box = bs.bs_mesh_box_l2g(5, 4, 3, 4)
    assert ng == bs.bs_mesh_box_count(5, 4, 3, 4)[1]
    _, first, inv = np.unique(box, return_index=True, return_inverse=True)
    rank = np.empty(len(first), dtype=np.int64)
    rank[np.argsort(first)] = np.arange(len(first))
    assert np.array_equal(l2g, rank[inv.ravel()])


def test_hex_l2g_errors(bs):
    ev, nv = bs_inputs.hex_box(2, 1, 1)
    with pytest.raises(bs.BSError) as e:
        bs.bs_mesh_hex_l2g(ev, 0, nv)
    assert e.value.status == bs.BS_EINVAL
    bad = ev.copy()
    bad[0, 5] = bad[0, 2]
    with pytest.raises(bs.BSError):
        bs.bs_mesh_hex_l2g(bad, 2, nv)
    with pytest.raises(bs.BSError):
        bs.bs_mesh_hex_l2g(ev, 2, int(ev.max()))  # a vertex id out of range
    # the shared face x = 1 presented with two of its vertices swapped in the
    # second element: same four vertices, different quadrilateral
    twisted = ev.copy()
    a, b = twisted[1, 0], twisted[1, 2]  # corners (0,0,0) and (0,1,0): an edge
    twisted[1, 0], twisted[1, 2] = b, a
    a, b = twisted[1, 2], twisted[1, 6]  # then (0,1,0) <-> (0,1,1)
    twisted[1, 2], twisted[1, 6] = b, a
    with pytest.raises(bs.BSError) as e:
        bs.bs_mesh_hex_l2g(twisted, 2, nv)
    assert e.value.status == bs.BS_EINVAL
    with pytest.raises(bs.BSError) as e:
        bs.bs_mesh_hex_l2g(np.zeros((1, 8), np.int32) + np.arange(8, dtype=np.int32), 3000, 8)
    assert e.value.status == bs.BS_ERANGE
    l2g, ng = bs.bs_mesh_hex_l2g(np.zeros((0, 8), np.int32), 3, 0)
    assert l2g.size == 0 and ng == 0


# ------------------------------------------------ property-based tables ----

from hypothesis import given, settings, strategies as st  # noqa: E402


@settings(max_examples=60, deadline=None, derandomize=True)
@given(st.integers(0, 400), st.integers(1, 60), st.integers(0, 2 ** 32 - 1), st.integers(0, 4))
def test_g2l_property(bs, orc, n_local, n_global, seed, mask_mod):
    """Any I_l->g (random ids, optional masks): the library's counting-sort
    CSR equals the oracle's sort-based one."""
    ids = (bs_inputs.splitmix64(seed, n_local) % np.uint64(n_global)).astype(np.int32)
    if mask_mod:
        ids[bs_inputs.splitmix64(seed + 1, n_local) % np.uint64(mask_mod + 1) == 0] = -1
    off, got = bs.bs_index_g2l(ids, n_global)
    ooff, oids = orc.g2l(ids, n_global)
    assert np.array_equal(off, ooff) and np.array_equal(got, oids)


@settings(max_examples=60, deadline=None, derandomize=True)
@given(st.lists(st.integers(0, 40), min_size=0, max_size=300), st.integers(1, 1024))
def test_gather_plan_property(bs, rows, npb):
    """blockStarts of any row-length profile: covers every row once, in
    order, each block within both caps unless it is a single row, and greedy
    up to the 16-row rounding of every inner boundary; launched in runs of 8
    per XCD."""
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    blocks = bs.bs_gather_plan(off, npb)
    ng = len(rows)
    if ng == 0:
        assert blocks.shape == (0, 4)
        return
    plan = plan_tiling(blocks, off)
    for a, b in zip(plan[:-1], plan[1:]):
        ent, nr = off[b] - off[a], b - a
        assert nr == 1 or (ent <= npb and nr <= npb)
        if b < ng:
            # the greedy end g (the next row would break a cap) rounded down
            # to b = 16 k, or kept where no multiple of 16 follows row a
            g = b
            while g < ng and g - a < npb and off[g + 1] - off[a] <= npb:
                g += 1
            assert (b % 16 == 0 and b <= g < b + 16) or (b == g and g // 16 * 16 <= a)
    assert plan == plan_rule(off, npb)
    assert list(blocks[:, 0]) == [plan[b] for b in runs_slots(len(plan) - 1)]


def region_slots(off, ids, starts, region):
    """Launch order of plan blocks placed by region, as the rule states it:
    a block's region is that of its first entry's local index (an empty
    block's, its own index mod 8); slot s goes to XCD s mod 8, which takes
    its region's next block in row order, or, once that region has run out,
    the next block of the region with the most left (the lowest such
    region)."""
    nb = len(starts) - 1
    queues = [[] for _ in range(8)]
    for b in range(nb):
        e0, e1 = off[starts[b]], off[starts[b + 1]]
        x = (ids[e0] // region) % 8 if e1 > e0 else b % 8
        queues[x].append(b)
    out = []
    for s in range(nb):
        x = s % 8
        if not queues[x]:
            x = max(range(8), key=lambda y: (len(queues[y]), -y))
        out.append(queues[x].pop(0))
    return out


@settings(max_examples=80, deadline=None, derandomize=True)
@given(st.integers(0, 5000), st.integers(1, 700))
def test_xcd_interleave_property(bs, E, chunk):
    """Any element count and run length: a permutation in which slot s holds
    region (s // chunk) % 8, each region being the next consecutive run of
    the given order, kept in order."""
    perm = bs.bs_mesh_xcd_interleave(E, chunk)
    assert perm.size == E and np.array_equal(np.sort(perm), np.arange(E))
    region = (np.arange(E) // chunk) % 8
    nxt = 0
    for x in range(8):
        got = perm[region == x]
        assert np.array_equal(got, np.arange(nxt, nxt + got.size))
        nxt += got.size


@settings(max_examples=60, deadline=None, derandomize=True)
@given(st.lists(st.integers(0, 9), min_size=1, max_size=400), st.integers(1, 1024), st.integers(1, 50),
       st.integers(0, 2 ** 32 - 1))
def test_gather_plan_region_property(bs, rows, npb, region, seed):
    """Any row-length profile and any assignment of local indices to the
    entries: the plan's rows follow the greedy rule and its launch order
    follows the region rule exactly."""
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    ne = int(off[-1])
    ids = np.random.default_rng(seed).permutation(max(ne, 1))[:ne].astype(np.int32)
    blocks = bs.bs_gather_plan(off, npb, ids, region)
    starts = plan_tiling(blocks, off)
    assert starts == plan_rule(off, npb)
    assert list(blocks[:, 0]) == [starts[b] for b in region_slots(off, ids, starts, region)]


@settings(max_examples=25, deadline=None, derandomize=True)
@given(st.integers(1, 4), st.integers(1, 4), st.integers(1, 3), st.integers(1, 6), st.integers(0, 2 ** 32 - 1),
       st.booleans())
def test_hex_l2g_property(bs, orc, nx, ny, nz, N, seed, shuffle):
    """Random box dimensions and orders, every element in a random cube
    orientation, vertices renamed, elements optionally shuffled: library
    table == oracle table, and its node count is the lattice count."""
    ev, nv = bs_inputs.hex_box(nx, ny, nz)
    ev, _ = bs_inputs.hex_orient(ev, seed)
    ev, nv = bs_inputs.hex_relabel(ev, nv, seed + 1, spare=seed % 5)
    if shuffle:
        ev = ev[bs_inputs.permutation(seed + 2, len(ev))]
    l2g, ng = bs.bs_mesh_hex_l2g(ev, N, nv)
    ol2g, ong = orc.mesh_hex(ev, N, nv)
    assert ng == ong == (nx * N + 1) * (ny * N + 1) * (nz * N + 1)
    assert np.array_equal(l2g, ol2g)


@pytest.mark.parametrize("N", [1, 2, 4, 7])
def test_hex_mass_matches_oracle(bs, orc, N):
    """The library's weights (edge-vector Jacobian, scalar triple product) and
    the oracle's (shape-function derivatives, cofactor determinant) agree to
    rounding on oriented tet-split elements, affine boxes and a frustum."""
    ev, nv, X = bs_inputs.hex_tet_split(2, 1, 1)
    xe = bs_inputs.reorder_corners(X[ev], (bs_inputs.splitmix64(611, len(ev)) % np.uint64(48)).astype(np.int64))
    A = np.array([[1.1, 0.3, 0.0], [-0.2, 0.8, 0.1], [0.0, 0.4, 1.2]])
    boxes = bs_inputs.hex_box_coords(2, 2, 2) @ A.T
    s = 0.6
    frustum = np.array([[[0, 0, 0], [1, 0, 0], [0, 1, 0], [1, 1, 0],
                         [0, 0, 1], [s, 0, 1], [0, s, 1], [s, s, 1]]], dtype=np.float64)
    for geom in (xe, boxes, frustum):
        got = bs.bs_mesh_hex_mass(geom, N)
        want = orc.mesh_hex_mass(geom, N)
        assert np.allclose(got, want, rtol=1e-13, atol=0)


def test_hex_mass_errors(bs):
    xe = bs_inputs.hex_box_coords(1, 1, 1)
    with pytest.raises(bs.BSError):
        bs.bs_mesh_hex_mass(xe, 0)
    flat = xe.copy()
    flat[0, 4:, 2] = 0.0  # top face on the bottom face: det J = 0
    with pytest.raises(bs.BSError) as e:
        bs.bs_mesh_hex_mass(flat, 3)
    assert e.value.status == bs.BS_EINVAL
    tangled = xe.copy()
    tangled[0, 7] = (-1.0, -1.0, -1.0)  # far corner pulled through the element
    with pytest.raises(bs.BSError):
        bs.bs_mesh_hex_mass(tangled, 3)
    L = bs._lib()
    assert L.bs_mesh_hex_mass(1, 3, None, None) == bs.BS_EINVAL
    assert bs.bs_mesh_hex_mass(np.zeros((0, 8, 3)), 3).size == 0


# ------------------------------------------------------- table validators --

def _tables(bs, dims=(5, 4, 3), N=4):
    l2g = bs.bs_mesh_box_l2g(*dims, N)
    ng = bs.bs_mesh_box_count(*dims, N)[1]
    off, ids = bs.bs_index_g2l(l2g, ng)
    return l2g, ng, off, ids


def test_validate_g2l_accepts_built_tables(bs):
    l2g, ng, off, ids = _tables(bs)
    bs.bs_validate_g2l(off, ids, l2g.size)
    bs.bs_validate_g2l(off, ids, l2g.size, l2g)
    masked = l2g.copy()
    masked[::5] = -1
    moff, mids = bs.bs_index_g2l(masked, ng)
    bs.bs_validate_g2l(moff, mids, masked.size, masked)
    # an empty mesh
    bs.bs_validate_g2l(np.zeros(1, dtype=np.int32), np.zeros(0, dtype=np.int32), 0)


@pytest.mark.parametrize("fault", ["first_offset", "decreasing", "too_many", "id_negative", "id_high",
                                   "descending", "repeated", "wrong_row", "missing"])
def test_validate_g2l_rejects(bs, fault):
    l2g, ng, off, ids = _tables(bs)
    off, ids, nl = off.copy(), ids.copy(), l2g.size
    row = 37  # a row with several entries
    a, b = int(off[row]), int(off[row + 1])
    assert b - a >= 2
    use_l2g = False
    if fault == "first_offset":
        off[0] = 1
    elif fault == "decreasing":
        off[row + 1] = off[row] - 1
    elif fault == "too_many":
        nl = int(off[-1]) - 1
    elif fault == "id_negative":
        ids[a] = -1
    elif fault == "id_high":
        ids[a] = nl
    elif fault == "descending":
        ids[a], ids[a + 1] = ids[a + 1], ids[a]
    elif fault == "repeated":
        ids[a + 1] = ids[a]
    elif fault == "wrong_row":
        # a well-formed CSR that is not the transpose of this l2g
        j = int(off[row + 1])
        ids[a], ids[j] = ids[j], ids[a]
        ids[a:b] = np.sort(ids[a:b])
        use_l2g = True
    elif fault == "missing":
        # drop the last entry of the last row: still well formed, but not the whole transpose
        off[-1] -= 1
        use_l2g = True
    with pytest.raises(bs.BSError) as e:
        bs.bs_validate_g2l(off, ids, nl, l2g if use_l2g else None)
    assert e.value.status == bs.BS_EINVAL


def test_validate_plan(bs):
    l2g, ng, off, ids = _tables(bs)
    for npb in (1, 5, 300, 1024):
        bs.bs_validate_plan(bs.bs_gather_plan(off, npb), off)
    plan = bs.bs_gather_plan(off, 64)
    # any launch order is a plan
    bs.bs_validate_plan(plan[::-1].copy(), off)
    bad = [plan.copy() for _ in range(7)]
    bad[0][0, 1] = bad[0][0, 0]                   # an empty block
    bad[1][0, 2] += 1                             # an entry that is not off[row]
    bad[2][-1, 3] -= 1
    r = plan[:, 0].argsort()
    bad[3][r[1], 0] -= 1                          # two blocks overlap
    bad[3][r[1], 2] = off[bad[3][r[1], 0]]
    bad[4][r[1], 0] += 1                          # a gap between two blocks
    bad[4][r[1], 2] = off[bad[4][r[1], 0]]
    bad[5][1] = bad[5][0]                         # one block twice, another missing
    bad[6][r[-1], 1] = ng + 1                     # past the end
    for p in bad:
        with pytest.raises(bs.BSError):
            bs.bs_validate_plan(p, off)
    with pytest.raises(bs.BSError):  # a plan for other offsets
        off2 = off.copy()
        off2[5:] += 1
        bs.bs_validate_plan(plan, off2)
    with pytest.raises(ValueError):  # row starts alone are not a plan
        bs.bs_validate_plan(plan[:, 0].copy(), off)
    bs.bs_validate_plan(np.zeros((0, 4), dtype=np.int32), np.zeros(1, dtype=np.int32))
    L = bs._lib()
    assert L.bs_validate_plan(2 ** 31 - 1, off.ctypes.data, plan.ctypes.data, 1) == bs.BS_ERANGE
    assert L.bs_validate_plan(ng, off.ctypes.data, None, 1) == bs.BS_EINVAL
    assert L.bs_validate_plan(ng, None, plan.ctypes.data, 1) == bs.BS_EINVAL
    assert L.bs_validate_plan(ng, off.ctypes.data, plan.ctypes.data, ng + 1) == bs.BS_EINVAL


# --------------------------------------------- element order along a curve --

@pytest.mark.parametrize("n", [2, 4, 8, 16])
def test_hex_order_is_a_hilbert_walk_on_power_of_two_lattices(bs, n):
    """On a lattice of 2^k unit cubes the Hilbert curve visits the cubes one
    face neighbour after another (a Z-order curve would jump); the order is a
    permutation."""
    xe = bs_inputs.hex_box_coords(n, n, n)
    perm = bs.bs_mesh_hex_order(xe)
    assert np.array_equal(np.sort(perm), np.arange(n ** 3))
    c = xe.mean(axis=1)[perm]
    steps = np.abs(np.diff(c, axis=0)).sum(axis=1)
    assert np.all(steps == 1.0)


def test_hex_order_depends_only_on_the_centroids(bs):
    ev, nv, coords = bs_inputs.hex_tet_split(3, 3, 2)
    xe = coords[ev]
    perm = bs.bs_mesh_hex_order(xe)
    c = xe.mean(axis=1)
    # corners presented in other orders, elements shuffled: the same walk
    ev2, sym = bs_inputs.hex_orient(ev, 77)
    shuffle = bs_inputs.permutation(78, len(ev))
    xe2 = bs_inputs.reorder_corners(xe, sym)[shuffle]
    perm2 = bs.bs_mesh_hex_order(xe2)
    assert np.allclose(xe2.mean(axis=1)[perm2], c[perm], rtol=0, atol=1e-12)
    # it keeps neighbours closer than the generator's order does
    step = lambda cc: np.sqrt((np.diff(cc, axis=0) ** 2).sum(axis=1)).mean()  # noqa: E731
    assert step(c[perm]) < step(c)


def test_hex_order_edge_cases(bs):
    assert bs.bs_mesh_hex_order(np.zeros((0, 8, 3))).size == 0
    one = bs_inputs.hex_box_coords(1, 1, 1)
    assert list(bs.bs_mesh_hex_order(one)) == [0]
    same = np.repeat(one, 5, axis=0)  # all in one cell: the input order stays
    assert list(bs.bs_mesh_hex_order(same)) == [0, 1, 2, 3, 4]
    bad = bs_inputs.hex_box_coords(2, 1, 1)
    bad[1, 3, 2] = np.nan
    with pytest.raises(bs.BSError) as e:
        bs.bs_mesh_hex_order(bad)
    assert e.value.status == bs.BS_EINVAL
    L = bs._lib()
    assert L.bs_mesh_hex_order(3, None, None) == bs.BS_EINVAL
    assert L.bs_mesh_hex_order(-1, None, None) == bs.BS_EINVAL
