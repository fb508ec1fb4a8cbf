"""The allocation-free CG solve (bs_cg_solve_static) against bs_cg_solve.

Both run the same kernels in the same order; only where the reduction
scratch lives differs (a static device array of the library against a
context's allocation), so x, r, p and the residual history must agree bit for
bit. Two calls in a row, the second on a smaller mesh, so the second finds
the first's leftovers in the shared static scratch; with and without a
gather plan; across the cache-keeping and the hand-off regimes of the
iteration. A gather with more blocks than the static scratch holds partials
is refused with nothing enqueued.
"""
import ctypes

import numpy as np
import pytest

import bs_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import cg_streaming_vector_amd as bs
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device")
    return bs, torch, torch.device("cuda:0")


def mesh(bs, torch, d, dims, N, seed, npb=1024):
    l2g = bs.bs_mesh_box_l2g(*dims, N)
    ng = bs.bs_mesh_box_count(*dims, N)[1]
    off, ids = bs.bs_index_g2l(l2g, ng)
    plan = bs.bs_gather_plan(off, npb)

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(d)
    return {"l2g": t(l2g), "off": t(off), "ids": t(ids), "plan": t(plan), "nb": plan.shape[0],
            "b": t(bs_inputs.uniform_pm1(seed, ng)), "ng": ng, "nl": l2g.size}


def solve(bs, torch, d, m, static, use_plan, iters):
    """One solve through the C ABI; returns (status, x, r, p, history)."""
    L = bs._lib()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    x = torch.zeros(m["ng"], dtype=torch.float64, device=d)
    r, p = m["b"].clone(), m["b"].clone()
    q = torch.empty(m["ng"], dtype=torch.float64, device=d)
    pl = torch.empty(m["nl"], dtype=torch.float64, device=d)
    h = torch.full((iters + 1,), np.nan, dtype=torch.float64, device=d)
    plan, nb = (P(m["plan"]), m["nb"]) if use_plan else (None, 0)
    args = (m["ng"], m["nl"], P(m["l2g"]), P(m["off"]), P(m["ids"]), plan, nb, P(x), P(r), P(p), P(q), P(pl),
            iters, 0.0, P(h), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if static:
        st = L.bs_cg_solve_static(*args)
    else:
        st = L.bs_cg_solve(bs.context().handle, *args)
    torch.cuda.synchronize()
    return st, x.cpu().numpy(), r.cpu().numpy(), p.cpu().numpy(), h.cpu().numpy()


def same_bits(a, b, what):
    assert np.array_equal(np.asarray(a).view(np.uint64), np.asarray(b).view(np.uint64)), what


@pytest.mark.parametrize("use_plan", [True, False])
def test_static_solve_matches_context_solve(env, use_plan):
    bs, torch, d = env
    # 24^3 order 7: r and p fit the last-level cache, the rest streams (hand-off
    # regime); then 8^3 order 3, whose whole iteration stays in the cache
    for dims, N, seed, iters in [((24, 24, 24), 7, 3101, 5), ((8, 8, 8), 3, 3102, 4)]:
        m = mesh(bs, torch, d, dims, N, seed)
        want = solve(bs, torch, d, m, False, use_plan, iters)
        got = solve(bs, torch, d, m, True, use_plan, iters)
        assert want[0] == 0 and got[0] == 0
        for k, name in enumerate(["x", "r", "p", "rr_hist"], start=1):
            same_bits(got[k], want[k], f"{name} {dims} order {N} plan={use_plan}")
        h = got[4]
        assert np.all(np.isfinite(h)) and h[0] > 0 and h[iters] <= 1e-20 * h[0]


def test_static_solve_refuses_more_gather_blocks_than_it_holds(env):
    bs, torch, d = env
    m = mesh(bs, torch, d, (16, 16, 16), 5, 3103, npb=1)  # one node per plan block: 531441 blocks
    assert m["nb"] > 1 << 17
    st, x, r, p, h = solve(bs, torch, d, m, True, True, 3)
    assert st == bs.BS_ERANGE
    assert np.all(x == 0) and np.all(np.isnan(h))  # nothing ran
    # the context's scratch holds them
    st, *_ = solve(bs, torch, d, m, False, True, 3)
    assert st == 0
    # and the static solve still works afterwards
    small = mesh(bs, torch, d, (4, 4, 4), 3, 3104)
    want, got = solve(bs, torch, d, small, False, True, 3), solve(bs, torch, d, small, True, True, 3)
    assert got[0] == 0
    same_bits(got[4], want[4], "rr_hist after a refused call")


def test_static_solve_under_graph_capture(env):
    """What the allocation-free solve is for: a caller that captures the solve
    into a HIP graph (nothing in it allocates, and its counters are cleared by
    a kernel, not a memset). The graph is replayed several times, with eager
    work (resetting x, r, p) and synchronisations between the replays; every
    replay matches the eager solve bit for bit."""
    bs, torch, d = env
    for dims, N, seed, iters in [((8, 8, 8), 3, 3201, 4), ((16, 16, 12), 5, 3202, 5)]:
        m = mesh(bs, torch, d, dims, N, seed)
        want = solve(bs, torch, d, m, True, True, iters)  # eager; also the first call's set-up
        assert want[0] == 0
        s = torch.cuda.Stream()
        x = torch.zeros(m["ng"], dtype=torch.float64, device=d)
        r, p = m["b"].clone(), m["b"].clone()
        q = torch.empty(m["ng"], dtype=torch.float64, device=d)
        pl = torch.empty(m["nl"], dtype=torch.float64, device=d)
        h = torch.empty(iters + 1, dtype=torch.float64, device=d)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            bs.bs_cg_solve_static(m["l2g"], m["off"], m["ids"], x, r, p, q, pl, iters, h,
                                  block_starts=m["plan"], stream=torch.cuda.current_stream())
        for rep in range(3):
            x.zero_()
            r.copy_(m["b"])
            p.copy_(m["b"])
            h.fill_(np.nan)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            same_bits(h.cpu().numpy(), want[4], f"rr_hist replay {rep} {dims}")
            same_bits(x.cpu().numpy(), want[1], f"x replay {rep} {dims}")
            same_bits(r.cpu().numpy(), want[2], f"r replay {rep} {dims}")
        del g
