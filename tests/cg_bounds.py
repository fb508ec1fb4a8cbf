"""How far two floating-point runs of CG on A = Z^T Z may drift apart.

The device-resident CG and the oracle's CG ("Portable high-order finite
element kernels I", CG vector-operation list and the fused update of the BS
tests) run the same elementwise arithmetic; they differ only in how their
reductions (r.r and p.q) are summed. The GPU sums in a fixed tree, the
oracle with compensated Dot2, so each reduction differs by a relative amount
bounded by eta (the GPU's) plus the oracle's few ulps. Those differences
enter alpha and beta, and every later residual depends on them.

A = Z^T Z is diagonal with the node multiplicities m on its diagonal. On
each multiplicity class c (the nodes with m_i = lam_c) it acts as the scalar
lam_c, so CG started from r0 = p0 = b keeps every vector class-wise parallel
to b: r_k = rho_{k,c} b, p_k = pi_{k,c} b, x_k = xi_{k,c} b on class c, and
    r.r = sum_c rho_c^2 S_c,   p.q = sum_c lam_c pi_c^2 S_c,   S_c = sum_{i in c} b_i^2.
So the whole scalar recurrence is a J-dimensional one (J classes).

Every rounding of either run is a perturbation of that recurrence:
  - alpha_k carries the relative errors of two reductions and a division:
    |d alpha| <= 2 eta + u; beta_k likewise;
  - the elementwise updates r - RN(alpha q), RN(beta p) + r, x + RN(alpha p)
    and the gather's sum of lam_c equal terms (q) perturb each entry by at
    most a few u times the magnitudes involved. Only the component of such a
    perturbation along b (within its class) enters the later scalars to first
    order; its coefficient is bounded by the same relative size. The part
    orthogonal to b stays orthogonal (A is a scalar on the class) and adds to
    norms in squares; it is carried as a separate, feedback-free magnitude.
The first-order sensitivity of rr_k, rho_k and xi_k to each source is
computed by finite differences of the recurrence in 80-digit decimal
arithmetic (the recurrence is exact there, so only the injected perturbation
moves it). Summing |sensitivity| x bound over all sources gives, per step,
  rel_tol[k]: the largest relative difference |rr_a - rr_b| / rr_b that
              rounding can explain between runs with reduction bounds eta_a
              and eta_b (first order; meaningful while it is small);
  floor[k]:   an upper bound on a computed rr_k (for steps where exact CG has
              converged and only rounding noise is left);
  x_tol[c]:   per class, |x_a,i - x_b,i| <= x_tol[c] |b_i| after the last step;
  x_exact[c]: per class, |x_a,i - xi_c b_i| <= x_exact[c] |b_i| for run a alone,
              xi_c being exact CG's coefficient (1/lam_c once converged).
This is a first-order (linearised) bound: valid while rel_tol is well below
one, which the tests require before they compare two histories relatively.
"""
from __future__ import annotations

from decimal import Decimal, localcontext

import numpy as np

U = 2.0 ** -53
# Every reduction in these tests sums its terms along chains of at most 1024
# additions (per-lane accumulation, then wavefront, block and partials), so
# for nonnegative terms its relative error is at most 1024 u / (1 - 1024 u)
# (Higham, "Accuracy and Stability of Numerical Algorithms", ch. 4). The dot
# p.q of CG is a sum of nonnegative terms lam p_i^2 as well.
ETA_GPU = 1024 * U / (1 - 1024 * U)
# The oracle's Dot2 result, then its own final rounding.
ETA_ORACLE = 4 * U

_PREC = 80
_H = Decimal("1e-40")


def class_data(m, b):
    """Distinct multiplicities lam (ascending), the class of each node, and
    the class sums S_c of b_i^2."""
    m = np.asarray(m, dtype=np.int64)
    lam = np.nonzero(np.bincount(m))[0]
    lut = np.zeros(int(lam[-1]) + 1, dtype=np.int64)
    lut[lam] = np.arange(lam.size)
    inv = lut[m]
    b = np.asarray(b, dtype=np.float64)
    S = np.bincount(inv, weights=b * b, minlength=lam.size)
    return [float(v) for v in lam], inv, [float(s) for s in S]


def _run(lam, S, iters, pert=None):
    """The class-space CG recurrence with one injected perturbation.

    pert: (kind, k, c, size) or None. Kinds "alpha", "beta" multiply the
    scalar of step k by (1 + size); "r", "p", "x", "q" add size (an absolute
    coefficient amount) to class c's coefficient of that vector at step k.
    Returns (rr history [iters+1], rho per step, pi per step, xi per step,
    alpha per step, beta per step), all Decimal."""
    J = len(lam)
    L = [Decimal(v) for v in lam]
    Sd = [Decimal(v) for v in S]
    rho = [Decimal(1)] * J
    pi = [Decimal(1)] * J
    xi = [Decimal(0)] * J

    def add(kind, k, c):
        if pert and pert[0] == kind and pert[1] == k and pert[2] == c:
            return pert[3]
        return Decimal(0)

    def mul(kind, k):
        if pert and pert[0] == kind and pert[1] == k:
            return 1 + pert[3]
        return Decimal(1)

    rr = sum(rho[c] ** 2 * Sd[c] for c in range(J))
    hist, rhos, pis, xis, alphas, betas = [rr], [rho[:]], [pi[:]], [xi[:]], [], []
    for k in range(iters):
        q = [L[c] * pi[c] + add("q", k, c) for c in range(J)]
        pq = sum(pi[c] * q[c] * Sd[c] for c in range(J))
        if pq == 0 or rr == 0:
            alpha = Decimal(0)
        else:
            alpha = rr / pq * mul("alpha", k)
        xi = [xi[c] + alpha * pi[c] + add("x", k, c) for c in range(J)]
        rho = [rho[c] - alpha * q[c] + add("r", k, c) for c in range(J)]
        rr_new = sum(rho[c] ** 2 * Sd[c] for c in range(J))
        beta = (rr_new / rr * mul("beta", k)) if rr != 0 else Decimal(0)
        pi = [rho[c] + beta * pi[c] + add("p", k, c) for c in range(J)]
        rr = rr_new
        hist.append(rr)
        rhos.append(rho[:])
        pis.append(pi[:])
        xis.append(xi[:])
        alphas.append(alpha)
        betas.append(beta)
    return hist, rhos, pis, xis, alphas, betas


def _sources(lam, iters, base, eta):
    """Every rounding source of one run with reduction bound eta, and the
    bound on its size: (kind, k, c, bound)."""
    hist, rhos, pis, xis, alphas, betas = base
    J = len(lam)
    out = []
    for k in range(iters):
        out.append(("alpha", k, None, 2 * eta + U))
        out.append(("beta", k, None, 2 * eta + U))
        a, b_ = float(abs(alphas[k])), float(abs(betas[k]))
        for c in range(J):
            lc = lam[c]
            pc = float(abs(pis[k][c]))
            rc_new, xc_new = float(abs(rhos[k + 1][c])), float(abs(xis[k + 1][c]))
            qc = lc * pc
            # q = Z^T Z p: lam_c equal values summed left to right, each partial
            # sum rounded: at most (lam_c - 1) u lam_c |p|
            out.append(("q", k, c, (lc - 1) * U * qc))
            # r - RN(alpha q), rounded: u |alpha q| + u |r_new|
            out.append(("r", k, c, U * (a * qc + rc_new)))
            # RN(beta p) + r, rounded (1 r is exact): u |beta p| + u (|r| + |beta p|)
            out.append(("p", k, c, U * (rc_new + 2 * b_ * pc)))
            # x + RN(alpha p), rounded
            out.append(("x", k, c, U * (a * pc + xc_new)))
    return out


class CgBounds:
    """First-order drift bounds between two runs of CG on diag(lam) with
    class sums S (see the module docstring)."""

    def __init__(self, lam, S, iters, eta_a=ETA_GPU, eta_b=ETA_ORACLE):
        self.lam, self.S, self.iters = list(lam), list(S), int(iters)
        J = len(lam)
        with localcontext() as ctx:
            ctx.prec = _PREC
            base = _run(lam, S, iters)
            hist, rhos, pis, xis = base[0], base[1], base[2], base[3]
            self.rr_exact = [float(h) for h in hist]
            self.xi_exact = [float(v) for v in xis[-1]]
            # sensitivities of rr_k, rho_{k,c}, xi_{K,c} to each source (per unit size)
            sens = {}
            for src in _sources(lam, iters, base, ETA_GPU):
                kind, k, c, _ = src
                key = (kind, k, c)
                if key in sens:
                    continue
                h2 = _run(lam, S, iters, (kind, k, c, _H))
                sens[key] = ([(h2[0][j] - hist[j]) / _H for j in range(iters + 1)],
                             [[(h2[1][j][cc] - rhos[j][cc]) / _H for cc in range(J)] for j in range(iters + 1)],
                             [(h2[3][-1][cc] - xis[-1][cc]) / _H for cc in range(J)])

            def one_run(eta):
                """(drift of rr_k, drift of rho_{k,c}, drift of xi_{K,c}) of a
                run with reduction bound eta from exact CG, first order."""
                drr = [0.0] * (iters + 1)
                drho = [[0.0] * J for _ in range(iters + 1)]
                dxi = [0.0] * J
                for kind, k, c, size in _sources(lam, iters, base, eta):
                    s_rr, s_rho, s_xi = sens[(kind, k, c)]
                    for j in range(iters + 1):
                        drr[j] += float(abs(s_rr[j])) * size
                        for cc in range(J):
                            drho[j][cc] += float(abs(s_rho[j][cc])) * size
                    for cc in range(J):
                        dxi[cc] += float(abs(s_xi[cc])) * size
                # the reported rr_k is itself one more reduction
                drr = [drr[j] + eta * float(hist[j]) for j in range(iters + 1)]
                return drr, drho, dxi

            ra, rb = one_run(eta_a), one_run(eta_b)
            # components orthogonal to b inside each class: no scalar feedback,
            # propagated in magnitude (triangle inequality) with the exact scalars
            er = [0.0] * J
            ep = [0.0] * J
            ex = [0.0] * J
            orth_r = [[0.0] * J]
            srcs = _sources(lam, iters, base, max(eta_a, eta_b))
            by = {(kind, k, c): size for kind, k, c, size in srcs if c is not None}
            for k in range(iters):
                a, b_ = float(abs(base[4][k])), float(abs(base[5][k]))
                eq = [lam[c] * ep[c] + by[("q", k, c)] for c in range(J)]
                ex = [ex[c] + a * ep[c] + by[("x", k, c)] for c in range(J)]
                er = [er[c] + a * eq[c] + by[("r", k, c)] for c in range(J)]
                ep = [er[c] + b_ * ep[c] + by[("p", k, c)] for c in range(J)]
                orth_r.append(er[:])

        self.rel_tol = []
        for j in range(iters + 1):
            rr = self.rr_exact[j]
            self.rel_tol.append((ra[0][j] + rb[0][j]) / rr if rr > 0 else float("inf"))
        self.floor = []
        for j in range(iters + 1):
            par = sum((abs(float(rhos[j][c])) + max(ra[1][j][c], rb[1][j][c])) ** 2 * S[c] for c in range(J))
            orth = sum(orth_r[j][c] ** 2 * S[c] for c in range(J))
            self.floor.append((par + orth) * (1 + max(eta_a, eta_b)))
        self.x_tol = [ra[2][c] + rb[2][c] + 2 * ex[c] for c in range(J)]
        self.x_exact = [ra[2][c] + ex[c] for c in range(J)]

    def significant(self, k, limit=1e-3):
        """Is step k's relative comparison inside the first-order regime?"""
        return self.rel_tol[k] <= limit


def check_cg(h, ohist, x, ox, m, b, iters, what=""):
    """The whole comparison of a GPU CG run (history h, solution x) with the
    oracle's (ohist, ox) on A = diag(m) from r0 = p0 = b: every step inside
    the first-order regime relatively, the converged ones against the
    rounding floor, and x per class. Returns the bounds."""
    lam, cls, S = class_data(m, b)
    bounds = CgBounds(lam, S, iters)
    compared = check_history(h, ohist, bounds, what)
    assert compared and compared == list(range(len(compared))), f"{what}: steps compared {compared}"
    check_x(x, ox, b, cls, bounds, what)
    return bounds


def check_history(h, ohist, bounds, what=""):
    """GPU history h against the oracle's ohist: relative agreement within
    the derived bound while it is significant, below the rounding floor after
    exact CG has converged. Returns the steps compared relatively."""
    compared = []
    for k in range(bounds.iters + 1):
        if bounds.significant(k):
            tol = bounds.rel_tol[k]
            assert abs(h[k] - ohist[k]) <= tol * abs(ohist[k]), (
                f"{what} rr[{k}]: {h[k]!r} vs {ohist[k]!r}, rel {abs(h[k] - ohist[k]) / abs(ohist[k]):.3g} "
                f"> bound {tol:.3g}")
            compared.append(k)
        else:
            fl = bounds.floor[k]
            assert 0 <= h[k] <= fl and 0 <= ohist[k] <= fl, f"{what} rr[{k}]: {h[k]!r}, {ohist[k]!r} > floor {fl:.3g}"
    return compared


def check_x(x, ox, b, cls, bounds, what=""):
    """x of the GPU run against the oracle's x and against exact CG's x."""
    x, ox, b = (np.asarray(a, dtype=np.float64) for a in (x, ox, b))
    tol = np.asarray(bounds.x_tol)[cls] * np.abs(b)
    d = np.abs(x - ox)
    bad = np.nonzero(d > tol)[0]
    assert bad.size == 0, f"{what} x vs oracle: {bad.size} entries, worst {np.max(d - tol):.3g} over the bound"
    xe = np.asarray(bounds.xi_exact)[cls] * b
    # the exact coefficient itself is rounded once when formed in doubles
    tol_e = np.asarray(bounds.x_exact)[cls] * np.abs(b) + 2 * U * np.abs(xe)
    bad = np.nonzero(np.abs(x - xe) > tol_e)[0]
    assert bad.size == 0, f"{what} x vs exact CG: {bad.size} entries over the bound"
