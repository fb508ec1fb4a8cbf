// bs_host.cpp -- host-side index tables for the scatter and gather operators.
//
// I_l->g of a structured box of hexahedra with (order+1)^3 Gauss-Lobatto
// nodes each ("Portable high-order finite element kernels I", arXiv
// 2009.10917, eqs. 1-3; "GPU accelerated spectral finite elements on all-hex
// meshes", arXiv 1506.05996, local-to-global table), its transpose in CSR
// form (the global-to-local table), and the blockStarts array of the
// LDS-staged gather (arXiv 2009.10917, implementation section, BS6).
//
// Because the GLL end points are the element corners, a node on an element
// face, edge or vertex coincides with the matching node of the neighbour.
// On the box this makes the global node lattice (E*order + 1) points per
// axis, and the node (i,j,k) of element (cx,cy,cz) the lattice point
// (cx*order + i, cy*order + j, cz*order + k): a closed form, no search.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "bs.h"

namespace {

bool is_permutation(const int32_t *p, int64_t n)
{
    std::vector<uint8_t> seen((size_t)n, 0);
    for (int64_t i = 0; i < n; ++i) {
        if (p[i] < 0 || p[i] >= n || seen[(size_t)p[i]]) return false;
        seen[(size_t)p[i]] = 1;
    }
    return true;
}

}  // namespace

extern "C" {

int bs_mesh_box_count(int ex, int ey, int ez, int order, int64_t *n_local, int64_t *n_global)
{
    if (ex < 1 || ey < 1 || ez < 1 || order < 1) return BS_EINVAL;
    const int64_t nq = (int64_t)order + 1;
    const int64_t K = (int64_t)ex * ey * ez;
    // guard the products against overflow before forming them
    if (nq > 2048 || K > (int64_t)INT32_MAX) return BS_ERANGE;
    const int64_t nl = K * nq * nq * nq;
    const int64_t gx = (int64_t)ex * order + 1, gy = (int64_t)ey * order + 1, gz = (int64_t)ez * order + 1;
    const int64_t ng = gx * gy * gz;
    if (nl > INT32_MAX || ng > INT32_MAX) return BS_ERANGE;
    if (n_local) *n_local = nl;
    if (n_global) *n_global = ng;
    return BS_OK;
}

int bs_mesh_box_l2g(int ex, int ey, int ez, int order, const int32_t *elem_perm, const int32_t *node_perm,
                    int32_t *l2g)
{
    int64_t nl, ng;
    if (int s = bs_mesh_box_count(ex, ey, ez, order, &nl, &ng)) return s;
    if (!l2g) return BS_EINVAL;
    const int64_t K = (int64_t)ex * ey * ez;
    if (elem_perm && !is_permutation(elem_perm, K)) return BS_EINVAL;
    if (node_perm && !is_permutation(node_perm, ng)) return BS_EINVAL;
    const int64_t nq = order + 1, Np = nq * nq * nq;
    const int64_t Gx = (int64_t)ex * order + 1, Gy = (int64_t)ey * order + 1;
    for (int64_t s = 0; s < K; ++s) {
        const int64_t e = elem_perm ? elem_perm[s] : s;
        const int64_t cx = e % ex, cy = (e / ex) % ey, cz = e / ((int64_t)ex * ey);
        int32_t *dst = l2g + s * Np;
        for (int64_t k = 0; k < nq; ++k) {
            const int64_t gz = cz * order + k;
            for (int64_t j = 0; j < nq; ++j) {
                const int64_t row = (gz * Gy + cy * order + j) * Gx + cx * order;
                for (int64_t i = 0; i < nq; ++i) {
                    const int64_t g = row + i;
                    dst[i + nq * (j + nq * k)] = node_perm ? node_perm[g] : (int32_t)g;
                }
            }
        }
    }
    return BS_OK;
}

int bs_gll(int order, double *nodes, double *weights)
{
    if (order < 1 || !nodes || !weights) return BS_EINVAL;
    const int n = order;
    // Legendre P_n and P_{n-1} at t by the three-term recurrence
    auto legendre = [n](double t, double &pn, double &pn1) {
        double a = 1.0, b = t;
        for (int k = 2; k <= n; ++k) {
            const double c = ((2.0 * k - 1.0) * t * b - (k - 1.0) * a) / k;
            a = b;
            b = c;
        }
        pn = (n == 0) ? 1.0 : b;
        pn1 = (n == 0) ? 0.0 : a;
    };
    // interior nodes: roots of q(t) = P_{n+1}(t) - P_{n-1}(t), which vanishes
    // exactly at the GLL points (q = (2n+1)/(n(n+1)) (t^2-1) P_n'(t)); Newton
    // with q'(t) = (2n+1) P_n(t), from the Chebyshev-Gauss-Lobatto points
    nodes[0] = -1.0;
    nodes[n] = 1.0;
    for (int i = 1; i < n; ++i) {
        double t = -std::cos(M_PI * i / n);
        for (int it = 0; it < 60; ++it) {
            double pn, pn1;
            legendre(t, pn, pn1);
            const double pn2 = ((2.0 * n + 1.0) * t * pn - n * pn1) / (n + 1.0);  // P_{n+1}
            const double q = pn2 - pn1;
            const double dq = (2.0 * n + 1.0) * pn;
            const double step = q / dq;
            t -= step;
            if (std::fabs(step) <= 4e-16 * std::fabs(t) + 1e-300) break;
        }
        nodes[i] = t;
    }
    for (int i = 0; i <= n; ++i) {
        double pn, pn1;
        legendre(nodes[i], pn, pn1);
        weights[i] = 2.0 / (n * (n + 1.0) * pn * pn);
    }
    return BS_OK;
}

int bs_mesh_box_mass(int ex, int ey, int ez, int order, double *w_local)
{
    int64_t nl, ng;
    if (int s = bs_mesh_box_count(ex, ey, ez, order, &nl, &ng)) return s;
    if (!w_local) return BS_EINVAL;
    const int64_t nq = order + 1, Np = nq * nq * nq, K = (int64_t)ex * ey * ez;
    std::vector<double> r(nq), w(nq), block(Np);
    bs_gll(order, r.data(), w.data());
    // one element's weights, w_i w_j w_k times the Jacobian 1/8 of the map
    // from [-1,1]^3 onto a unit cube; every element of the box is a unit cube
    for (int64_t k = 0; k < nq; ++k)
        for (int64_t j = 0; j < nq; ++j)
            for (int64_t i = 0; i < nq; ++i) block[i + nq * (j + nq * k)] = w[i] * w[j] * w[k] / 8.0;
    for (int64_t e = 0; e < K; ++e) std::memcpy(w_local + e * Np, block.data(), sizeof(double) * Np);
    return BS_OK;
}

int bs_validate_l2g(int64_t n_local, int64_t n_global, const int32_t *l2g)
{
    if (n_local < 0 || n_global < 0 || (n_local > 0 && !l2g)) return BS_EINVAL;
    for (int64_t i = 0; i < n_local; ++i)
        if (l2g[i] >= n_global) return BS_EINVAL;
    return BS_OK;
}

int bs_index_g2l(int64_t n_local, int64_t n_global, const int32_t *l2g, int32_t *off, int32_t *ids)
{
    if (n_local < 0 || n_global < 0 || !off || (n_local > 0 && (!l2g || !ids))) return BS_EINVAL;
    if (n_local > INT32_MAX || n_global >= INT32_MAX) return BS_ERANGE;
    // counting sort: histogram of ids, exclusive scan, then a stable fill in
    // ascending local index
    std::memset(off, 0, sizeof(int32_t) * (size_t)(n_global + 1));
    for (int64_t i = 0; i < n_local; ++i) {
        const int32_t g = l2g[i];
        if (g < 0) continue;
        if (g >= n_global) return BS_EINVAL;
        ++off[g + 1];
    }
    for (int64_t g = 0; g < n_global; ++g) off[g + 1] += off[g];
    std::vector<int32_t> cursor(off, off + n_global);
    for (int64_t i = 0; i < n_local; ++i) {
        const int32_t g = l2g[i];
        if (g >= 0) ids[cursor[(size_t)g]++] = (int32_t)i;
    }
    return BS_OK;
}

int bs_gather_plan(int64_t n_global, const int32_t *off, int nodes_per_block, int32_t *block_starts,
                   int64_t *n_blocks)
{
    if (n_global < 0 || !off || !block_starts || !n_blocks) return BS_EINVAL;
    if (nodes_per_block < 1 || nodes_per_block > 1024) return BS_EINVAL;
    if (n_global >= INT32_MAX) return BS_ERANGE;
    // greedy: extend the block row by row while it holds at most
    // nodes_per_block rows and nodes_per_block entries; a row longer than
    // that gets a block of its own
    int64_t nb = 0;
    int64_t g = 0;
    block_starts[0] = 0;
    while (g < n_global) {
        const int64_t start = off[g];
        int64_t end = g + 1;
        while (end < n_global && end - g < nodes_per_block && (int64_t)off[end + 1] - start <= nodes_per_block)
            ++end;
        block_starts[++nb] = (int32_t)end;
        g = end;
    }
    *n_blocks = nb;
    return BS_OK;
}

}  // extern "C"
