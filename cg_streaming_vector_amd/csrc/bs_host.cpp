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
//
// On an unstructured mesh given by element corner vertices the same sharing
// is found topologically: a node on a vertex, edge or face belongs to that
// entity, whose nodes are laid out in a frame fixed by the entity's own
// vertex ids (an edge counted from its smaller vertex, a face from its
// smallest vertex towards the smaller neighbour), so every element that
// holds the entity, in whatever orientation, names its nodes alike.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "bs.h"

namespace {
// MI355X has eight XCDs; gather plans place their blocks for them.
constexpr int64_t kXcds = 8, kXcdRun = 8;
}  // namespace

namespace {

// Throws std::bad_alloc; every caller converts that into BS_ENOMEM.
bool is_permutation(const int32_t *p, int64_t n)
{
    std::vector<uint8_t> seen((size_t)n, 0);
    for (int64_t i = 0; i < n; ++i) {
        if (p[i] < 0 || p[i] >= n || seen[(size_t)p[i]]) return false;
        seen[(size_t)p[i]] = 1;
    }
    return true;
}

// A face of an element seen from the mesh: its four vertices sorted, and the
// vertex diagonally opposite the smallest one. Two elements share the face
// when the sorted quadruples agree; they agree on its shape only if the
// opposite vertex agrees too.
struct FaceKey {
    int32_t v[4];
    int32_t opposite;
    bool operator<(const FaceKey &o) const
    {
        for (int t = 0; t < 4; ++t)
            if (v[t] != o.v[t]) return v[t] < o.v[t];
        return opposite < o.opposite;
    }
    bool same_set(const FaceKey &o) const { return std::equal(v, v + 4, o.v); }
};

// Face of an element with the reference axis `a` fixed at `side`: its corner
// at face position (u, w) along the two other axes a1 < a2.
struct FaceFrame {
    int a, a1, a2, side;
    int corner(int u, int w) const { return (side << a) | (u << a1) | (w << a2); }
};

FaceFrame face_frame(int f)
{
    FaceFrame fr;
    fr.a = f >> 1;
    fr.side = f & 1;
    fr.a1 = fr.a == 0 ? 1 : 0;
    fr.a2 = fr.a == 2 ? 1 : 2;
    return fr;
}

FaceKey face_key(const int32_t *v, int f)
{
    const FaceFrame fr = face_frame(f);
    FaceKey k;
    int32_t q[2][2];
    for (int u = 0; u < 2; ++u)
        for (int w = 0; w < 2; ++w) q[u][w] = v[fr.corner(u, w)];
    int ua = 0, wa = 0;
    for (int u = 0; u < 2; ++u)
        for (int w = 0; w < 2; ++w)
            if (q[u][w] < q[ua][wa]) ua = u, wa = w;
    k.v[0] = q[0][0], k.v[1] = q[0][1], k.v[2] = q[1][0], k.v[3] = q[1][1];
    std::sort(k.v, k.v + 4);
    k.opposite = q[1 - ua][1 - wa];
    return k;
}

// Bits per axis of the Hilbert curve that orders elements: 3 x 21 = 63 bits.
constexpr int kHilbertBits = 21;

// Position along the 3D Hilbert curve of the cell with integer coordinates
// X (each below 2^kHilbertBits), after J. Skilling, "Programming the Hilbert
// curve" (AIP Conf. Proc. 707, 2004): the coordinates are transformed in
// place into the "transposed" curve index (a sequence of inversions and
// exchanges of their low bits, level by level from the top, then a Gray
// code), whose bits, read across the three words from the most significant
// level down, form the index.
uint64_t hilbert_index(uint32_t X[3])
{
    constexpr uint32_t top = 1u << (kHilbertBits - 1);
    for (uint32_t Q = top; Q > 1; Q >>= 1) {
        const uint32_t P = Q - 1;
        for (int i = 0; i < 3; ++i) {
            if (X[i] & Q) {
                X[0] ^= P;  // invert the low bits of the first axis
            } else {
                const uint32_t t = (X[0] ^ X[i]) & P;  // exchange low bits with it
                X[0] ^= t;
                X[i] ^= t;
            }
        }
    }
    for (int i = 1; i < 3; ++i) X[i] ^= X[i - 1];
    uint32_t t = 0;
    for (uint32_t Q = top; Q > 1; Q >>= 1)
        if (X[2] & Q) t ^= Q - 1;
    for (int i = 0; i < 3; ++i) X[i] ^= t;
    uint64_t key = 0;
    for (int j = kHilbertBits - 1; j >= 0; --j)
        for (int i = 0; i < 3; ++i) key = key << 1 | ((X[i] >> j) & 1u);
    return key;
}

}  // namespace

extern "C" {

int bs_mesh_hex_order(int64_t n_elements, const double *xe, int32_t *perm)
{
    if (n_elements < 0 || (n_elements > 0 && (!xe || !perm))) return BS_EINVAL;
    if (n_elements > INT32_MAX) return BS_ERANGE;
    const int64_t E = n_elements;
    try {
        std::vector<double> c((size_t)E * 3);
        double lo[3] = {INFINITY, INFINITY, INFINITY}, hi[3] = {-INFINITY, -INFINITY, -INFINITY};
        for (int64_t e = 0; e < E; ++e) {
            for (int a = 0; a < 3; ++a) {
                double s = 0.0;
                for (int k = 0; k < 8; ++k) s += xe[24 * e + 3 * k + a];
                s /= 8.0;
                if (!std::isfinite(s)) return BS_EINVAL;
                c[(size_t)(3 * e + a)] = s;
                lo[a] = std::min(lo[a], s);
                hi[a] = std::max(hi[a], s);
            }
        }
        // one scale for all axes (cubic cells) over the widest extent
        double extent = 0.0;
        for (int a = 0; a < 3; ++a) extent = std::max(extent, hi[a] - lo[a]);
        const double cells = (double)((1u << kHilbertBits) - 1);
        const double scale = extent > 0.0 ? cells / extent : 0.0;
        std::vector<std::pair<uint64_t, int32_t>> key((size_t)E);
        for (int64_t e = 0; e < E; ++e) {
            uint32_t X[3];
            for (int a = 0; a < 3; ++a) {
                const double q = std::floor((c[(size_t)(3 * e + a)] - lo[a]) * scale);
                X[a] = (uint32_t)std::min(std::max(q, 0.0), cells);
            }
            key[(size_t)e] = {hilbert_index(X), (int32_t)e};
        }
        // ties (equal cells) keep the elements' own order
        std::sort(key.begin(), key.end());
        for (int64_t s = 0; s < E; ++s) perm[s] = key[(size_t)s].second;
    } catch (const std::bad_alloc &) {
        return BS_ENOMEM;
    }
    return BS_OK;
}

int bs_mesh_box_count(int ex, int ey, int ez, int order, int64_t *n_local, int64_t *n_global)
{
    if (ex < 1 || ey < 1 || ez < 1 || order < 1) return BS_EINVAL;
    // Every product below is bounded before it is formed, so none can
    // overflow int64: a dimension times the order stays within int32, and
    // each running product is compared with INT32_MAX divided by the next
    // factor.
    const int64_t lim = INT32_MAX;
    if (order > 2047) return BS_ERANGE;
    if (ex > lim / order || ey > lim / order || ez > lim / order) return BS_ERANGE;
    const int64_t nq = (int64_t)order + 1, np = nq * nq * nq;  // np < 2^33
    const int64_t exy = (int64_t)ex * ey;                       // < 2^62
    if (exy > lim / ez) return BS_ERANGE;
    const int64_t K = exy * ez;  // <= INT32_MAX
    if (K > lim / np) return BS_ERANGE;
    const int64_t nl = K * np;
    const int64_t gx = (int64_t)ex * order + 1, gy = (int64_t)ey * order + 1, gz = (int64_t)ez * order + 1;
    const int64_t gxy = gx * gy;  // each factor <= 2^31, so < 2^62
    if (gxy > lim / gz) return BS_ERANGE;
    const int64_t ng = gxy * gz;
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
    try {
        if (elem_perm && !is_permutation(elem_perm, K)) return BS_EINVAL;
        if (node_perm && !is_permutation(node_perm, ng)) return BS_EINVAL;
    } catch (const std::bad_alloc &) {
        return BS_ENOMEM;
    }
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

int bs_mesh_hex_l2g(int64_t n_elements, int order, int64_t n_vertices, const int32_t *ev, int32_t *l2g,
                    int64_t *n_global)
{
    if (n_elements < 0 || order < 1 || n_vertices < 0 || !n_global) return BS_EINVAL;
    if (n_elements > 0 && (!ev || !l2g)) return BS_EINVAL;
    const int64_t N = order, nq = N + 1;
    if (nq > 2048) return BS_ERANGE;
    const int64_t Np = nq * nq * nq;
    if (n_elements > INT32_MAX / Np || n_vertices > INT32_MAX) return BS_ERANGE;
    const int64_t E = n_elements;
    for (int64_t e = 0; e < E; ++e) {
        const int32_t *v = ev + 8 * e;
        for (int c = 0; c < 8; ++c) {
            if (v[c] < 0 || v[c] >= n_vertices) return BS_EINVAL;
            for (int c2 = 0; c2 < c; ++c2)
                if (v[c2] == v[c]) return BS_EINVAL;
        }
    }
    try {
        // Entities shared between elements: edges by their two vertices,
        // faces by their four. Sort and deduplicate the keys of all elements.
        std::vector<uint64_t> edges;
        edges.reserve((size_t)E * 12);
        std::vector<FaceKey> faces;
        faces.reserve((size_t)E * 6);
        for (int64_t e = 0; e < E; ++e) {
            const int32_t *v = ev + 8 * e;
            for (int a = 0; a < 3; ++a)
                for (int c = 0; c < 8; ++c) {
                    if ((c >> a) & 1) continue;
                    const uint32_t x = (uint32_t)v[c], y = (uint32_t)v[c | 1 << a];
                    edges.push_back((uint64_t)std::min(x, y) << 32 | std::max(x, y));
                }
            for (int f = 0; f < 6; ++f) faces.push_back(face_key(v, f));
        }
        std::sort(edges.begin(), edges.end());
        edges.erase(std::unique(edges.begin(), edges.end()), edges.end());
        std::sort(faces.begin(), faces.end());
        // a shared face must be the same quadrilateral in every element
        for (size_t t = 1; t < faces.size(); ++t)
            if (faces[t].same_set(faces[t - 1]) && faces[t].opposite != faces[t - 1].opposite) return BS_EINVAL;
        faces.erase(std::unique(faces.begin(), faces.end(),
                                [](const FaceKey &x, const FaceKey &y) { return x.same_set(y); }),
                    faces.end());

        // Provisional ids: the vertices, then N-1 nodes per edge, (N-1)^2 per
        // face, (N-1)^3 per element, each entity's nodes in a frame fixed by
        // its vertex ids so that every element sharing it agrees.
        const int64_t m = N - 1;
        const int64_t base_edge = n_vertices;
        const int64_t base_face = base_edge + (int64_t)edges.size() * m;
        const int64_t base_cell = base_face + (int64_t)faces.size() * m * m;
        const int64_t n_raw = base_cell + E * m * m * m;
        // final ids: provisional ids renamed in order of first appearance
        std::vector<int32_t> rename((size_t)n_raw, -1);
        int64_t ng = 0;
        for (int64_t e = 0; e < E; ++e) {
            const int32_t *v = ev + 8 * e;
            int64_t eid[3][8], fid[6];
            for (int a = 0; a < 3; ++a)
                for (int c = 0; c < 8; ++c) {
                    if ((c >> a) & 1) continue;
                    const uint32_t x = (uint32_t)v[c], y = (uint32_t)v[c | 1 << a];
                    const uint64_t key = (uint64_t)std::min(x, y) << 32 | std::max(x, y);
                    eid[a][c] = std::lower_bound(edges.begin(), edges.end(), key) - edges.begin();
                }
            for (int f = 0; f < 6; ++f) {
                const FaceKey k = face_key(v, f);
                fid[f] = std::lower_bound(faces.begin(), faces.end(), k,
                                          [](const FaceKey &x, const FaceKey &y) {
                                              return std::lexicographical_compare(x.v, x.v + 4, y.v, y.v + 4);
                                          }) -
                         faces.begin();
            }
            int32_t *dst = l2g + e * Np;
            for (int64_t k = 0; k < nq; ++k)
                for (int64_t j = 0; j < nq; ++j)
                    for (int64_t i = 0; i < nq; ++i) {
                        const int64_t idx[3] = {i, j, k};
                        int bnd[3], nb = 0;
                        for (int a = 0; a < 3; ++a) {
                            bnd[a] = idx[a] == 0 ? 0 : idx[a] == N ? 1 : -1;
                            nb += bnd[a] >= 0;
                        }
                        int64_t raw;
                        if (nb == 3) {
                            raw = v[bnd[0] | bnd[1] << 1 | bnd[2] << 2];
                        } else if (nb == 2) {
                            // edge along the one interior axis, counted from its
                            // end with the smaller vertex id
                            const int a = bnd[0] < 0 ? 0 : bnd[1] < 0 ? 1 : 2;
                            int c0 = 0;
                            for (int b = 0; b < 3; ++b)
                                if (b != a) c0 |= bnd[b] << b;
                            const int c1 = c0 | 1 << a;
                            const int64_t u = v[c0] < v[c1] ? idx[a] : N - idx[a];
                            raw = base_edge + eid[a][c0] * m + (u - 1);
                        } else if (nb == 1) {
                            // face: origin at its smallest vertex, first axis
                            // towards the smaller of that vertex's two neighbours
                            const int a = bnd[0] >= 0 ? 0 : bnd[1] >= 0 ? 1 : 2;
                            const FaceFrame fr = face_frame(2 * a + bnd[a]);
                            int ua = 0, wa = 0;
                            for (int u = 0; u < 2; ++u)
                                for (int w = 0; w < 2; ++w)
                                    if (v[fr.corner(u, w)] < v[fr.corner(ua, wa)]) ua = u, wa = w;
                            const int64_t dp = ua ? N - idx[fr.a1] : idx[fr.a1];
                            const int64_t dq = wa ? N - idx[fr.a2] : idx[fr.a2];
                            const bool p_first = v[fr.corner(1 - ua, wa)] < v[fr.corner(ua, 1 - wa)];
                            const int64_t x = p_first ? dp : dq, y = p_first ? dq : dp;
                            raw = base_face + fid[2 * a + bnd[a]] * m * m + (y - 1) * m + (x - 1);
                        } else {
                            raw = base_cell + e * m * m * m + ((k - 1) * m + (j - 1)) * m + (i - 1);
                        }
                        int32_t &g = rename[(size_t)raw];
                        if (g < 0) g = (int32_t)ng++;
                        dst[i + nq * (j + nq * k)] = g;
                    }
        }
        *n_global = ng;
    } catch (const std::bad_alloc &) {
        return BS_ENOMEM;
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
    std::vector<double> r, w, block;
    try {
        r.resize(nq);
        w.resize(nq);
        block.resize(Np);
    } catch (const std::bad_alloc &) {
        return BS_ENOMEM;
    }
    bs_gll(order, r.data(), w.data());
    // one element's weights, w_i w_j w_k times the Jacobian 1/8 of the map
    // from [-1,1]^3 onto a unit cube; every element of the box is a unit cube
    for (int64_t k = 0; k < nq; ++k)
        for (int64_t j = 0; j < nq; ++j)
            for (int64_t i = 0; i < nq; ++i) block[i + nq * (j + nq * k)] = w[i] * w[j] * w[k] / 8.0;
    for (int64_t e = 0; e < K; ++e) std::memcpy(w_local + e * Np, block.data(), sizeof(double) * Np);
    return BS_OK;
}

int bs_mesh_hex_mass(int64_t n_elements, int order, const double *xe, double *w_local)
{
    if (n_elements < 0 || order < 1 || (n_elements > 0 && (!xe || !w_local))) return BS_EINVAL;
    const int64_t nq = order + 1;
    if (nq > 2048) return BS_ERANGE;
    const int64_t Np = nq * nq * nq;
    if (n_elements > INT32_MAX / Np) return BS_ERANGE;
    std::vector<double> r, w, h0, h1;
    try {
        r.resize(nq);
        w.resize(nq);
        h0.resize(nq);
        h1.resize(nq);
    } catch (const std::bad_alloc &) {
        return BS_ENOMEM;
    }
    bs_gll(order, r.data(), w.data());
    // the two linear blending functions of one axis at the GLL points
    for (int64_t t = 0; t < nq; ++t) {
        h0[t] = (1.0 - r[t]) / 2.0;
        h1[t] = (1.0 + r[t]) / 2.0;
    }
    for (int64_t e = 0; e < n_elements; ++e) {
        const double *X = xe + 24 * e;  // X[3 c + a], corner c = a + 2b + 4d
        // edge vectors along each reference axis: for axis a, the four edges
        // from corner c (bit a clear) to c + 2^a, halved (d/dxi of a linear
        // blend over [-1, 1])
        double edge[3][4][3];
        for (int a = 0; a < 3; ++a) {
            int m = 0;
            for (int c = 0; c < 8; ++c) {
                if ((c >> a) & 1) continue;
                for (int x = 0; x < 3; ++x) edge[a][m][x] = (X[3 * (c | 1 << a) + x] - X[3 * c + x]) / 2.0;
                ++m;
            }
        }
        int sign = 0;
        for (int64_t k = 0; k < nq; ++k)
            for (int64_t j = 0; j < nq; ++j)
                for (int64_t i = 0; i < nq; ++i) {
                    const int64_t idx[3] = {i, j, k};
                    double col[3][3];
                    for (int a = 0; a < 3; ++a) {
                        // bilinear blend of axis a's four edges over the other
                        // two axes (edges listed with the lower axis fastest)
                        const int b0 = a == 0 ? 1 : 0, b1 = a == 2 ? 1 : 2;
                        const double u0 = h0[idx[b0]], u1 = h1[idx[b0]];
                        const double v0 = h0[idx[b1]], v1 = h1[idx[b1]];
                        for (int x = 0; x < 3; ++x)
                            col[a][x] = (u0 * v0) * edge[a][0][x] + (u1 * v0) * edge[a][1][x] +
                                        (u0 * v1) * edge[a][2][x] + (u1 * v1) * edge[a][3][x];
                    }
                    // det J = col0 . (col1 x col2)
                    const double cx = col[1][1] * col[2][2] - col[1][2] * col[2][1];
                    const double cy = col[1][2] * col[2][0] - col[1][0] * col[2][2];
                    const double cz = col[1][0] * col[2][1] - col[1][1] * col[2][0];
                    const double det = col[0][0] * cx + col[0][1] * cy + col[0][2] * cz;
                    const int sg = det > 0.0 ? 1 : det < 0.0 ? -1 : 0;
                    if (sg == 0 || (sign != 0 && sg != sign)) return BS_EINVAL;
                    sign = sg;
                    w_local[e * Np + i + nq * (j + nq * k)] = w[i] * w[j] * w[k] * std::fabs(det);
                }
    }
    return BS_OK;
}

int bs_validate_l2g(int64_t n_local, int64_t n_global, const int32_t *l2g)
{
    if (n_local < 0 || n_global < 0 || (n_local > 0 && !l2g)) return BS_EINVAL;
    for (int64_t i = 0; i < n_local; ++i)
        if (l2g[i] >= n_global) return BS_EINVAL;
    return BS_OK;
}

int bs_validate_g2l(int64_t n_global, int64_t n_local, const int32_t *off, const int32_t *ids, const int32_t *l2g)
{
    if (n_global < 0 || n_local < 0 || !off) return BS_EINVAL;
    if (n_global >= INT32_MAX || n_local > INT32_MAX) return BS_ERANGE;
    if (off[0] != 0) return BS_EINVAL;
    for (int64_t g = 0; g < n_global; ++g)
        if (off[g + 1] < off[g]) return BS_EINVAL;
    const int64_t nnz = off[n_global];
    if (nnz > n_local) return BS_EINVAL;
    if (nnz > 0 && !ids) return BS_EINVAL;
    for (int64_t g = 0; g < n_global; ++g) {
        for (int64_t j = off[g]; j < off[g + 1]; ++j) {
            const int32_t i = ids[j];
            // in range, and strictly ascending inside the row (the order the
            // gather adds in; a repeated id would count an entry twice)
            if (i < 0 || i >= n_local) return BS_EINVAL;
            if (j > off[g] && i <= ids[j - 1]) return BS_EINVAL;
            if (l2g && l2g[i] != g) return BS_EINVAL;
        }
    }
    if (l2g) {
        // every unmasked local entry appears: the CSR is the whole transpose
        int64_t unmasked = 0;
        for (int64_t i = 0; i < n_local; ++i) unmasked += l2g[i] >= 0;
        if (unmasked != nnz) return BS_EINVAL;
    }
    return BS_OK;
}

int bs_validate_plan(int64_t n_global, const int32_t *off, const int32_t *plan, int64_t n_blocks)
{
    if (n_global < 0 || n_blocks < 0 || !off || (n_blocks > 0 && !plan)) return BS_EINVAL;
    if (n_global >= INT32_MAX) return BS_ERANGE;
    if (n_global == 0) return n_blocks == 0 ? BS_OK : BS_EINVAL;
    if (n_blocks < 1 || n_blocks > n_global) return BS_EINVAL;
    try {
        // each block a non-empty row range with the offsets of its ends; the
        // ranges, in any launch order, tile [0, n_global) once
        std::vector<std::pair<int32_t, int32_t>> rows((size_t)n_blocks);
        for (int64_t b = 0; b < n_blocks; ++b) {
            const int32_t *q = plan + 4 * b;
            if (q[0] < 0 || q[0] >= q[1] || q[1] > n_global) return BS_EINVAL;
            if (q[2] != off[q[0]] || q[3] != off[q[1]]) return BS_EINVAL;
            rows[(size_t)b] = {q[0], q[1]};
        }
        std::sort(rows.begin(), rows.end());
        if (rows.front().first != 0 || rows.back().second != n_global) return BS_EINVAL;
        for (size_t b = 1; b < rows.size(); ++b)
            if (rows[b].first != rows[b - 1].second) return BS_EINVAL;
    } catch (const std::bad_alloc &) {
        return BS_ENOMEM;
    }
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
    std::vector<int32_t> cursor;
    try {
        cursor.assign(off, off + n_global);
    } catch (const std::bad_alloc &) {
        return BS_ENOMEM;
    }
    for (int64_t i = 0; i < n_local; ++i) {
        const int32_t g = l2g[i];
        if (g >= 0) ids[cursor[(size_t)g]++] = (int32_t)i;
    }
    return BS_OK;
}

int bs_gather_plan(int64_t n_global, const int32_t *off, const int32_t *ids, int nodes_per_block,
                   int64_t region_entries, int32_t *plan, int64_t *n_blocks)
{
    if (n_global < 0 || !off || (n_global > 0 && !plan) || !n_blocks || region_entries < 0) return BS_EINVAL;
    if (region_entries > 0 && n_global > 0 && !ids) return BS_EINVAL;
    if (nodes_per_block < 1 || nodes_per_block > 1024) return BS_EINVAL;
    if (n_global >= INT32_MAX) return BS_ERANGE;
    // The offsets must be those of a CSR (non-decreasing from a non-negative
    // first entry): the blocks copy them, and region placement reads ids at
    // them.
    if (n_global > 0 && off[0] < 0) return BS_EINVAL;
    for (int64_t g = 0; g < n_global; ++g)
        if (off[g + 1] < off[g]) return BS_EINVAL;
    // Blocks in row order, greedily: extend the block row by row while it
    // holds at most nodes_per_block rows and nodes_per_block entries; a row
    // longer than that gets a block of its own. Then, unless it is the last
    // block, its end is rounded down to a multiple of kPlanAlign rows if that
    // leaves the block non-empty: every block then writes whole 128-byte
    // lines of v_global (16 doubles), where blocks cut at arbitrary rows left
    // two partial lines each (measured 2-3% faster gathers on the boxes, 1.6%
    // on an unstructured mesh, same bits).
    constexpr int64_t kPlanAlign = 16;
    try {
        std::vector<int32_t> start;
        for (int64_t g = 0; g < n_global;) {
            const int64_t first = off[g];
            int64_t end = g + 1;
            while (end < n_global && end - g < nodes_per_block && (int64_t)off[end + 1] - first <= nodes_per_block)
                ++end;
            if (end < n_global && end - end % kPlanAlign > g) end -= end % kPlanAlign;
            start.push_back((int32_t)g);
            g = end;
        }
        const int64_t nb = (int64_t)start.size();
        start.push_back((int32_t)n_global);
        // Launch order. The hardware hands the workgroups of a launch to the
        // eight XCDs in turn (workgroup s to XCD s mod 8), each XCD with an
        // L2 of its own, and blocks that read the same lines of v_local
        // should meet in one L2.
        std::vector<int64_t> order((size_t)nb);
        if (region_entries == 0) {
            // Neighbouring blocks read neighbouring lines: each XCD takes
            // runs of kXcdRun consecutive blocks while the eight XCDs work
            // in one narrow window of the arrays (runs of 8 measured best
            // against 4, 16 and one contiguous range per XCD). Slots past
            // the last whole round keep their own block.
            const int64_t span = kXcds * kXcdRun, full = nb / span * span;
            for (int64_t s = 0; s < nb; ++s) {
                const int64_t x = s % kXcds, k = s / kXcds;
                order[(size_t)s] = s >= full ? s : ((k / kXcdRun) * kXcds + x) * kXcdRun + k % kXcdRun;
            }
        } else {
            // Local storage interleaves eight regions in runs of
            // region_entries entries (bs_mesh_xcd_interleave): a block
            // belongs to the region of its first entry, which is its first
            // row's first copy, and XCD x takes the blocks of region x in
            // order. An XCD whose region has run out takes from the region
            // with the most blocks left.
            std::vector<std::vector<int64_t>> queue(kXcds);
            for (int64_t b = 0; b < nb; ++b) {
                const int32_t e0 = off[start[(size_t)b]], e1 = off[start[(size_t)b + 1]];
                if (e1 > e0 && ids[e0] < 0) return BS_EINVAL;  // not a local index
                const int64_t x = e1 > e0 ? ((int64_t)ids[e0] / region_entries) % kXcds : b % kXcds;
                queue[(size_t)x].push_back(b);
            }
            size_t next[kXcds] = {};
            for (int64_t s = 0; s < nb; ++s) {
                int64_t x = s % kXcds;
                if (next[x] == queue[(size_t)x].size()) {
                    size_t most = 0;
                    for (int64_t y = 0; y < kXcds; ++y) {
                        const size_t left = queue[(size_t)y].size() - next[y];
                        if (left > most) most = left, x = y;
                    }
                }
                order[(size_t)s] = queue[(size_t)x][next[x]++];
            }
        }
        // Each block as (first row, end row, first entry, end entry), the
        // entries being off at those rows, so that a block's whole extent
        // arrives in one round of scalar loads.
        for (int64_t s = 0; s < nb; ++s) {
            const int64_t b = order[(size_t)s];
            const int32_t r0 = start[(size_t)b], r1 = start[(size_t)b + 1];
            int32_t *q = plan + 4 * s;
            q[0] = r0;
            q[1] = r1;
            q[2] = off[r0];
            q[3] = off[r1];
        }
        *n_blocks = nb;
    } catch (const std::bad_alloc &) {
        return BS_ENOMEM;
    }
    return BS_OK;
}

int bs_mesh_xcd_interleave(int64_t n_elements, int64_t chunk, int32_t *perm)
{
    if (n_elements < 0 || chunk < 1 || (n_elements > 0 && !perm)) return BS_EINVAL;
    if (n_elements > INT32_MAX) return BS_ERANGE;
    // A run as long as the mesh puts every element in region 0 (the identity),
    // as any longer one does; the clamp keeps 8 * chunk from overflowing.
    chunk = std::min(chunk, std::max(n_elements, (int64_t)1));
    // Region x owns the storage slots s with (s / chunk) mod 8 == x and takes
    // the next count[x] elements of the given order, keeping their order.
    const int64_t round = kXcds * chunk, full = n_elements / round, rest = n_elements % round;
    int64_t first[kXcds];
    for (int64_t x = 0, sum = 0; x < kXcds; ++x) {
        first[x] = sum;
        sum += full * chunk + std::min(std::max(rest - x * chunk, (int64_t)0), chunk);
    }
    for (int64_t s = 0; s < n_elements; ++s) {
        const int64_t x = (s / chunk) % kXcds;
        perm[s] = (int32_t)(first[x] + (s / round) * chunk + s % chunk);
    }
    return BS_OK;
}

}  // extern "C"
