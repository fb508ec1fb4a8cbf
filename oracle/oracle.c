/*
 * oracle.c -- plain CPU reference for the seven Benchmark Streaming (BS)
 * operations of "Portable high-order finite element kernels I: Streaming
 * Operations" (arXiv 2009.10917), and for the mesh tables they run on.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library. It shares no source with
 * the HIP library and includes none of its headers.
 *
 * Arithmetic: IEEE binary64, round to nearest even, every product and sum
 * rounded on its own (built with -ffp-contract=off; the only fused
 * multiply-add is the explicit fma() of the error-free product below).
 *
 * Functions and the passages they follow (arXiv 2009.10917 unless noted):
 *   or_copy       BS1 copy, y = x                 (BS test list, "copy")
 *   or_axpy       BS2 y = alpha x + beta y         (CG vector operations, "vector addition")
 *   or_dot        BS4 alpha = x . y                (CG vector operations, "dot product")
 *   or_norm       BS3, the square root of x . x    (CG vector operations, "norm")
 *   or_cg_update  BS5 fused CG update              (BS test list: CG steps 8-10 fused)
 *   or_scatter    BS7 v_L = Z v_G                  (eq. 3; scatterIds with negative = masked)
 *   or_gather     BS6 v_G = Z^T v_L                (eq. 3 and the gather operator after it)
 *   or_gll_nodes  GLL points of degree p           (nodes of eqs. 1-2)
 *   or_mesh_box   I_l->g of a box hex mesh         (eqs. 1-3; arXiv 1506.05996, local-to-global table)
 *   or_g2l        CSR form of I_g->l               (arXiv 1506.05996, global-to-local table)
 *   or_gll_weights, or_mesh_box_mass, or_scale   lumped mass and the 1/m scaling
 *                 (arXiv 1506.05996, coarse-grid correction)
 *   or_mesh_hex   I_l->g of an unstructured hex mesh given by corner vertices
 *   or_mesh_hex_mass   lumped-mass weights of an unstructured hex mesh (arXiv 1506.05996)
 *                 (unstructured mesh of the CEED formulation section; arXiv 1506.05996, local-to-global table)
 *
 * The reductions (dot, norm, the residual norm of the fused update) are
 * evaluated accurately with Dot2 of Ogita, Rump and Oishi ("Accurate sum and
 * dot product", SIAM J. Sci. Comput. 26(6), 2005): error-free products and
 * sums inside fixed chunks of 2^16 terms, then the chunk results summed with
 * cascaded error-free sums in chunk order. The result does not depend on the
 * thread count and is far more accurate than the 1e-12 relative tolerance the
 * GPU is held to.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_CHUNK 65536

/* Threads the parallel loops below use. */
int or_threads(void)
{
    return omp_get_max_threads();
}

/* Sets how many threads the parallel loops below use from now on (n > 0;
   other values change nothing): the baseline is timed on all cores and on
   one. No result depends on it: the reductions combine fixed chunks in a
   fixed order. */
void or_set_threads(int n)
{
    if (n > 0) omp_set_num_threads(n);
}

/* ---------------------------------------------------------------- BS1 --- */
/* y = x as a bit copy: NaN payloads and signed zeros are preserved. */
void or_copy(int64_t n, const double *x, double *y)
{
    if (n > 0) memcpy(y, x, (size_t)n * sizeof(double));
}

/* ---------------------------------------------------------------- BS2 --- */
/* y = (alpha * x) + (beta * y), each product rounded, then the sum rounded.
 * y is always read, also for beta == 0. */
void or_axpy(int64_t n, double alpha, const double *x, double beta, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double t1 = alpha * x[i];
        double t2 = beta * y[i];
        y[i] = t1 + t2;
    }
}

/* ------------------------------------------- accurate reductions (Dot2) --- */
static void two_sum(double a, double b, double *s, double *e)
{
    double x = a + b;
    double z = x - a;
    *e = (a - (x - z)) + (b - z);
    *s = x;
}

static void two_prod(double a, double b, double *p, double *e)
{
    double x = a * b;
    *e = fma(a, b, -x);
    *p = x;
}

/* Dot2 over one chunk: returns the leading sum in *hi and the accumulated
 * error terms in *lo. */
static void dot2_chunk(int64_t n, const double *x, const double *y, double *hi, double *lo)
{
    double p = 0.0, s = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double h, r, q;
        two_prod(x[i], y[i], &h, &r);
        two_sum(p, h, &p, &q);
        s = s + (q + r);
    }
    *hi = p;
    *lo = s;
}

double or_dot(int64_t n, const double *x, const double *y)
{
    if (n <= 0) return 0.0;
    int64_t nc = (n + OR_CHUNK - 1) / OR_CHUNK;
    double *part = (double *)malloc((size_t)(2 * nc) * sizeof(double));
    if (!part) return NAN;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < nc; ++c) {
        int64_t a = c * OR_CHUNK;
        int64_t len = (n - a < OR_CHUNK) ? (n - a) : OR_CHUNK;
        dot2_chunk(len, x + a, y + a, &part[2 * c], &part[2 * c + 1]);
    }
    /* cascaded error-free summation of hi_0, lo_0, hi_1, lo_1, ... in order */
    double pi = part[0], sigma = 0.0;
    for (int64_t k = 1; k < 2 * nc; ++k) {
        double q;
        two_sum(pi, part[k], &pi, &q);
        sigma = sigma + q;
    }
    free(part);
    return pi + sigma;
}

/* ---------------------------------------------------------------- BS3 --- */
double or_norm(int64_t n, const double *x)
{
    return sqrt(or_dot(n, x, x));
}

/* ---------------------------------------------------------------- BS5 --- */
/* x = x + (alpha p); r = r - (alpha q); returns r . r of the updated r. */
double or_cg_update(int64_t n, double alpha, const double *p, const double *q,
                    double *x, double *r)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double ap = alpha * p[i];
        double aq = alpha * q[i];
        x[i] = x[i] + ap;
        r[i] = r[i] - aq;
    }
    return or_dot(n, r, r);
}

/* ---------------------------------------------------------------- BS7 --- */
/* v_L[i] = v_G[l2g[i]]; a negative id is a masked row of Z, giving +0.0. */
void or_scatter(int64_t n_local, const int32_t *l2g, const double *v_global, double *v_local)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_local; ++i)
        v_local[i] = (l2g[i] >= 0) ? v_global[l2g[i]] : 0.0;
}

/* ---------------------------------------------------------------- BS6 --- */
/* v_G = Z^T v_L straight from the definition of Z: every global entry starts
 * at +0.0 and receives the local values that map to it, in ascending local
 * index. Masked (negative) ids contribute nothing. */
void or_gather(int64_t n_local, int64_t n_global, const int32_t *l2g,
               const double *v_local, double *v_global)
{
    for (int64_t g = 0; g < n_global; ++g) v_global[g] = 0.0;
    for (int64_t i = 0; i < n_local; ++i)
        if (l2g[i] >= 0) v_global[l2g[i]] = v_global[l2g[i]] + v_local[i];
}

/* -------------------------------------------------------- GLL points --- */
/* Legendre P_p(t) and P_{p-1}(t) by the three-term recurrence. */
static void legendre(int p, double t, double *Pp, double *Pm)
{
    double a = 1.0, b = t;            /* P_0, P_1 */
    if (p == 0) { *Pp = 1.0; *Pm = 0.0; return; }
    for (int k = 1; k < p; ++k) {
        double c = ((2.0 * k + 1.0) * t * b - k * a) / (k + 1.0);
        a = b;
        b = c;
    }
    *Pp = b;
    *Pm = a;
}

/* The p+1 Gauss-Lobatto-Legendre points on [-1, 1], ascending: the end points
 * and the roots of P_p'. Newton's method from the Chebyshev-Lobatto points,
 * with P_p' = p (t P_p - P_{p-1}) / (t^2 - 1) and, from Legendre's equation,
 * P_p'' = (2 t P_p' - p (p+1) P_p) / (1 - t^2). Returns 0, or -1 if p < 1. */
int or_gll_nodes(int p, double *r)
{
    if (p < 1) return -1;
    r[0] = -1.0;
    r[p] = 1.0;
    for (int i = 1; i < p; ++i) {
        double t = -cos(M_PI * i / p);
        for (int it = 0; it < 100; ++it) {
            double P, Pm;
            legendre(p, t, &P, &Pm);
            double d1 = p * (t * P - Pm) / (t * t - 1.0);
            double d2 = (2.0 * t * d1 - p * (p + 1.0) * P) / (1.0 - t * t);
            double dt = d1 / d2;
            t -= dt;
            if (fabs(dt) < 1e-16) break;
        }
        r[i] = t;
    }
    return 0;
}

/* --------------------------------------------------------- box mesh --- */
static int cmp_double(const void *pa, const void *pb)
{
    double a = *(const double *)pa, b = *(const double *)pb;
    return (a < b) ? -1 : (a > b);
}

/* Position of the GLL point r_i in cell c of one axis: c + (1 + r_i)/2. The
 * end points r_0 = -1 and r_p = 1 land exactly on c and c+1, so neighbouring
 * cells share their boundary positions. */
static double axis_pos(int64_t c, double ri)
{
    return (double)c + (1.0 + ri) / 2.0;
}

/* Sorted distinct positions of one axis with `cells` cells; returns count. */
static int64_t axis_values(int64_t cells, int p, const double *r, double *u)
{
    int64_t m = 0;
    for (int64_t c = 0; c < cells; ++c)
        for (int i = 0; i <= p; ++i) u[m++] = axis_pos(c, r[i]);
    qsort(u, (size_t)m, sizeof(double), cmp_double);
    int64_t d = 0;
    for (int64_t t = 0; t < m; ++t)
        if (t == 0 || u[t] != u[d - 1]) u[d++] = u[t];
    return d;
}

/* Index of v in the sorted distinct array u[0..n-1] (v is present). */
static int64_t axis_rank(const double *u, int64_t n, double v)
{
    int64_t lo = 0, hi = n - 1;
    while (lo < hi) {
        int64_t mid = (lo + hi) / 2;
        if (u[mid] < v) lo = mid + 1; else hi = mid;
    }
    return lo;
}

/*
 * I_l->g of the box [0,ex]x[0,ey]x[0,ez] cut into unit hexahedra, each
 * carrying the (p+1)^3 tensor-product GLL nodes mapped from the reference
 * cube. Global nodes are the distinct physical positions: two local nodes
 * share a global id exactly when their positions coincide. Ids run over the
 * distinct positions in lexicographic order, x fastest, then y, then z;
 * node_perm (optional) renames id g to node_perm[g].
 *
 * Positions are compared through their per-axis ranks among the distinct
 * coordinate values of that axis: equal positions have equal rank triples and
 * the rank triple orders positions lexicographically. The distinct triples
 * present are then numbered in that order.
 *
 * Local storage is element by element; inside an element the node (i,j,k)
 * sits at i + (p+1)(j + (p+1)k). Storage slot s holds element elem_perm[s]
 * (optional; identity otherwise), element e being (e % ex, (e/ex) % ey,
 * e/(ex*ey)).
 *
 * Returns the number of global nodes, or -1 on bad arguments or no memory.
 */
int64_t or_mesh_box(int ex, int ey, int ez, int p, const int32_t *elem_perm,
                    const int32_t *node_perm, int32_t *l2g)
{
    if (ex < 1 || ey < 1 || ez < 1 || p < 1) return -1;
    const int64_t nq = p + 1, Np = nq * nq * nq;
    const int64_t K = (int64_t)ex * ey * ez, NL = K * Np;
    double *r = (double *)malloc((size_t)nq * sizeof(double));
    double *ux = (double *)malloc((size_t)(ex * nq) * sizeof(double));
    double *uy = (double *)malloc((size_t)(ey * nq) * sizeof(double));
    double *uz = (double *)malloc((size_t)(ez * nq) * sizeof(double));
    int64_t *key = (int64_t *)malloc((size_t)NL * sizeof(int64_t));
    if (!r || !ux || !uy || !uz || !key) goto fail;
    or_gll_nodes(p, r);
    int64_t nx = axis_values(ex, p, r, ux);
    int64_t ny = axis_values(ey, p, r, uy);
    int64_t nz = axis_values(ez, p, r, uz);
    int64_t nkeys = nx * ny * nz;
    int32_t *rank = (int32_t *)calloc((size_t)nkeys, sizeof(int32_t));
    if (!rank) goto fail;
    for (int64_t s = 0; s < K; ++s) {
        int64_t e = elem_perm ? elem_perm[s] : s;
        int64_t cx = e % ex, cy = (e / ex) % ey, cz = e / ((int64_t)ex * ey);
        for (int64_t k = 0; k < nq; ++k)
            for (int64_t j = 0; j < nq; ++j)
                for (int64_t i = 0; i < nq; ++i) {
                    int64_t L = s * Np + i + nq * (j + nq * k);
                    int64_t ix = axis_rank(ux, nx, axis_pos(cx, r[i]));
                    int64_t iy = axis_rank(uy, ny, axis_pos(cy, r[j]));
                    int64_t iz = axis_rank(uz, nz, axis_pos(cz, r[k]));
                    key[L] = (iz * ny + iy) * nx + ix;
                    rank[key[L]] = 1;
                }
    }
    int64_t NG = 0;
    for (int64_t t = 0; t < nkeys; ++t) {
        int32_t present = rank[t];
        rank[t] = (int32_t)NG;
        NG += present;
    }
    for (int64_t L = 0; L < NL; ++L) {
        int32_t g = rank[key[L]];
        l2g[L] = node_perm ? node_perm[g] : g;
    }
    free(rank);
    free(key); free(uz); free(uy); free(ux); free(r);
    return NG;
fail:
    free(key); free(uz); free(uy); free(ux); free(r);
    return -1;
}

/* ---------------------------------------------------- CSR of I_g->l --- */
typedef struct { int32_t g; int64_t i; } or_pair;

static int cmp_pair(const void *pa, const void *pb)
{
    const or_pair *a = (const or_pair *)pa, *b = (const or_pair *)pb;
    if (a->g != b->g) return a->g < b->g ? -1 : 1;
    return (a->i < b->i) ? -1 : (a->i > b->i);
}

/* For each global node g, ids[off[g] .. off[g+1]-1] lists the local indices
 * i with l2g[i] == g, ascending. Masked (negative) entries are left out.
 * Returns the number of entries, or -1 on an id out of range / no memory. */
int64_t or_g2l(int64_t n_local, int64_t n_global, const int32_t *l2g,
               int32_t *off, int32_t *ids)
{
    or_pair *pr = (or_pair *)malloc((size_t)(n_local > 0 ? n_local : 1) * sizeof(or_pair));
    if (!pr) return -1;
    int64_t m = 0;
    for (int64_t i = 0; i < n_local; ++i) {
        if (l2g[i] < 0) continue;
        if (l2g[i] >= n_global) { free(pr); return -1; }
        pr[m].g = l2g[i];
        pr[m].i = i;
        ++m;
    }
    qsort(pr, (size_t)m, sizeof(or_pair), cmp_pair);
    int64_t t = 0;
    for (int64_t g = 0; g < n_global; ++g) {
        off[g] = (int32_t)t;
        while (t < m && pr[t].g == g) {
            ids[t] = (int32_t)pr[t].i;
            ++t;
        }
    }
    off[n_global] = (int32_t)t;
    free(pr);
    return m;
}

/* ------------------------------------------------ lumped mass, 1/m scale --- */
/* GLL quadrature weights on [-1, 1]: w_i = 2 / (p (p+1) P_p(r_i)^2) at the
 * nodes of or_gll_nodes. Returns 0, or -1 if p < 1. */
int or_gll_weights(int p, double *w)
{
    if (p < 1) return -1;
    double *r = (double *)malloc((size_t)(p + 1) * sizeof(double));
    if (!r) return -1;
    or_gll_nodes(p, r);
    for (int i = 0; i <= p; ++i) {
        double P, Pm;
        legendre(p, r[i], &P, &Pm);
        w[i] = 2.0 / ((double)p * (p + 1.0) * P * P);
    }
    free(r);
    return 0;
}

/* Local (diagonal) mass weights of the box mesh of unit hexahedra: node
 * (i,j,k) of every element carries w_i w_j w_k / 8 (the GLL weights times
 * the Jacobian of the map from [-1,1]^3 onto a unit cube). The lumped global
 * mass is the gather of these weights, m = Z^T w_L ("GPU accelerated spectral
 * finite elements on all-hex meshes", coarse-grid correction: the lumped mass
 * as the global components of the local weights). */
int or_mesh_box_mass(int ex, int ey, int ez, int p, double *w_local)
{
    if (ex < 1 || ey < 1 || ez < 1 || p < 1) return -1;
    const int64_t nq = p + 1, Np = nq * nq * nq, K = (int64_t)ex * ey * ez;
    double *w = (double *)malloc((size_t)nq * sizeof(double));
    if (!w) return -1;
    or_gll_weights(p, w);
    for (int64_t e = 0; e < K; ++e)
        for (int64_t k = 0; k < nq; ++k)
            for (int64_t j = 0; j < nq; ++j)
                for (int64_t i = 0; i < nq; ++i)
                    w_local[e * Np + i + nq * (j + nq * k)] = w[i] * w[j] * w[k] / 8.0;
    free(w);
    return 0;
}

/* y[i] = x[i] / d[i], one correctly rounded division ("scaling by the
 * inverted mass matrix", arXiv 1506.05996, coarse-grid correction). */
void or_scale(int64_t n, const double *x, const double *d, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = x[i] / d[i];
}

/* ------------------------------------------- unstructured hex meshes --- */
/*
 * I_l->g of an unstructured mesh of hexahedra ("Portable high-order finite
 * element kernels I", the unstructured hexahedral mesh of the CEED
 * formulation section; "GPU accelerated spectral finite elements on all-hex
 * meshes", local-to-global table: one global number per GLL node of the
 * mesh).
 *
 * Element e is given by its 8 corner vertices: corner c = a + 2b + 4d is the
 * corner (a, b, d) in {0,1}^3 of the reference cube (x, y, z), so corner c is
 * local node (a p, b p, d p) of the node order i + (p+1)(j + (p+1)k). Its
 * vertex is ev[8e + c], an id in [0, n_vert).
 *
 * Local node (i,j,k) is the point sum_c phi_c X_{ev[8e+c]} of the trilinear
 * map, phi_c the product over the three axes of (1 - r)/2 (bit 0) or
 * (1 + r)/2 (bit 1) at the node's GLL coordinate. Two local nodes are the same
 * global node exactly when they put the same weight on every vertex. The
 * weights are kept exactly, as symbols: the factor of axis a is identified by
 * m_a = i_a for bit 1 and p - i_a for bit 0, the node's GLL index counted
 * from the far end of that axis. GLL points are distinct and symmetric
 * (r_{p-i} = -r_i), so equal m give equal factors; m = 0 is the zero factor.
 * A vertex's weight is the multiset of its three m (a product does not depend
 * on the order of its factors), and a node's signature is the list of
 * (vertex, sorted m triple) over its vertices with nonzero weight, sorted.
 *
 * Global ids number the distinct signatures in order of first appearance in
 * local storage order. Returns the number of global nodes, or -1 on bad
 * arguments (a vertex id out of range, an element with a repeated vertex) or
 * no memory.
 */
#define OR_SIG 16   /* 8 (vertex, weight code) pairs */

static const int32_t *or_sig_base;

static int cmp_sig(const void *pa, const void *pb)
{
    const int32_t *a = or_sig_base + (int64_t)OR_SIG * *(const int64_t *)pa;
    const int32_t *b = or_sig_base + (int64_t)OR_SIG * *(const int64_t *)pb;
    for (int t = 0; t < OR_SIG; ++t)
        if (a[t] != b[t]) return a[t] < b[t] ? -1 : 1;
    return 0;
}

int64_t or_mesh_hex(int64_t n_elem, int p, int64_t n_vert, const int32_t *ev, int32_t *l2g)
{
    if (n_elem < 0 || p < 1 || n_vert < 0) return -1;
    for (int64_t e = 0; e < n_elem; ++e)
        for (int c = 0; c < 8; ++c) {
            if (ev[8 * e + c] < 0 || ev[8 * e + c] >= n_vert) return -1;
            for (int c2 = 0; c2 < c; ++c2)
                if (ev[8 * e + c2] == ev[8 * e + c]) return -1;
        }
    const int64_t nq = p + 1, Np = nq * nq * nq, NL = n_elem * Np;
    int32_t *sig = (int32_t *)malloc((size_t)(NL > 0 ? NL : 1) * OR_SIG * sizeof(int32_t));
    int64_t *order = (int64_t *)malloc((size_t)(NL > 0 ? NL : 1) * sizeof(int64_t));
    int64_t *cls = (int64_t *)malloc((size_t)(NL > 0 ? NL : 1) * sizeof(int64_t));
    if (!sig || !order || !cls) goto fail;
    for (int64_t e = 0; e < n_elem; ++e)
        for (int64_t k = 0; k < nq; ++k)
            for (int64_t j = 0; j < nq; ++j)
                for (int64_t i = 0; i < nq; ++i) {
                    const int64_t L = e * Np + i + nq * (j + nq * k);
                    const int64_t idx[3] = {i, j, k};
                    int32_t *s = sig + OR_SIG * L;
                    int n = 0;
                    for (int c = 0; c < 8; ++c) {
                        int64_t m[3];
                        int zero = 0;
                        for (int a = 0; a < 3; ++a) {
                            m[a] = ((c >> a) & 1) ? idx[a] : p - idx[a];
                            if (m[a] == 0) zero = 1;
                        }
                        if (zero) continue;
                        /* sort the three factors */
                        for (int x = 0; x < 3; ++x)
                            for (int y = x + 1; y < 3; ++y)
                                if (m[y] < m[x]) { int64_t t = m[x]; m[x] = m[y]; m[y] = t; }
                        s[2 * n] = ev[8 * e + c];
                        s[2 * n + 1] = (int32_t)((m[0] * nq + m[1]) * nq + m[2]);
                        ++n;
                    }
                    /* sort the (vertex, code) pairs by vertex: insertion sort */
                    for (int x = 1; x < n; ++x)
                        for (int y = x; y > 0 && s[2 * y] < s[2 * (y - 1)]; --y) {
                            int32_t t0 = s[2 * y], t1 = s[2 * y + 1];
                            s[2 * y] = s[2 * (y - 1)];
                            s[2 * y + 1] = s[2 * (y - 1) + 1];
                            s[2 * (y - 1)] = t0;
                            s[2 * (y - 1) + 1] = t1;
                        }
                    for (int x = n; x < 8; ++x) s[2 * x] = s[2 * x + 1] = -1;
                }
    /* group equal signatures */
    for (int64_t L = 0; L < NL; ++L) order[L] = L;
    or_sig_base = sig;
    qsort(order, (size_t)NL, sizeof(int64_t), cmp_sig);
    int64_t ncls = 0;
    for (int64_t t = 0; t < NL; ++t) {
        if (t > 0 && cmp_sig(&order[t - 1], &order[t]) != 0) ++ncls;
        cls[order[t]] = ncls;
    }
    if (NL > 0) ++ncls;
    /* number the classes by first appearance */
    int64_t *first = order;   /* reused: class -> global id */
    for (int64_t t = 0; t < ncls; ++t) first[t] = -1;
    int64_t NG = 0;
    for (int64_t L = 0; L < NL; ++L) {
        if (first[cls[L]] < 0) first[cls[L]] = NG++;
        l2g[L] = (int32_t)first[cls[L]];
    }
    free(cls); free(order); free(sig);
    return NG;
fail:
    free(cls); free(order); free(sig);
    return -1;
}

/* Local lumped-mass weights of an unstructured hex mesh: node (i,j,k) of
 * element e carries w_i w_j w_k |det J(r_i, r_j, r_k)|, J the Jacobian of the
 * element's trilinear map x(xi) = sum_c phi_c(xi) X_c ("GPU accelerated
 * spectral finite elements on all-hex meshes": the geometry of each element
 * is its own map, and the lumped mass takes the quadrature weights times the
 * Jacobian at the nodes). xe[24 e + 3 c + a] is coordinate a of corner
 * c = a + 2b + 4d of element e (the corner order of or_mesh_hex).
 * phi_c is the product over the axes of (1 - t)/2 (bit 0) or (1 + t)/2
 * (bit 1), so dphi_c/dxi_a is that product with axis a's factor replaced by
 * -1/2 or +1/2. Returns 0, or -1 if p < 1, n_elem < 0 or no memory. */
int or_mesh_hex_mass(int64_t n_elem, int p, const double *xe, double *w_local)
{
    if (n_elem < 0 || p < 1) return -1;
    const int64_t nq = p + 1, Np = nq * nq * nq;
    double *r = (double *)malloc((size_t)nq * sizeof(double));
    double *w = (double *)malloc((size_t)nq * sizeof(double));
    if (!r || !w) { free(r); free(w); return -1; }
    or_gll_nodes(p, r);
    or_gll_weights(p, w);
    for (int64_t e = 0; e < n_elem; ++e)
        for (int64_t k = 0; k < nq; ++k)
            for (int64_t j = 0; j < nq; ++j)
                for (int64_t i = 0; i < nq; ++i) {
                    const double t[3] = {r[i], r[j], r[k]};
                    double J[3][3] = {{0}};   /* J[row = x,y,z][col = d/dxi_a] */
                    for (int c = 0; c < 8; ++c)
                        for (int a = 0; a < 3; ++a) {
                            double d = 1.0;
                            for (int b = 0; b < 3; ++b) {
                                const int bit = (c >> b) & 1;
                                if (b == a) d *= bit ? 0.5 : -0.5;
                                else d *= bit ? (1.0 + t[b]) / 2.0 : (1.0 - t[b]) / 2.0;
                            }
                            for (int x = 0; x < 3; ++x) J[x][a] += d * xe[24 * e + 3 * c + x];
                        }
                    const double det = J[0][0] * (J[1][1] * J[2][2] - J[1][2] * J[2][1])
                                     - J[0][1] * (J[1][0] * J[2][2] - J[1][2] * J[2][0])
                                     + J[0][2] * (J[1][0] * J[2][1] - J[1][1] * J[2][0]);
                    w_local[e * Np + i + nq * (j + nq * k)] = w[i] * w[j] * w[k] * fabs(det);
                }
    free(r);
    free(w);
    return 0;
}
