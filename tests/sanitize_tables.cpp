// sanitize_tables.cpp -- the host-side table builders of libbs and the CPU
// oracle's builders and vector operations, run under AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitize_host.py builds this file
// with bs_host.cpp and oracle.c, all instrumented, and runs it).
//
// Every builder runs on boxes of several shapes and orders (with and without
// element and node permutations) and on the unstructured meshes whose corner
// vertices and coordinates the test writes to the directory given as argv[1];
// the library's tables are compared with the oracle's (exactly) and checked by
// the library's own validators, and the error paths are exercised with bad
// sizes, ids, permutations and tables. Exit status 0 and a final "OK" line
// mean every check held and no sanitizer fired.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "bs.h"

extern "C" {
int64_t or_mesh_box(int ex, int ey, int ez, int p, const int32_t *elem_perm, const int32_t *node_perm,
                    int32_t *l2g);
int64_t or_g2l(int64_t n_local, int64_t n_global, const int32_t *l2g, int32_t *off, int32_t *ids);
int64_t or_mesh_hex(int64_t n_elem, int p, int64_t n_vert, const int32_t *ev, int32_t *l2g);
int or_mesh_hex_mass(int64_t n_elem, int p, const double *xe, double *w_local);
int or_gll_nodes(int p, double *r);
int or_gll_weights(int p, double *w);
int or_mesh_box_mass(int ex, int ey, int ez, int p, double *w_local);
void or_copy(int64_t n, const double *x, double *y);
void or_axpy(int64_t n, double alpha, const double *x, double beta, double *y);
double or_dot(int64_t n, const double *x, const double *y);
double or_norm(int64_t n, const double *x);
double or_cg_update(int64_t n, double alpha, const double *p, const double *q, double *x, double *r);
void or_scatter(int64_t n_local, const int32_t *l2g, const double *v_global, double *v_local);
void or_gather(int64_t n_local, int64_t n_global, const int32_t *l2g, const double *v_local, double *v_global);
void or_scale(int64_t n, const double *x, const double *d, double *y);
}

#define CHECK(c)                                                                 \
    do {                                                                         \
        if (!(c)) {                                                              \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            std::exit(2);                                                        \
        }                                                                        \
    } while (0)

namespace {

// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): test data only.
uint64_t next(uint64_t &s)
{
    uint64_t z = (s += 0x9E3779B97F4A7C15ULL);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

std::vector<int32_t> permutation(int64_t n, uint64_t seed)
{
    std::vector<int32_t> p((size_t)n);
    for (int64_t i = 0; i < n; ++i) p[(size_t)i] = (int32_t)i;
    for (int64_t i = n - 1; i > 0; --i) std::swap(p[(size_t)i], p[(size_t)(next(seed) % (uint64_t)(i + 1))]);
    return p;
}

std::vector<double> values(int64_t n, uint64_t seed)
{
    std::vector<double> v((size_t)n);
    for (auto &x : v) x = (double)(next(seed) >> 11) * 0x1.0p-52 - 1.0;
    return v;
}

// The CSR of the library and of the oracle agree, the validators accept the
// tables, and plans of several block sizes are valid.
void check_tables(const std::vector<int32_t> &l2g, int64_t ng)
{
    const int64_t nl = (int64_t)l2g.size();
    CHECK(bs_validate_l2g(nl, ng, l2g.data()) == BS_OK);
    std::vector<int32_t> off((size_t)ng + 1), ids((size_t)nl + 1), ooff((size_t)ng + 1), oids((size_t)nl + 1);
    CHECK(bs_index_g2l(nl, ng, l2g.data(), off.data(), ids.data()) == BS_OK);
    const int64_t m = or_g2l(nl, ng, l2g.data(), ooff.data(), oids.data());
    CHECK(m == off[(size_t)ng]);
    CHECK(off == ooff);
    CHECK(std::equal(ids.begin(), ids.begin() + m, oids.begin()));
    CHECK(bs_validate_g2l(ng, nl, off.data(), ids.data(), l2g.data()) == BS_OK);
    for (int npb : {1, 3, 64, 1000, 1024}) {
        std::vector<int32_t> plan(4 * (size_t)ng);
        int64_t nb = -1;
        CHECK(bs_gather_plan(ng, off.data(), ids.data(), npb, 0, plan.data(), &nb) == BS_OK);
        CHECK(nb >= 1 && nb <= ng);
        CHECK(bs_validate_plan(ng, off.data(), plan.data(), nb) == BS_OK);
        // placed by region as if the local vector interleaved runs of 37 entries
        CHECK(bs_gather_plan(ng, off.data(), ids.data(), npb, 37, plan.data(), &nb) == BS_OK);
        CHECK(bs_validate_plan(ng, off.data(), plan.data(), nb) == BS_OK);
    }
    // the oracle's scatter and gather on these tables: gather(1) is the multiplicity
    std::vector<double> ones((size_t)nl, 1.0), mult((size_t)ng), vg = values(ng, 7), vl((size_t)nl);
    or_gather(nl, ng, l2g.data(), ones.data(), mult.data());
    for (int64_t g = 0; g < ng; ++g) CHECK(mult[(size_t)g] == (double)(off[(size_t)g + 1] - off[(size_t)g]));
    or_scatter(nl, l2g.data(), vg.data(), vl.data());
    for (int64_t i = 0; i < nl; ++i) CHECK(vl[(size_t)i] == (l2g[(size_t)i] >= 0 ? vg[(size_t)l2g[(size_t)i]] : 0.0));
}

void box(int ex, int ey, int ez, int p, bool perms)
{
    int64_t nl = 0, ng = 0;
    CHECK(bs_mesh_box_count(ex, ey, ez, p, &nl, &ng) == BS_OK);
    std::vector<int32_t> ep, npm;
    if (perms) {
        ep = permutation((int64_t)ex * ey * ez, 11 + ex + p);
        npm = permutation(ng, 12 + ey + p);
    }
    const int32_t *epp = perms ? ep.data() : nullptr, *npp = perms ? npm.data() : nullptr;
    std::vector<int32_t> l2g((size_t)nl), ol2g((size_t)nl);
    CHECK(bs_mesh_box_l2g(ex, ey, ez, p, epp, npp, l2g.data()) == BS_OK);
    CHECK(or_mesh_box(ex, ey, ez, p, epp, npp, ol2g.data()) == ng);
    CHECK(l2g == ol2g);
    check_tables(l2g, ng);
    // a masked copy
    for (size_t i = 0; i < l2g.size(); i += 7) l2g[i] = -1;
    check_tables(l2g, ng);
    // lumped mass of the box: the library's and the oracle's weights agree
    std::vector<double> w((size_t)nl), ow((size_t)nl);
    CHECK(bs_mesh_box_mass(ex, ey, ez, p, w.data()) == BS_OK);
    CHECK(or_mesh_box_mass(ex, ey, ez, p, ow.data()) == 0);
    for (int64_t i = 0; i < nl; ++i) CHECK(std::fabs(w[(size_t)i] - ow[(size_t)i]) <= 1e-14 * std::fabs(ow[(size_t)i]));
}

void hex_mesh(const std::string &dir, const std::string &name, int64_t E, int64_t nv, int p)
{
    std::vector<int32_t> ev((size_t)E * 8);
    std::vector<double> xe((size_t)E * 24);
    FILE *f = std::fopen((dir + "/" + name + ".ev").c_str(), "rb");
    CHECK(f && std::fread(ev.data(), 4, ev.size(), f) == ev.size());
    std::fclose(f);
    f = std::fopen((dir + "/" + name + ".xe").c_str(), "rb");
    CHECK(f && std::fread(xe.data(), 8, xe.size(), f) == xe.size());
    std::fclose(f);
    const int64_t nl = E * (p + 1) * (p + 1) * (p + 1);
    std::vector<int32_t> l2g((size_t)nl), ol2g((size_t)nl);
    int64_t ng = -1;
    CHECK(bs_mesh_hex_l2g(E, p, nv, ev.data(), l2g.data(), &ng) == BS_OK);
    CHECK(or_mesh_hex(E, p, nv, ev.data(), ol2g.data()) == ng);
    CHECK(l2g == ol2g);
    check_tables(l2g, ng);
    // the Hilbert order of the elements is a permutation
    std::vector<int32_t> order((size_t)E), seen((size_t)E, 0);
    CHECK(bs_mesh_hex_order(E, xe.data(), order.data()) == BS_OK);
    for (int32_t e : order) {
        CHECK(e >= 0 && e < E && !seen[(size_t)e]);
        seen[(size_t)e] = 1;
    }
    std::vector<double> w((size_t)nl), ow((size_t)nl);
    CHECK(bs_mesh_hex_mass(E, p, xe.data(), w.data()) == BS_OK);
    CHECK(or_mesh_hex_mass(E, p, xe.data(), ow.data()) == 0);
    for (int64_t i = 0; i < nl; ++i) CHECK(std::fabs(w[(size_t)i] - ow[(size_t)i]) <= 1e-13 * std::fabs(ow[(size_t)i]));
    // error paths on this mesh: an id out of range, a repeated vertex, a flat element
    std::vector<int32_t> bad = ev;
    bad[5] = (int32_t)nv;
    CHECK(bs_mesh_hex_l2g(E, p, nv, bad.data(), l2g.data(), &ng) == BS_EINVAL);
    bad = ev;
    bad[3] = bad[0];
    CHECK(bs_mesh_hex_l2g(E, p, nv, bad.data(), l2g.data(), &ng) == BS_EINVAL);
    std::vector<double> flat = xe;
    for (int c = 0; c < 8; ++c) flat[(size_t)3 * c + 2] = 0.0;  // element 0 squashed into a plane
    CHECK(bs_mesh_hex_mass(E, p, flat.data(), w.data()) == BS_EINVAL);
}

void errors()
{
    int64_t a = 0, b = 0;
    CHECK(bs_mesh_box_count(0, 1, 1, 1, &a, &b) == BS_EINVAL);
    CHECK(bs_mesh_box_count(1 << 21, 1 << 21, 1 << 21, 1, &a, &b) == BS_ERANGE);
    CHECK(bs_mesh_box_count(2147483647, 2147483647, 2147483647, 2047, &a, &b) == BS_ERANGE);
    CHECK(bs_mesh_box_count(1, 1, 1, 1 << 30, &a, &b) == BS_ERANGE);
    std::vector<int32_t> l2g(8);
    std::vector<int32_t> notperm = {0, 1, 2, 3, 4, 5, 6, 6};
    CHECK(bs_mesh_box_l2g(2, 2, 2, 1, notperm.data(), nullptr, std::vector<int32_t>(64).data()) == BS_EINVAL);
    std::vector<int32_t> ids = {0, 1, 5}, off(6), col(4), plan(20);
    CHECK(bs_index_g2l(3, 5, ids.data(), off.data(), col.data()) == BS_EINVAL);
    CHECK(bs_validate_l2g(3, 5, ids.data()) == BS_EINVAL);
    std::vector<int32_t> good = {0, 1, 2, 3, 4}, col5(5);
    CHECK(bs_index_g2l(5, 5, good.data(), off.data(), col5.data()) == BS_OK);
    int64_t nb = 0;
    CHECK(bs_gather_plan(5, off.data(), nullptr, 0, 0, plan.data(), &nb) == BS_EINVAL);
    CHECK(bs_gather_plan(5, off.data(), nullptr, 1025, 0, plan.data(), &nb) == BS_EINVAL);
    CHECK(bs_gather_plan(5, off.data(), nullptr, 4, 8, plan.data(), &nb) == BS_EINVAL);
    CHECK(bs_gather_plan(5, off.data(), nullptr, 4, -1, plan.data(), &nb) == BS_EINVAL);
    {
        std::vector<int32_t> perm(1000);
        CHECK(bs_mesh_xcd_interleave(1000, 13, perm.data()) == BS_OK);
        std::vector<int32_t> seen(1000, 0);
        for (int32_t v : perm) {
            CHECK(v >= 0 && v < 1000);
            ++seen[(size_t)v];
        }
        for (int32_t c : seen) CHECK(c == 1);
        CHECK(bs_mesh_xcd_interleave(10, 0, perm.data()) == BS_EINVAL);
    }
    CHECK(bs_validate_plan(5, off.data(), nullptr, 1) == BS_EINVAL);
    CHECK(bs_validate_plan(5, nullptr, plan.data(), 1) == BS_EINVAL);
    CHECK(bs_validate_g2l(-1, 0, off.data(), nullptr, nullptr) == BS_EINVAL);
    std::vector<int32_t> ev = {0, 1, 2, 3, 4, 5, 6, 7};
    int64_t ng = 0;
    CHECK(bs_mesh_hex_l2g(1, 0, 8, ev.data(), l2g.data(), &ng) == BS_EINVAL);
    CHECK(bs_mesh_hex_l2g(1, 3000, 8, ev.data(), l2g.data(), &ng) == BS_ERANGE);
    double r[4], w[4];
    CHECK(bs_gll(0, r, w) == BS_EINVAL);
}

void gll()
{
    for (int p = 1; p <= 24; ++p) {
        std::vector<double> r((size_t)p + 1), w((size_t)p + 1), o((size_t)p + 1), ow((size_t)p + 1);
        CHECK(bs_gll(p, r.data(), w.data()) == BS_OK);
        CHECK(or_gll_nodes(p, o.data()) == 0 && or_gll_weights(p, ow.data()) == 0);
        double s = 0.0;
        for (int i = 0; i <= p; ++i) {
            CHECK(std::fabs(r[(size_t)i] - o[(size_t)i]) <= 1e-14);
            CHECK(std::fabs(w[(size_t)i] - ow[(size_t)i]) <= 1e-14);
            s += w[(size_t)i];
        }
        CHECK(std::fabs(s - 2.0) <= 1e-13);
    }
}

void vectors()
{
    for (int64_t n : {0, 1, 2, 3, 65535, 65536, 65537, 200003}) {
        std::vector<double> x = values(n, 21), y = values(n, 22), p = values(n, 23), q = values(n, 24), d(
                                                                                                    (size_t)n, 2.0);
        std::vector<double> z((size_t)n);
        or_copy(n, x.data(), z.data());
        CHECK(z == x);
        or_axpy(n, 0.5, x.data(), 1.0, z.data());
        const double s = or_dot(n, x.data(), y.data());
        const double nn = or_norm(n, x.data());
        CHECK(std::isfinite(s) && std::isfinite(nn) && nn >= 0.0);
        const double rr = or_cg_update(n, 0.37, p.data(), q.data(), x.data(), y.data());
        CHECK(rr >= 0.0);
        or_scale(n, x.data(), d.data(), z.data());
    }
}

}  // namespace

int main(int argc, char **argv)
{
    if (argc != 2) {
        std::fprintf(stderr, "usage: %s MESH_DIR\n", argv[0]);
        return 1;
    }
    const std::string dir = argv[1];
    for (int p = 1; p <= 6; ++p) {
        box(1, 1, 1, p, false);
        box(3, 2, 4, p, false);
        box(3, 2, 4, p, true);
        box(5, 1, 2, p, true);
    }
    box(8, 8, 8, 3, true);
    box(2, 3, 2, 15, false);
    // the unstructured meshes listed in MESH_DIR/meshes.txt: name E n_vertices order
    FILE *f = std::fopen((dir + "/meshes.txt").c_str(), "r");
    CHECK(f);
    char name[256];
    long long E, nv;
    int p, count = 0;
    while (std::fscanf(f, "%255s %lld %lld %d", name, &E, &nv, &p) == 4) {
        hex_mesh(dir, name, E, nv, p);
        ++count;
    }
    std::fclose(f);
    CHECK(count > 0);
    errors();
    gll();
    vectors();
    std::printf("sanitized host tables: %d unstructured meshes, OK\n", count);
    return 0;
}
