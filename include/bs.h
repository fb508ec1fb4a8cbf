/*
 * bs.h -- C ABI of the MI355X (gfx950) Benchmark Streaming library.
 *
 * The seven streaming operations of a Conjugate Gradient solve on high-order
 * hexahedral meshes, as named in "Portable high-order finite element kernels
 * I: Streaming Operations" (arXiv 2009.10917, the BS test list): BS1 copy,
 * BS2 AXPY, BS3 norm, BS4 inner product, BS5 fused CG update, BS6 gather,
 * BS7 scatter; plus the host-side builder of the index tables they need
 * (I_l->g and the CSR form of I_g->l of "GPU accelerated spectral finite
 * elements on all-hex meshes", arXiv 1506.05996).
 *
 * Conventions for every call below:
 *  - Vector and index pointers passed to the bs_* device operations are HIP
 *    device pointers owned by the caller. The library never allocates, frees
 *    or retains them. Scalars results are written to a caller-owned device
 *    double, so no call forces a host synchronisation.
 *  - Arithmetic is IEEE binary64, round to nearest even, each product and sum
 *    rounded separately (no fused multiply-add) wherever a result is required
 *    to be bit-exact. Indices are int32.
 *  - Every device operation is enqueued on `stream` (a hipStream_t passed as
 *    void*; NULL is the default stream) and returns at once. A fault inside a
 *    kernel surfaces at the caller's next synchronisation, not here.
 *  - Return value: BS_OK, or a negative bs_status; on error nothing has been
 *    enqueued. n == 0 is a no-op for vector outputs; reductions then store
 *    +0.0. n < 0, or a NULL pointer with n > 0, is BS_EINVAL. Double pointers
 *    must be 8-byte aligned and int32 pointers 4-byte aligned (BS_EALIGN).
 *    The vector operations run fastest on operands that share one 16-byte
 *    phase (all aligned, or all 8 bytes off); operands in different phases
 *    take 8-byte kernels, 14-21% slower for AXPY and the fused update. The
 *    scatter likewise wants l2g 8-byte and v_local 16-byte aligned (else
 *    about 7% slower). Elementwise results are the same bits either way;
 *    reductions sum in another fixed order, within the same tolerance.
 *  - A context owns the reduction scratch of one device. Calls that use the
 *    same context must be ordered (one stream, or explicit dependencies);
 *    concurrent reductions on one context race.
 *  - A call makes its context's device current while it runs and gives the
 *    calling thread its previous current device back before it returns.
 *  - Overlapping operands are checked where the sizes say how far each one
 *    reaches (the vector operations and the CG iteration): an overlap the
 *    call does not allow is BS_EINVAL.
 */
#ifndef BS_H
#define BS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BS_OK = 0,
    BS_EINVAL = -1, /* bad size, NULL pointer, bad mesh argument, bad table   */
    BS_EALIGN = -2, /* pointer not aligned to its element size                */
    BS_ERANGE = -3, /* size beyond what int32 indices or the builder can hold */
    BS_EHIP = -4,   /* the HIP runtime reported an error (launch, device)     */
    BS_ENOMEM = -5  /* host or device allocation failed                       */
} bs_status;

typedef struct bs_ctx bs_ctx;

/* Text for a status code (static storage; never NULL). */
const char *bs_strerror(int status);

/* Library version as major*10000 + minor*100 + patch. */
int bs_version(void);

/* Create a context on HIP device `device`: queries its compute-unit count and
 * allocates the reduction scratch (one partial sum per block of a first-stage
 * launch) on that device. *out receives the context; the caller releases it with
 * bs_ctx_destroy. Errors: BS_EINVAL (out NULL), BS_EHIP (no such device),
 * BS_ENOMEM. */
int bs_ctx_create(int device, bs_ctx **out);

/* Release a context and its scratch. Waits for the device to finish work that
 * may use the scratch. NULL is accepted. */
void bs_ctx_destroy(bs_ctx *ctx);

/* Device and compute-unit count of a context; NULL outputs are skipped. */
int bs_ctx_info(const bs_ctx *ctx, int *device, int *cu_count, int *max_partials);

/* Kernel timing, for measuring each operation against the pages' bandwidth
 * model (arXiv 2009.10917, performance model: time per operation and the
 * bytes it streams). Arms the context so that the next kernel it launches
 * (the first, streaming kernel of the next device operation called with it)
 * records the HIP events `start_event` and `stop_event` (hipEvent_t passed as
 * void*, created by the caller with timing enabled; either may be NULL) at
 * that kernel's own start and end, as hipExtLaunchKernel does, so that
 * hipEventElapsedTime gives the kernel's duration without the queue gaps that
 * events recorded on the stream around the call include. One-shot: the
 * launch disarms the context. An operation that enqueues nothing (an error, a
 * zero-length copy) leaves it armed; NULL, NULL disarms. The caller owns the
 * events and keeps them alive until they have completed. Errors: BS_EINVAL
 * (ctx NULL). */
int bs_ctx_time_next(bs_ctx *ctx, void *start_event, void *stop_event);

/* ------------------------------------------------------------------------
 * BS1 copy (arXiv 2009.10917, BS test list): y[i] = x[i] for 0 <= i < n, a
 * bit copy (NaN payloads and signed zeros kept). x and y are contiguous
 * double[n]; x == y is allowed (nothing to do), any other overlap is
 * BS_EINVAL. */
int bs_copy(bs_ctx *ctx, int64_t n, const double *x, double *y, void *stream);

/* BS2 AXPY, the CG "vector addition" y = alpha x + beta y (arXiv
 * 2009.10917, CG vector-operation list): y[i] = (alpha*x[i]) + (beta*y[i]),
 * each product rounded, then the sum; bit-exact. y is read also when
 * beta == 0. x, y contiguous double[n]; x == y allowed, any other overlap is
 * BS_EINVAL. */
int bs_axpy(bs_ctx *ctx, int64_t n, double alpha, const double *x, double beta,
            double *y, void *stream);

/* Pointwise scale y[i] = x[i] / d[i], one correctly rounded division each:
 * the scaling of a global vector by the inverted (lumped, diagonal) mass
 * matrix (arXiv 1506.05996, coarse-grid correction: y = r / m), the one
 * streaming operation that a lumped-mass / Jacobi step adds to the BS set.
 * x, d, y contiguous double[n]; y may be x or d, any other overlap of y
 * with them is BS_EINVAL. Bit-exact. */
int bs_scale(bs_ctx *ctx, int64_t n, const double *x, const double *d, double *y, void *stream);

/* BS3 norm (arXiv 2009.10917, CG vector-operation list and the two-kernel
 * reduction of the implementation section): *result = sqrt(sum x[i]^2), the
 * 2-norm, written to the device double `result`. The sum is reduced in a
 * fixed order that depends only on n and the device's compute-unit count, so
 * repeated calls give the same bits; it agrees with the exact value to a
 * relative 1e-12. x contiguous double[n]. */
int bs_norm(bs_ctx *ctx, int64_t n, const double *x, double *result, void *stream);

/* BS4 inner product (arXiv 2009.10917, CG vector-operation list): *result =
 * sum x[i]*y[i] into the device double `result`, same reduction guarantees as
 * bs_norm. x, y contiguous double[n]. */
int bs_dot(bs_ctx *ctx, int64_t n, const double *x, const double *y, double *result,
           void *stream);

/* BS5 fused CG update (arXiv 2009.10917, BS test list: CG steps 8-10 in one
 * pass, saving a read and a write of r): x[i] = x[i] + (alpha*p[i]);
 * r[i] = r[i] - (alpha*q[i]) (bit-exact), and *rr = sum of the updated r[i]^2
 * into the device double `rr` (reduction guarantees as bs_norm). p, q, x, r
 * contiguous double[n]. x and r are written: neither may overlap the other,
 * p or q (BS_EINVAL); p and q are only read and may be the same array. */
int bs_cg_update(bs_ctx *ctx, int64_t n, double alpha, const double *p, const double *q,
                 double *x, double *r, double *rr, void *stream);

/* BS7 scatter v_L = Z v_G (arXiv 2009.10917, eq. 3 and the scatterIds array
 * of the implementation section; arXiv 1506.05996, local-to-global table):
 * v_local[i] = v_global[l2g[i]] for l2g[i] >= 0, and +0.0 for a negative
 * (masked) id. l2g int32[n_local] in element-major local order; v_local
 * double[n_local]; v_global double[>= 1 + max id]. Ids are not range-checked
 * on the device: check tables once with bs_validate_l2g. n_local > INT32_MAX
 * is BS_ERANGE. */
int bs_scatter(bs_ctx *ctx, int64_t n_local, const int32_t *l2g, const double *v_global,
               double *v_local, void *stream);

/* BS6 gather v_G = Z^T v_L (arXiv 2009.10917, eq. 3, the gather operator and
 * the CSR/blockStarts kernel of the implementation section; arXiv
 * 1506.05996, global-to-local table): v_global[g] = sum of v_local[ids[j]] for
 * off[g] <= j < off[g+1], added left to right starting from +0.0, so with ids
 * ascending inside each row the result is bit-identical to Z^T v_L summed in
 * ascending local index. off int32[n_global+1], ids int32[off[n_global]],
 * v_local double[> max id], v_global double[n_global]. block_starts NULL
 * cuts the rows into fixed spans of 512, each staged in LDS (up to 2048
 * entries, else read from global memory): 2-5% slower than a plan on the
 * box and tet-split meshes measured. Otherwise the n_blocks blocks of int32[4]
 * that bs_gather_plan makes (16-byte aligned, else BS_EALIGN) select the
 * plan kernel, launched in the plan's order. Same bits either way. Neither the
 * CSR nor the plan is range-checked on the device: pass tables built by
 * bs_index_g2l and bs_gather_plan, or check others once with
 * bs_validate_g2l and bs_validate_plan. n_global >= INT32_MAX is
 * BS_ERANGE. */
int bs_gather(bs_ctx *ctx, int64_t n_global, const int32_t *off, const int32_t *ids,
              const double *v_local, double *v_global, const int32_t *block_starts,
              int64_t n_blocks, void *stream);

/* BS6 gather with the inner product of the CG iteration folded into the same
 * pass (arXiv 2009.10917, the CG vector-operation list: q = A p followed by
 * p.q): v_global as bs_gather computes it (same bits), and *result =
 * sum over g of v_global[g]*w[g] into the device double `result`, reduced in
 * a fixed order (repeatable bits, relative 1e-12 of the exact value). w is
 * double[n_global], distinct from v_global. Other arguments and errors as
 * bs_gather; BS_ERANGE if the gather would use more blocks than the context
 * holds partials (bs_ctx_info). */
int bs_gather_dot(bs_ctx *ctx, int64_t n_global, const int32_t *off, const int32_t *ids,
                  const double *v_local, double *v_global, const int32_t *block_starts,
                  int64_t n_blocks, const double *w, double *result, void *stream);

/* Device-resident unpreconditioned Conjugate Gradient on A = Z^T Z (the
 * element operator taken as the identity: the streaming skeleton of the CG
 * method whose vector operations the BS tests isolate, arXiv 2009.10917, CG
 * vector-operation list and the fused update of the BS tests). Runs up to
 * `iters` iterations on `stream` with no host synchronisation: alpha and beta
 * are computed on the device. Each iteration: p_local = Z p (bs_scatter);
 * q = Z^T p_local with p.q in the same pass (bs_gather_dot); alpha = rr/p.q;
 * x += alpha p, r -= alpha q, rr' = r.r (bs_cg_update); beta = rr'/rr;
 * p = (1 r) + (beta p) (bs_axpy). On entry x, r, p hold x0, r0 = b - A x0 and
 * p0 = r0 (for x0 = 0: r = p = b). rr_hist (device double[iters+1]) receives
 * r.r before the first iteration and after each; once rr <= tol^2 * rr0 (or
 * rr == 0) the remaining iterations do nothing and their entries stay -1.
 * x, r, p, q: device double[n_global]; p_local: device double[n_local];
 * no two of these five may overlap (BS_EINVAL); all 16-byte aligned
 * (BS_EALIGN), l2g 8-byte aligned.
 * l2g, off, ids, block_starts as bs_scatter / bs_gather. Uses the context's
 * scratch: one solve at a time per context. When the iteration's vectors and
 * tables together fit in the device's 256 MB last-level cache, its kernels
 * read and write them with the ordinary cache policy so that each kernel
 * finds what the previous one left there; larger working sets stream
 * non-temporally, like the standalone operations, except that while r and p
 * alone fit (16 n_global bytes up to 210 MB) the update passes them to the
 * direction update p = r + beta p through the cache. The results are the
 * same bits either way. */
int bs_cg_solve(bs_ctx *ctx, int64_t n_global, int64_t n_local, const int32_t *l2g,
                const int32_t *off, const int32_t *ids, const int32_t *block_starts,
                int64_t n_blocks, double *x, double *r, double *p, double *q, double *p_local,
                int iters, double tol, double *rr_hist, void *stream);

/* bs_cg_solve without a context and without any allocation, for callers
 * that cannot allocate device memory: code under HIP stream or graph
 * capture, tight solver or serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results (the same bits) and errors as bs_cg_solve, on the
 * calling thread's current HIP device. Its reduction scratch (ticket
 * counters, CG scalars and up to 131072 partials, about 1 MiB) is a static
 * device array of the library that every GPU it runs on holds until the
 * process ends; the first call on a device looks up that array's address,
 * later calls allocate and look up nothing. Each call first clears the
 * counters with a small kernel on `stream` (no memset, so the call can be
 * captured). All calls on one GPU share that one array: calls that overlap
 * in time on a GPU (different streams, or host threads racing) race on it
 * and give wrong results; order them. A gather with more than 131072 blocks
 * (block_starts with n_blocks > 131072, or n_global > 67108864 without a
 * plan) is BS_ERANGE, with nothing enqueued. BS_EHIP if the device or the
 * array's address cannot be queried; BS_EINVAL on a device numbered 64 or
 * above. Make the first call on a device outside stream capture, or accept
 * that its one-time address lookup happens inside it. */
int bs_cg_solve_static(int64_t n_global, int64_t n_local, const int32_t *l2g, const int32_t *off,
                       const int32_t *ids, const int32_t *block_starts, int64_t n_blocks, double *x, double *r,
                       double *p, double *q, double *p_local, int iters, double tol, double *rr_hist,
                       void *stream);

/* ---------------------------------------------------- host-side tables --
 * These run on the host, need no GPU, and write caller-allocated host arrays.
 */

/* Sizes of a box mesh of ex*ey*ez hexahedra of order `order`:
 * *n_local = ex*ey*ez*(order+1)^3, *n_global = (ex*order+1)(ey*order+1)(ez*order+1).
 * BS_EINVAL for a dimension or order < 1, BS_ERANGE if either exceeds INT32_MAX. */
int bs_mesh_box_count(int ex, int ey, int ez, int order, int64_t *n_local, int64_t *n_global);

/* I_l->g of the structured box of unit hexahedra with (order+1)^3 GLL nodes
 * each (arXiv 2009.10917, eqs. 1-3; arXiv 1506.05996, local-to-global
 * table). Element e = cx + ex*(cy + ey*cz); slot s of local storage holds
 * element elem_perm[s] (NULL: s). Within a slot the node (i,j,k) sits at
 * s*(order+1)^3 + i + (order+1)*(j + (order+1)*k). Its lexicographic global
 * id is gx + Gx*(gy + Gy*gz) with gx = cx*order + i, Gx = ex*order + 1 (same for
 * y, z); node_perm (NULL: identity) renames id g to node_perm[g]. Both
 * permutations must be permutations (checked: BS_EINVAL). l2g receives
 * int32[n_local]. Sizes as bs_mesh_box_count; BS_ENOMEM if the host memory
 * for the permutation check is not available. */
int bs_mesh_box_l2g(int ex, int ey, int ez, int order, const int32_t *elem_perm,
                    const int32_t *node_perm, int32_t *l2g);

/* I_l->g of an unstructured mesh of hexahedra given by corner vertices
 * (arXiv 2009.10917, the unstructured hexahedral mesh of the CEED
 * formulation section; arXiv 1506.05996, local-to-global table: one global
 * number per GLL node of the mesh, so nodes on a shared vertex, edge or face
 * get one id whatever the orientation of the elements that share it).
 *   ev        int32[n_elements * 8], host: ev[8e + c] is the vertex at corner
 *             c = a + 2b + 4d of element e, (a, b, d) in {0,1}^3 the corner of
 *             the reference cube along (x, y, z) -- local node (a*order,
 *             b*order, d*order). Ids in [0, n_vertices); unused ids allowed.
 *   l2g       int32[n_elements * (order+1)^3], host, written: element by
 *             element, node (i,j,k) at i + (order+1)(j + (order+1)k).
 *   n_global  written: the number of global nodes. Ids are numbered in order
 *             of first appearance in l2g.
 * Entities are identified by their vertex sets: two elements share an edge
 * when they share its two end vertices, a face when they share its four. A
 * mesh in which distinct edges or faces have the same vertex set (a periodic
 * direction of fewer than 3 elements) cannot be told apart and is shared.
 * BS_EINVAL: bad sizes or NULL, a vertex id out of range, an element with a
 * repeated vertex, or a face whose four vertices two elements connect in
 * different cyclic orders (not a conforming mesh). BS_ERANGE: n_elements *
 * (order+1)^3 above INT32_MAX or order > 2047. BS_ENOMEM: no host memory.
 * Nothing is written to n_global on error; l2g may be partly written. */
int bs_mesh_hex_l2g(int64_t n_elements, int order, int64_t n_vertices, const int32_t *ev,
                    int32_t *l2g, int64_t *n_global);

/* A storage order for the elements of an unstructured hex mesh that keeps
 * neighbours near in memory (arXiv 2009.10917, the gather paragraph: local
 * spatial locality of the elements helps the reads of the local vector;
 * arXiv 1506.05996, the mesh-setup tables): the elements sorted along a 3D
 * Hilbert curve through their centroids (J. Skilling, "Programming the
 * Hilbert curve", AIP Conf. Proc. 707, 2004), on a grid of 2^21 cells per
 * axis over the centroids' bounding cube; elements in one cell keep their
 * order. perm receives int32[n_elements]: perm[s] is the element to store in
 * slot s. Reorder the corner vertices (and coordinates) by it before
 * bs_mesh_hex_l2g, whose first-appearance numbering then makes the global
 * ids follow the curve too. xe as for bs_mesh_hex_mass. BS_EINVAL: NULL with
 * n_elements > 0, n_elements < 0, a non-finite coordinate; BS_ERANGE:
 * n_elements > INT32_MAX; BS_ENOMEM: no host memory. */
int bs_mesh_hex_order(int64_t n_elements, const double *xe, int32_t *perm);

/* Gauss-Lobatto-Legendre points and weights of degree `order` on [-1, 1]:
 * nodes double[order+1] ascending (the end points and the roots of P_order'),
 * weights double[order+1], w_i = 2 / (order (order+1) P_order(r_i)^2). These
 * are the element nodes of arXiv 2009.10917 eqs. 1-2. BS_EINVAL for order < 1
 * or a NULL output. */
int bs_gll(int order, double *nodes, double *weights);

/* Local lumped-mass weights of the box mesh of unit hexahedra: every element's
 * node (i,j,k) gets w_i w_j w_k / 8 (GLL weights times the Jacobian of the map
 * from [-1,1]^3 onto the unit cube), in the local layout of bs_mesh_box_l2g.
 * The lumped global mass is their gather, m = Z^T w_L (arXiv 1506.05996,
 * coarse-grid correction: m_N as the global components of the local weights).
 * w_local receives double[n_local]. Errors as bs_mesh_box_count, BS_EINVAL
 * for a NULL output, BS_ENOMEM without host memory for one element's block. */
int bs_mesh_box_mass(int ex, int ey, int ez, int order, double *w_local);

/* Local lumped-mass weights of an unstructured hex mesh (arXiv 1506.05996,
 * the element geometry as a map from the reference cube and the lumped mass
 * as quadrature weights times the Jacobian at the nodes): node (i,j,k) of
 * element e gets w_i w_j w_k |det J(r_i, r_j, r_k)| with J the Jacobian of
 * the element's trilinear map. The lumped global mass is their gather.
 *   xe        double[n_elements * 24], host: xe[24e + 3c + a] is coordinate a
 *             of corner c = a + 2b + 4d of element e (the corner order of
 *             bs_mesh_hex_l2g).
 *   w_local   double[n_elements * (order+1)^3], host, written in the local
 *             layout of bs_mesh_hex_l2g.
 * BS_EINVAL: bad sizes or NULL, or an element whose Jacobian vanishes or
 * changes sign at one of its nodes (a degenerate or tangled element; w_local
 * may then be partly written). BS_ERANGE as bs_mesh_hex_l2g. BS_ENOMEM: no
 * host memory. */
int bs_mesh_hex_mass(int64_t n_elements, int order, const double *xe, double *w_local);

/* Check that every id is < n_global (negative ids are masks): BS_OK or
 * BS_EINVAL. */
int bs_validate_l2g(int64_t n_local, int64_t n_global, const int32_t *l2g);

/* Check a CSR form of I_g->l before a gather trusts it (the device reads it
 * unchecked): off[0] == 0, off nondecreasing, off[n_global] <= n_local,
 * every id in [0, n_local) and ids strictly ascending inside each row (the
 * order the gather adds in; a repeated id would count an entry twice). With
 * l2g (int32[n_local], may be NULL) also that the CSR is exactly its
 * transpose: l2g[ids[j]] == g for every entry j of row g, and every unmasked
 * local entry appears once. off int32[n_global+1], ids int32[off[n_global]].
 * BS_OK or BS_EINVAL; BS_ERANGE for sizes beyond int32 indices. */
int bs_validate_g2l(int64_t n_global, int64_t n_local, const int32_t *off, const int32_t *ids, const int32_t *l2g);

/* Check a gather plan before a gather trusts it, against the CSR offsets off
 * int32[n_global+1] it was built for: plan holds n_blocks blocks of int32[4]
 * (first row, end row, off[first row], off[end row]) in any launch order;
 * every block is a non-empty row range with the offsets of its ends, and the
 * ranges tile [0, n_global) once; 1 <= n_blocks <= n_global (n_global == 0:
 * n_blocks == 0). Blocks above the LDS stage's capacity are allowed (the
 * kernel reads them from global memory). BS_OK or BS_EINVAL; BS_ERANGE for
 * n_global >= INT32_MAX; BS_ENOMEM without host memory for the sort. */
int bs_validate_plan(int64_t n_global, const int32_t *off, const int32_t *plan, int64_t n_blocks);

/* CSR form of I_g->l: a stable counting-sort transpose of l2g. off receives
 * int32[n_global+1]; ids receives the off[n_global] local indices (at most
 * n_local; masked entries are left out), ascending within each row. An id
 * >= n_global is BS_EINVAL (off and ids may then be partly written);
 * n_local > INT32_MAX or n_global >= INT32_MAX is BS_ERANGE; BS_ENOMEM
 * without host memory for the n_global fill cursors. */
int bs_index_g2l(int64_t n_local, int64_t n_global, const int32_t *l2g, int32_t *off,
                 int32_t *ids);

/* blockStarts of the LDS-staged gather (arXiv 2009.10917, implementation
 * section, BS6): rows are cut into consecutive blocks so that each thread
 * block reads and writes about the same amount: greedily, a block takes rows
 * while it holds at most nodes_per_block rows and at most nodes_per_block CSR
 * entries (a single longer row gets a block of its own). Every block but the
 * last then ends on a multiple of 16 rows, rounding its greedy end down,
 * unless no multiple of 16 lies after its first row: so each block writes
 * whole 128-byte lines of a 128-byte-aligned v_global.
 *
 * plan receives one int32[4] per block, (first row, end row, off[first row],
 * off[end row]), in the order the gather launches them: n_blocks * 4 int32
 * (capacity 4*n_global suffices). The launch order places the blocks on the
 * eight XCDs of MI355X, to which the hardware hands workgroup s of a launch
 * as s mod 8. region_entries == 0: each XCD takes runs of 8 consecutive
 * blocks (ids may be NULL). region_entries > 0: the local vector interleaves
 * eight regions of the mesh in runs of region_entries entries (local index i
 * in region (i / region_entries) mod 8, the layout bs_mesh_xcd_interleave
 * makes with region_entries = chunk * (N+1)^3); each block belongs to the
 * region of its first entry, ids[off[first row]], and XCD x takes the blocks
 * of region x in row order (an XCD whose region has run out takes from the
 * region with the most left). ids is then the CSR ids of off.
 * nodes_per_block must be in [1, 1024] (BS_EINVAL): the gather kernel stages
 * up to 1024 entries per block in LDS. off must be non-decreasing from a
 * non-negative off[0], and in region placement a block's first id must be
 * non-negative (BS_EINVAL otherwise; ids must hold off[n_global] entries).
 * BS_ENOMEM without host memory for the row starts. */
int bs_gather_plan(int64_t n_global, const int32_t *off, const int32_t *ids, int nodes_per_block,
                   int64_t region_entries, int32_t *plan, int64_t *n_blocks);

/* Storage order of n_elements elements that gives each XCD its own region of
 * the mesh while all eight work in one narrow window of memory: the given
 * order, cut into eight consecutive regions, is interleaved in runs of chunk
 * elements, region x taking the storage slots s with (s / chunk) mod 8 == x
 * (region x is the next as many elements of the given order, in order).
 * perm receives int32[n_elements], the element of the given order stored at
 * slot s. The caller reorders its element corners by perm before
 * bs_mesh_hex_l2g and builds the gather plan with region_entries = chunk *
 * (N+1)^3; the regions should be spatially compact, so the given order should
 * be a local one (a generator's sweep, or bs_mesh_hex_order). Measured on a
 * tet-split mesh of 11^3 cubes at order 7 with runs of 64: gather counter
 * traffic 1.20x -> 1.08x the algorithmic bytes, 60.8 -> 60.5 us.
 * BS_EINVAL for chunk < 1, BS_ERANGE for n_elements > INT32_MAX; a chunk of
 * n_elements or more gives the identity. */
int bs_mesh_xcd_interleave(int64_t n_elements, int64_t chunk, int32_t *perm);

/* ------------------------------------------------------------ measurement --
 * Host-timed loop for the streaming-model fit (arXiv 2009.10917, the
 * performance model: the time of one test is measured on the host around
 * back-to-back launches, and fitted to T(B) = T0 + B / W_max, eq. 8). */
typedef enum {
    BS_OP_COPY = 0,      /* n = length; set: x, y                              */
    BS_OP_AXPY = 1,      /* n = length; set: x, y                              */
    BS_OP_NORM = 2,      /* n = length; set: x                                 */
    BS_OP_DOT = 3,       /* n = length; set: x, y                              */
    BS_OP_CG_UPDATE = 4, /* n = length; set: p, q, x, r                        */
    BS_OP_SCALE = 5,     /* n = length; set: x, d, y                           */
    BS_OP_SCATTER = 6,   /* n = n_local; set: l2g, v_global, v_local           */
    BS_OP_GATHER = 7     /* n = n_global; set: off, ids, v_local, v_global,
                            block_starts (NULL: no plan; n_blocks its count)   */
} bs_op;

#define BS_BENCH_SET 6   /* pointers per set in bs_bench_loop */

/* Synchronise `stream`, then issue `reps` calls of operation `op` (a bs_op)
 * back to back on it, call k using pointer set k mod n_sets, synchronise
 * again, and write the host seconds in between to *seconds. sets holds
 * n_sets groups of BS_BENCH_SET device pointers, each group laid out as
 * listed above (unused slots NULL); alpha and beta are the scalars of AXPY
 * and the fused update; reductions write to the device double `result`.
 * Each call checks its arguments as the operation itself does; the first
 * failing status is returned after the stream is synchronised (*seconds is
 * then not written). BS_EINVAL: ctx, sets or seconds NULL, n < 0,
 * n_sets < 1, reps < 1, or an unknown op. */
int bs_bench_loop(bs_ctx *ctx, int op, int64_t n, double alpha, double beta, int64_t n_blocks,
                  int n_sets, void *const *sets, double *result, int reps, void *stream,
                  double *seconds);

#ifdef __cplusplus
}
#endif

#endif /* BS_H */
