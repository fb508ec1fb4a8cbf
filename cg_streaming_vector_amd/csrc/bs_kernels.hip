// bs_kernels.hip -- gfx950 kernels and C ABI of the Benchmark Streaming ops.
//
// The seven streaming operations of "Portable high-order finite element
// kernels I: Streaming Operations" (arXiv 2009.10917): BS1 copy, BS2 AXPY,
// BS3 norm, BS4 inner product, BS5 fused CG update, BS6 gather and BS7
// scatter. All are bound by HBM bandwidth (at most 0.25 flop per byte), so the
// kernels are written for bytes in flight, not for arithmetic:
//  - 128-bit (two-double) loads and stores, several per lane in flight before
//    any is consumed, coalesced across the 64-lane wavefront;
//  - grid-stride loops over a grid sized to the compute-unit count for the
//    vector ops, so the reduction partials are few and their order fixed;
//  - reductions: per-lane accumulation, then a wavefront butterfly through
//    cross-lane shuffles, then the block's wavefronts through LDS, one partial
//    per block, and the last block to finish (a completion counter, no
//    atomics on values) sums the partials in a fixed order;
//  - scatter and gather remap block indices so that each of the 8 XCDs walks
//    one contiguous eighth of the index table, keeping the reuse of shared
//    nodes inside one XCD's L2.
// No MFMA: nothing here is a dense contraction.
//
// Bit-exactness: the file is compiled with -ffp-contract=off and the pragma
// below, so a*x + b*y is two rounded products and one rounded sum, as in the
// IEEE definition. Reductions use explicit fma for the per-lane sums (they
// are checked against a relative tolerance, not bits).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <new>

#include "bs.h"

#pragma clang fp contract(off)

namespace {

constexpr int kBlock = 256;          // threads per block: 4 wavefronts
constexpr int kWave = 64;            // gfx950 wavefront width
constexpr int kUnroll = 4;           // 16-byte loads per lane per array per iteration
constexpr int kBlocksPerCU = 8;      // grid of the vector ops: CUs * this
constexpr int kMaxPartials = 16384;  // reduction scratch (blocks of one launch)
constexpr int kXcds = 8;             // MI355X: 8 XCDs of 32 CUs, round-robin dispatch
constexpr int kScatterPerLane = 4;   // local entries per lane in the scatter kernel
constexpr int kGatherLds = 4096;     // entries a gather block may stage in LDS

typedef double d2 __attribute__((ext_vector_type(2)));
typedef int i4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ d2 ld2(const d2 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st2(d2 *p, d2 v) { __builtin_nontemporal_store(v, p); }

// ------------------------------------------------------------ reductions --

// Butterfly over the 64 lanes of a wavefront; every lane ends with the sum.
__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// Sum over the block; the result is valid in thread 0.
__device__ __forceinline__ double block_sum(double v)
{
    __shared__ double wsum[kBlock / kWave];
    v = wave_sum(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) wsum[w] = v;
    __syncthreads();
    double s = 0.0;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 0; i < kBlock / kWave; ++i) s += wsum[i];
    }
    return s;
}

// Stores the block's partial, and in the last block to finish sums all
// partials in index order (then a fixed tree) and writes the result. The
// counter is left at zero for the next launch on the same context.
__device__ __forceinline__ void finish_reduction(double part, double *partials,
                                                 unsigned *counter, double *out, bool take_sqrt)
{
    __shared__ bool is_last;
    if (threadIdx.x == 0) {
        __hip_atomic_store(&partials[blockIdx.x], part, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        unsigned done = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        is_last = (done == gridDim.x - 1);
    }
    __syncthreads();
    if (!is_last) return;
    double s = 0.0;
    for (unsigned i = threadIdx.x; i < gridDim.x; i += kBlock)
        s += __hip_atomic_load(&partials[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s = block_sum(s);
    if (threadIdx.x == 0) {
        *out = take_sqrt ? std::sqrt(s) : s;
        __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ------------------------------------------------------- vector layout ----
// A vector of n doubles is split into an optional one-element head (when the
// pointers are 8 but not 16 byte aligned), a 16-byte aligned body of n2 pairs,
// and an optional one-element tail. Block 0 lane 0 handles head and tail.
struct Split {
    int64_t head;  // 0 or 1 leading scalar elements
    int64_t n2;    // pairs in the body
    int64_t tail;  // index of the trailing scalar element, or -1
};

__host__ __device__ inline Split split_of(int64_t n, int64_t head)
{
    Split s;
    s.head = (head && n > 0) ? 1 : 0;
    const int64_t rest = n - s.head;
    s.n2 = rest / 2;
    s.tail = (rest & 1) ? (n - 1) : -1;
    return s;
}

// ------------------------------------------------------------ BS1 copy ----
__global__ __launch_bounds__(kBlock) void k_copy(Split sp, const double *__restrict__ x,
                                                 double *__restrict__ y)
{
    const d2 *xv = reinterpret_cast<const d2 *>(x + sp.head);
    d2 *yv = reinterpret_cast<d2 *>(y + sp.head);
    const int64_t stride = (int64_t)gridDim.x * kBlock * kUnroll;
    int64_t i = (int64_t)blockIdx.x * kBlock * kUnroll + threadIdx.x;
    for (; i + (kUnroll - 1) * kBlock < sp.n2; i += stride) {
        d2 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = ld2(xv + i + u * kBlock);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) st2(yv + i + u * kBlock, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
        if (i + u * kBlock < sp.n2) st2(yv + i + u * kBlock, ld2(xv + i + u * kBlock));
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (sp.head) y[0] = x[0];
        if (sp.tail >= 0) y[sp.tail] = x[sp.tail];
    }
}

// ------------------------------------------------------------ BS2 AXPY ----
__device__ __forceinline__ d2 axpy2(double a, d2 x, double b, d2 y)
{
    d2 r;
    r.x = a * x.x + b * y.x;  // two rounded products, one rounded sum (contract off)
    r.y = a * x.y + b * y.y;
    return r;
}

__global__ __launch_bounds__(kBlock) void k_axpy(Split sp, double a, const double *x, double b,
                                                 double *y)
{
    const d2 *xv = reinterpret_cast<const d2 *>(x + sp.head);
    d2 *yv = reinterpret_cast<d2 *>(y + sp.head);
    const int64_t stride = (int64_t)gridDim.x * kBlock * kUnroll;
    int64_t i = (int64_t)blockIdx.x * kBlock * kUnroll + threadIdx.x;
    for (; i + (kUnroll - 1) * kBlock < sp.n2; i += stride) {
        d2 vx[kUnroll], vy[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            vx[u] = ld2(xv + i + u * kBlock);
            vy[u] = ld2(yv + i + u * kBlock);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) st2(yv + i + u * kBlock, axpy2(a, vx[u], b, vy[u]));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t k = i + u * kBlock;
        if (k < sp.n2) st2(yv + k, axpy2(a, ld2(xv + k), b, ld2(yv + k)));
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (sp.head) y[0] = a * x[0] + b * y[0];
        if (sp.tail >= 0) y[sp.tail] = a * x[sp.tail] + b * y[sp.tail];
    }
}

// ------------------------------------------------- BS3 norm, BS4 dot ----
// One kernel for both: with y == nullptr it sums x[i]^2 and takes the root.
template <bool kSquare>
__global__ __launch_bounds__(kBlock) void k_dot(Split sp, const double *x, const double *y,
                                                double *partials, unsigned *counter, double *out)
{
    const d2 *xv = reinterpret_cast<const d2 *>(x + sp.head);
    const d2 *yv = reinterpret_cast<const d2 *>((kSquare ? x : y) + sp.head);
    const int64_t stride = (int64_t)gridDim.x * kBlock * kUnroll;
    int64_t i = (int64_t)blockIdx.x * kBlock * kUnroll + threadIdx.x;
    double acc0 = 0.0, acc1 = 0.0;
    for (; i + (kUnroll - 1) * kBlock < sp.n2; i += stride) {
        d2 vx[kUnroll], vy[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            vx[u] = ld2(xv + i + u * kBlock);
            vy[u] = kSquare ? vx[u] : ld2(yv + i + u * kBlock);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            acc0 = __builtin_fma(vx[u].x, vy[u].x, acc0);
            acc1 = __builtin_fma(vx[u].y, vy[u].y, acc1);
        }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t k = i + u * kBlock;
        if (k < sp.n2) {
            const d2 a = ld2(xv + k);
            const d2 b = kSquare ? a : ld2(yv + k);
            acc0 = __builtin_fma(a.x, b.x, acc0);
            acc1 = __builtin_fma(a.y, b.y, acc1);
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        const double *yy = kSquare ? x : y;
        if (sp.head) acc0 = __builtin_fma(x[0], yy[0], acc0);
        if (sp.tail >= 0) acc1 = __builtin_fma(x[sp.tail], yy[sp.tail], acc1);
    }
    const double part = block_sum(acc0 + acc1);
    finish_reduction(part, partials, counter, out, kSquare);
}

// -------------------------------------------------- BS5 fused CG update ----
__global__ __launch_bounds__(kBlock) void k_cg_update(Split sp, double a, const double *p,
                                                      const double *q, double *x, double *r,
                                                      double *partials, unsigned *counter,
                                                      double *out)
{
    const d2 *pv = reinterpret_cast<const d2 *>(p + sp.head);
    const d2 *qv = reinterpret_cast<const d2 *>(q + sp.head);
    d2 *xv = reinterpret_cast<d2 *>(x + sp.head);
    d2 *rv = reinterpret_cast<d2 *>(r + sp.head);
    const int64_t stride = (int64_t)gridDim.x * kBlock * kUnroll;
    int64_t i = (int64_t)blockIdx.x * kBlock * kUnroll + threadIdx.x;
    double acc0 = 0.0, acc1 = 0.0;
    for (; i + (kUnroll - 1) * kBlock < sp.n2; i += stride) {
        d2 vp[kUnroll], vq[kUnroll], vx[kUnroll], vr[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            vp[u] = ld2(pv + i + u * kBlock);
            vq[u] = ld2(qv + i + u * kBlock);
            vx[u] = ld2(xv + i + u * kBlock);
            vr[u] = ld2(rv + i + u * kBlock);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            d2 nx, nr;
            nx.x = vx[u].x + a * vp[u].x;
            nx.y = vx[u].y + a * vp[u].y;
            nr.x = vr[u].x - a * vq[u].x;
            nr.y = vr[u].y - a * vq[u].y;
            st2(xv + i + u * kBlock, nx);
            st2(rv + i + u * kBlock, nr);
            acc0 = __builtin_fma(nr.x, nr.x, acc0);
            acc1 = __builtin_fma(nr.y, nr.y, acc1);
        }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t k = i + u * kBlock;
        if (k < sp.n2) {
            const d2 vp1 = ld2(pv + k), vq1 = ld2(qv + k), vx1 = ld2(xv + k), vr1 = ld2(rv + k);
            d2 nx, nr;
            nx.x = vx1.x + a * vp1.x;
            nx.y = vx1.y + a * vp1.y;
            nr.x = vr1.x - a * vq1.x;
            nr.y = vr1.y - a * vq1.y;
            st2(xv + k, nx);
            st2(rv + k, nr);
            acc0 = __builtin_fma(nr.x, nr.x, acc0);
            acc1 = __builtin_fma(nr.y, nr.y, acc1);
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (sp.head) {
            x[0] = x[0] + a * p[0];
            const double nr = r[0] - a * q[0];
            r[0] = nr;
            acc0 = __builtin_fma(nr, nr, acc0);
        }
        if (sp.tail >= 0) {
            const int64_t t = sp.tail;
            x[t] = x[t] + a * p[t];
            const double nr = r[t] - a * q[t];
            r[t] = nr;
            acc1 = __builtin_fma(nr, nr, acc1);
        }
    }
    const double part = block_sum(acc0 + acc1);
    finish_reduction(part, partials, counter, out, false);
}

// n == 0 reductions still store +0.0 (no memset: a kernel keeps it capturable).
__global__ void k_store_zero(double *out) { *out = 0.0; }

// ------------------------------------------------------ XCD-aware order ----
// Workgroups are dispatched round-robin over the XCDs: block b runs on XCD
// b % 8. Map the first 8*floor(nb/8) blocks so that XCD x takes the tiles
// x*q .. x*q+q-1 in order (q = floor(nb/8)); the remainder keeps its index.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t nb)
{
    const int64_t q = nb / kXcds;
    if (b >= q * kXcds) return b;
    return (b % kXcds) * q + b / kXcds;
}

// --------------------------------------------------------- BS7 scatter ----
// Each lane handles kScatterPerLane consecutive local entries: one 16-byte
// index load, four reads of v_G, two 16-byte stores. Tiles are kBlock lanes.
__global__ __launch_bounds__(kBlock) void k_scatter(int64_t nl, const int32_t *__restrict__ l2g,
                                                    const double *__restrict__ vg,
                                                    double *__restrict__ vl)
{
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t i0 = (tile * kBlock + threadIdx.x) * kScatterPerLane;
    if (i0 + kScatterPerLane <= nl) {
        const i4 id = __builtin_nontemporal_load(reinterpret_cast<const i4 *>(l2g + i0));
        d2 a, b;
        a.x = id.x >= 0 ? vg[id.x] : 0.0;
        a.y = id.y >= 0 ? vg[id.y] : 0.0;
        b.x = id.z >= 0 ? vg[id.z] : 0.0;
        b.y = id.w >= 0 ? vg[id.w] : 0.0;
        st2(reinterpret_cast<d2 *>(vl + i0), a);
        st2(reinterpret_cast<d2 *>(vl + i0 + 2), b);
    } else {
        for (int64_t i = i0; i < nl; ++i) {
            const int32_t g = l2g[i];
            vl[i] = g >= 0 ? vg[g] : 0.0;
        }
    }
}

// Fallback for index or value pointers without 16-byte alignment.
__global__ __launch_bounds__(kBlock) void k_scatter_scalar(int64_t nl, const int32_t *l2g,
                                                           const double *vg, double *vl)
{
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t i = tile * kBlock + threadIdx.x;
    if (i < nl) {
        const int32_t g = l2g[i];
        vl[i] = g >= 0 ? vg[g] : 0.0;
    }
}

// ---------------------------------------------------------- BS6 gather ----
// Row-per-lane: lane g walks ids[off[g] .. off[g+1]) and sums from +0.0.
__global__ __launch_bounds__(kBlock) void k_gather_rows(int64_t ng, const int32_t *__restrict__ off,
                                                        const int32_t *__restrict__ ids,
                                                        const double *__restrict__ vl,
                                                        double *__restrict__ vg)
{
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t g = tile * kBlock + threadIdx.x;
    if (g >= ng) return;
    const int32_t a = off[g], b = off[g + 1];
    double s = 0.0;
    for (int32_t j = a; j < b; ++j) s = s + vl[ids[j]];
    __builtin_nontemporal_store(s, vg + g);
}

// LDS-staged, after the blockStarts kernel of the paper: block b owns rows
// bs[b] .. bs[b+1]); it first reads the rows' CSR entries with consecutive
// lanes on consecutive entries and stages v_L[ids[j]] in LDS, then each lane
// sums its rows from LDS in ascending entry order. A block holding more than
// kGatherLds entries (a single very long row) reads from global memory.
__global__ __launch_bounds__(kBlock) void k_gather_lds(const int32_t *__restrict__ bstart,
                                                       const int32_t *__restrict__ off,
                                                       const int32_t *__restrict__ ids,
                                                       const double *__restrict__ vl,
                                                       double *__restrict__ vg)
{
    __shared__ double stage[kGatherLds];
    const int64_t blk = xcd_tile(blockIdx.x, gridDim.x);
    const int32_t r0 = bstart[blk], r1 = bstart[blk + 1];
    const int32_t e0 = off[r0], e1 = off[r1];
    const int32_t ne = e1 - e0;
    if (ne <= kGatherLds) {
        for (int32_t t = threadIdx.x; t < ne; t += kBlock) stage[t] = vl[ids[e0 + t]];
        __syncthreads();
        for (int32_t g = r0 + threadIdx.x; g < r1; g += kBlock) {
            const int32_t a = off[g] - e0, b = off[g + 1] - e0;
            double s = 0.0;
            for (int32_t j = a; j < b; ++j) s = s + stage[j];
            __builtin_nontemporal_store(s, vg + g);
        }
    } else {
        for (int32_t g = r0 + threadIdx.x; g < r1; g += kBlock) {
            double s = 0.0;
            for (int32_t j = off[g]; j < off[g + 1]; ++j) s = s + vl[ids[j]];
            vg[g] = s;
        }
    }
}

}  // namespace

// =================================================================== ABI ====

struct bs_ctx {
    int device;
    int cus;
    int max_partials;
    double *partials;
    unsigned *counter;
};

namespace {

inline bool misaligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

inline int launch_status()
{
    return hipGetLastError() == hipSuccess ? BS_OK : BS_EHIP;
}

// Grid of the grid-stride vector kernels: enough tiles to cover n2 pairs, at
// most CUs * kBlocksPerCU blocks (which also bounds the reduction partials).
inline unsigned vector_grid(const bs_ctx *c, int64_t n2)
{
    const int64_t per = (int64_t)kBlock * kUnroll;
    int64_t g = (n2 + per - 1) / per;
    const int64_t cap = (int64_t)c->cus * kBlocksPerCU;
    if (g > cap) g = cap;
    if (g > c->max_partials) g = c->max_partials;
    if (g < 1) g = 1;
    return (unsigned)g;
}

// All double pointers share the 16-byte phase? Then split off a one-element
// head when that phase is 8. Returns false if the phases differ.
inline bool common_head(const void *const *ptrs, int k, int64_t *head)
{
    const uintptr_t ph = reinterpret_cast<uintptr_t>(ptrs[0]) & 15;
    for (int i = 1; i < k; ++i)
        if ((reinterpret_cast<uintptr_t>(ptrs[i]) & 15) != ph) return false;
    *head = ph ? 1 : 0;
    return true;
}

// Scalar (8-byte) versions for operands whose 16-byte phases differ.
__global__ __launch_bounds__(kBlock) void k_copy_scalar(int64_t n, const double *x, double *y)
{
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock)
        y[i] = x[i];
}

__global__ __launch_bounds__(kBlock) void k_axpy_scalar(int64_t n, double a, const double *x,
                                                        double b, double *y)
{
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock)
        y[i] = a * x[i] + b * y[i];
}

template <bool kSquare>
__global__ __launch_bounds__(kBlock) void k_dot_scalar(int64_t n, const double *x, const double *y,
                                                       double *partials, unsigned *counter, double *out)
{
    double acc = 0.0;
    const double *yy = kSquare ? x : y;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock)
        acc = __builtin_fma(x[i], yy[i], acc);
    finish_reduction(block_sum(acc), partials, counter, out, kSquare);
}

__global__ __launch_bounds__(kBlock) void k_cg_update_scalar(int64_t n, double a, const double *p,
                                                             const double *q, double *x, double *r,
                                                             double *partials, unsigned *counter,
                                                             double *out)
{
    double acc = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock) {
        x[i] = x[i] + a * p[i];
        const double nr = r[i] - a * q[i];
        r[i] = nr;
        acc = __builtin_fma(nr, nr, acc);
    }
    finish_reduction(block_sum(acc), partials, counter, out, false);
}

inline unsigned scalar_grid(const bs_ctx *c, int64_t n)
{
    int64_t g = (n + kBlock - 1) / kBlock;
    const int64_t cap = (int64_t)c->cus * kBlocksPerCU;
    if (g > cap) g = cap;
    if (g > c->max_partials) g = c->max_partials;
    if (g < 1) g = 1;
    return (unsigned)g;
}

inline int check_ctx(const bs_ctx *c)
{
    if (!c) return BS_EINVAL;
    if (hipSetDevice(c->device) != hipSuccess) return BS_EHIP;
    return BS_OK;
}

}  // namespace

extern "C" {

const char *bs_strerror(int status)
{
    switch (status) {
        case BS_OK: return "ok";
        case BS_EINVAL: return "invalid argument";
        case BS_EALIGN: return "misaligned pointer";
        case BS_ERANGE: return "size out of range";
        case BS_EHIP: return "HIP runtime error";
        case BS_ENOMEM: return "out of memory";
        default: return "unknown status";
    }
}

int bs_version(void) { return 100; }

int bs_ctx_create(int device, bs_ctx **out)
{
    if (!out) return BS_EINVAL;
    *out = nullptr;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) return BS_EHIP;
    if (hipSetDevice(device) != hipSuccess) return BS_EHIP;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1)
        return BS_EHIP;
    bs_ctx *c = new (std::nothrow) bs_ctx;
    if (!c) return BS_ENOMEM;
    c->device = device;
    c->cus = cus;
    c->max_partials = kMaxPartials;
    c->partials = nullptr;
    c->counter = nullptr;
    if (hipMalloc(&c->partials, sizeof(double) * kMaxPartials) != hipSuccess ||
        hipMalloc(&c->counter, sizeof(unsigned)) != hipSuccess) {
        if (c->partials) (void)hipFree(c->partials);
        delete c;
        return BS_ENOMEM;
    }
    if (hipMemset(c->counter, 0, sizeof(unsigned)) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(c->partials);
        (void)hipFree(c->counter);
        delete c;
        return BS_EHIP;
    }
    *out = c;
    return BS_OK;
}

void bs_ctx_destroy(bs_ctx *c)
{
    if (!c) return;
    if (hipSetDevice(c->device) == hipSuccess) {
        (void)hipDeviceSynchronize();
        (void)hipFree(c->partials);
        (void)hipFree(c->counter);
    }
    delete c;
}

int bs_ctx_info(const bs_ctx *c, int *device, int *cu_count, int *max_partials)
{
    if (!c) return BS_EINVAL;
    if (device) *device = c->device;
    if (cu_count) *cu_count = c->cus;
    if (max_partials) *max_partials = c->max_partials;
    return BS_OK;
}

int bs_copy(bs_ctx *c, int64_t n, const double *x, double *y, void *stream)
{
    if (int s = check_ctx(c)) return s;
    if (n < 0 || (n > 0 && (!x || !y))) return BS_EINVAL;
    if (n == 0) return BS_OK;
    if (misaligned(x, 8) || misaligned(y, 8)) return BS_EALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const void *ptrs[2] = {x, y};
    int64_t head;
    if (common_head(ptrs, 2, &head)) {
        const Split sp = split_of(n, head);
        hipLaunchKernelGGL(k_copy, dim3(vector_grid(c, sp.n2)), dim3(kBlock), 0, st, sp, x, y);
    } else {
        hipLaunchKernelGGL(k_copy_scalar, dim3(scalar_grid(c, n)), dim3(kBlock), 0, st, n, x, y);
    }
    return launch_status();
}

int bs_axpy(bs_ctx *c, int64_t n, double alpha, const double *x, double beta, double *y, void *stream)
{
    if (int s = check_ctx(c)) return s;
    if (n < 0 || (n > 0 && (!x || !y))) return BS_EINVAL;
    if (n == 0) return BS_OK;
    if (misaligned(x, 8) || misaligned(y, 8)) return BS_EALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const void *ptrs[2] = {x, y};
    int64_t head;
    if (common_head(ptrs, 2, &head)) {
        const Split sp = split_of(n, head);
        hipLaunchKernelGGL(k_axpy, dim3(vector_grid(c, sp.n2)), dim3(kBlock), 0, st, sp, alpha, x, beta, y);
    } else {
        hipLaunchKernelGGL(k_axpy_scalar, dim3(scalar_grid(c, n)), dim3(kBlock), 0, st, n, alpha, x, beta, y);
    }
    return launch_status();
}

static int reduce_launch(bs_ctx *c, int64_t n, const double *x, const double *y, double *out,
                         bool square, hipStream_t st)
{
    if (n == 0) {
        hipLaunchKernelGGL(k_store_zero, dim3(1), dim3(1), 0, st, out);
        return launch_status();
    }
    const void *ptrs[2] = {x, square ? x : y};
    int64_t head;
    if (common_head(ptrs, 2, &head)) {
        const Split sp = split_of(n, head);
        const dim3 grid(vector_grid(c, sp.n2));
        if (square)
            hipLaunchKernelGGL(k_dot<true>, grid, dim3(kBlock), 0, st, sp, x, x, c->partials, c->counter, out);
        else
            hipLaunchKernelGGL(k_dot<false>, grid, dim3(kBlock), 0, st, sp, x, y, c->partials, c->counter, out);
    } else {
        const dim3 grid(scalar_grid(c, n));
        hipLaunchKernelGGL(k_dot_scalar<false>, grid, dim3(kBlock), 0, st, n, x, y, c->partials, c->counter, out);
    }
    return launch_status();
}

int bs_norm(bs_ctx *c, int64_t n, const double *x, double *result, void *stream)
{
    if (int s = check_ctx(c)) return s;
    if (n < 0 || !result || (n > 0 && !x)) return BS_EINVAL;
    if ((n > 0 && misaligned(x, 8)) || misaligned(result, 8)) return BS_EALIGN;
    return reduce_launch(c, n, x, x, result, true, static_cast<hipStream_t>(stream));
}

int bs_dot(bs_ctx *c, int64_t n, const double *x, const double *y, double *result, void *stream)
{
    if (int s = check_ctx(c)) return s;
    if (n < 0 || !result || (n > 0 && (!x || !y))) return BS_EINVAL;
    if ((n > 0 && (misaligned(x, 8) || misaligned(y, 8))) || misaligned(result, 8)) return BS_EALIGN;
    return reduce_launch(c, n, x, y, result, false, static_cast<hipStream_t>(stream));
}

int bs_cg_update(bs_ctx *c, int64_t n, double alpha, const double *p, const double *q, double *x,
                 double *r, double *rr, void *stream)
{
    if (int s = check_ctx(c)) return s;
    if (n < 0 || !rr || (n > 0 && (!p || !q || !x || !r))) return BS_EINVAL;
    if ((n > 0 && (misaligned(p, 8) || misaligned(q, 8) || misaligned(x, 8) || misaligned(r, 8))) ||
        misaligned(rr, 8))
        return BS_EALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (n == 0) {
        hipLaunchKernelGGL(k_store_zero, dim3(1), dim3(1), 0, st, rr);
        return launch_status();
    }
    const void *ptrs[4] = {p, q, x, r};
    int64_t head;
    if (common_head(ptrs, 4, &head)) {
        const Split sp = split_of(n, head);
        hipLaunchKernelGGL(k_cg_update, dim3(vector_grid(c, sp.n2)), dim3(kBlock), 0, st, sp, alpha, p, q, x,
                           r, c->partials, c->counter, rr);
    } else {
        hipLaunchKernelGGL(k_cg_update_scalar, dim3(scalar_grid(c, n)), dim3(kBlock), 0, st, n, alpha, p, q,
                           x, r, c->partials, c->counter, rr);
    }
    return launch_status();
}

int bs_scatter(bs_ctx *c, int64_t n_local, const int32_t *l2g, const double *v_global, double *v_local,
               void *stream)
{
    if (int s = check_ctx(c)) return s;
    if (n_local < 0 || (n_local > 0 && (!l2g || !v_global || !v_local))) return BS_EINVAL;
    if (n_local > INT32_MAX) return BS_ERANGE;
    if (n_local == 0) return BS_OK;
    if (misaligned(l2g, 4) || misaligned(v_global, 8) || misaligned(v_local, 8)) return BS_EALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!misaligned(l2g, 16) && !misaligned(v_local, 16)) {
        const int64_t per = (int64_t)kBlock * kScatterPerLane;
        const int64_t nb = (n_local + per - 1) / per;
        hipLaunchKernelGGL(k_scatter, dim3((unsigned)nb), dim3(kBlock), 0, st, n_local, l2g, v_global, v_local);
    } else {
        const int64_t nb = (n_local + kBlock - 1) / kBlock;
        hipLaunchKernelGGL(k_scatter_scalar, dim3((unsigned)nb), dim3(kBlock), 0, st, n_local, l2g, v_global,
                           v_local);
    }
    return launch_status();
}

int bs_gather(bs_ctx *c, int64_t n_global, const int32_t *off, const int32_t *ids, const double *v_local,
              double *v_global, const int32_t *block_starts, int64_t n_blocks, void *stream)
{
    if (int s = check_ctx(c)) return s;
    if (n_global < 0 || (n_global > 0 && (!off || !ids || !v_local || !v_global))) return BS_EINVAL;
    if (n_global >= INT32_MAX) return BS_ERANGE;
    if (n_global == 0) return BS_OK;
    if (misaligned(off, 4) || misaligned(ids, 4) || misaligned(v_local, 8) || misaligned(v_global, 8))
        return BS_EALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (block_starts) {
        if (n_blocks < 1 || n_blocks > n_global || misaligned(block_starts, 4)) return BS_EINVAL;
        hipLaunchKernelGGL(k_gather_lds, dim3((unsigned)n_blocks), dim3(kBlock), 0, st, block_starts, off, ids,
                           v_local, v_global);
    } else {
        const int64_t nb = (n_global + kBlock - 1) / kBlock;
        hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)nb), dim3(kBlock), 0, st, n_global, off, ids, v_local,
                           v_global);
    }
    return launch_status();
}

}  // extern "C"
