// bs_kernels.hip -- gfx950 kernels and C ABI of the Benchmark Streaming ops.
//
// The seven streaming operations of "Portable high-order finite element
// kernels I: Streaming Operations" (arXiv 2009.10917): BS1 copy, BS2 AXPY,
// BS3 norm, BS4 inner product, BS5 fused CG update, BS6 gather and BS7
// scatter. All are bound by HBM bandwidth (at most 0.25 flop per byte), so the
// kernels are written for bytes in flight, not for arithmetic:
//  - 128-bit (two-double) non-temporal loads and stores for every contiguous
//    stream, all loads of a lane issued before any is consumed, coalesced
//    across the 64-lane wavefront;
//  - grid-stride loops over a grid sized from the compute-unit count, with
//    the unroll depth and blocks per CU chosen per operation by measurement;
//  - reductions: per-lane accumulation, a wavefront sum by DPP lane moves,
//    the block's wavefronts through LDS, one partial per
//    block; the last block to arrive (an atomic ticket) sums the partials in
//    a fixed order in the same kernel. No atomics touch the values, so
//    results repeat bit for bit;
//  - fused CG update: two passes in one launch, x += alpha p over the whole
//    vector and then r -= alpha q with r.r, three open streams at a time (a
//    CG iteration too large for the last-level cache uses one pass over all
//    four arrays instead);
//  - scatter: each lane owns pairs of consecutive local entries, loads their
//    two indices as one 8-byte word and stores the two values as one 16-byte
//    word, 32 pairs per lane in flight;
//  - gather: the balanced blockStarts scheme of the paper, each block staging
//    at most 1024 CSR entries of v_L in LDS with coalesced index loads, then
//    one lane per global node summing its entries from LDS in ascending order,
//    plan blocks handed to the XCDs in runs of eight; without a plan, the
//    same staging over fixed spans of 512 rows (up to 2048 entries).
// Built from the same kernels: the pointwise scale y = x / d of the lumped
// mass, and a device-resident CG iteration on Z^T Z whose scalars (alpha,
// beta, |r|^2, a done flag) stay in device memory between launches. When the
// iteration's vectors and tables fit in the 256 MB last-level cache, it runs
// twins of its kernels that use the ordinary cache policy instead of
// non-temporal accesses, so each kernel finds the previous one's data there;
// above that, while r and p alone fit, the update passes them on to the
// direction update through the cache.
// No MFMA: nothing here is a dense contraction.
//
// Bit-exactness: the file is compiled with -ffp-contract=off and the pragma
// below, so a*x + b*y is two rounded products and one rounded sum, as in the
// IEEE definition. Reductions use explicit fma for the per-lane sums (they
// are checked against a relative tolerance, not bits).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <new>

#include "bs.h"

#pragma clang fp contract(off)

namespace {

constexpr int kBlock = 256;            // threads per block: 4 wavefronts
constexpr int kWave = 64;              // gfx950 wavefront width
constexpr int kFinishBlock = 1024;     // threads of the one-block reduction finish
constexpr int kMaxPartials = 1 << 20;  // reduction scratch (blocks of one first-stage launch)

// Device-resident CG scalars, one small array per context.
enum CgSlot { kRR = 0, kAlpha = 1, kBeta = 2, kDone = 3, kThreshold = 4, kCgSlots = 8 };

// A coefficient given by value or read from device memory (set by an earlier
// kernel on the same stream, so no host synchronisation is needed).
struct Coef {
    double v;
    const double *p;
    __device__ __forceinline__ double get() const { return p ? *p : v; }
};

// Kernels of a device-resident CG iteration return at once after convergence.
__device__ __forceinline__ bool skipped(const double *cgs) { return cgs && cgs[kDone] != 0.0; }

// Launch shape of a vector kernel: 16-byte loads per lane per array per loop
// iteration, blocks per compute unit (0: one tile per block, no loop) and
// threads per block.
struct VecShape {
    int unroll;
    int blocks_per_cu;
    int threads = kBlock;
};
// Chosen by sweeps of unroll {1,2,4,8,16} x blocks/CU {flat,1,2,4,8,16} x block
// size {256,512,1024} x non-temporal on/off x occupancy hint on cold data
// (vectors of 11.4M and 67M doubles, buffers rotated through > 2 GB so no
// operand is cache-resident). Fewer blocks keep the lockstep window of all
// streams narrow, which the multi-stream kernels prefer. The copy's flat
// tiles of 768 threads (12 KB per array) beat every other tile of 256-1024
// threads up to 2^25 pairs (28.6 against 30.3 us at 11.4M doubles, 114.1
// against 117.0 us at 47M) and tie at 2^25 pairs; beyond that 256-thread
// tiles are faster (by 0.8% at 2^27 doubles, 2.1% at 2^28).
constexpr VecShape kCopyShape{1, 0, 768};
constexpr VecShape kCopyLargeShape{1, 0, 256};
constexpr int64_t kCopyLargePairs = 1LL << 25;  // pairs above which kCopyLargeShape runs
constexpr VecShape kAxpyShape{1, 2};
constexpr VecShape kDotShape{2, 1, 512};
constexpr VecShape kNormShape{4, 2};
constexpr VecShape kCgShape{1, 1, 512};  // two passes: unroll of the x pass (the r pass: kCgRUnroll)
constexpr int kCgRUnroll = 2;
constexpr VecShape kCgOnePassShape{4, 1};

constexpr int kScatterPairs = 32;  // index pairs per lane in the scatter kernel
// Capacity of MI355X's last-level cache (the memory-side Infinity Cache,
// 256 MB): a CG iteration whose working set fits uses the cache-keeping
// kernels.
constexpr int64_t kCacheResidentBytes = 256LL << 20;
constexpr int64_t kHandoffBytes = 210LL << 20;  // r and p of a CG iteration passed on in the cache
constexpr int kGatherCap = 1024;   // CSR entries and rows a gather block stages in LDS
constexpr int kSpanRows = 512;     // rows per block of the gather without a plan
constexpr int kSpanCap = 2048;     // CSR entries such a block stages in LDS
constexpr int kSpanRun = 8;        // consecutive spans each XCD takes in turn

typedef double d2 __attribute__((ext_vector_type(2)));
typedef int i2 __attribute__((ext_vector_type(2)));

// Cache policy of a kernel's array streams.
//  kStream: non-temporal loads and stores. They neither allocate nor evict
//    lines of the 256 MB last-level cache, which suits data touched once: the
//    arrays of every standalone operation here.
//  kKeep: the ordinary policy. It allocates the lines, so the next kernel
//    finds whatever fits in that cache: the CG iteration's vectors and tables
//    when its whole working set fits (bs_cg_solve chooses).
enum Policy { kStream = 0, kKeep = 1 };

template <int P, typename T>
__device__ __forceinline__ T ldp(const T *p)
{
    if constexpr (P == kStream)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <int P, typename T>
__device__ __forceinline__ void stp(T *p, T v)
{
    if constexpr (P == kStream)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

__device__ __forceinline__ d2 ld2(const d2 *p) { return ldp<kStream>(p); }
__device__ __forceinline__ void st2(d2 *p, d2 v) { stp<kStream>(p, v); }

// ------------------------------------------------------------ reductions --

// A double moved across lanes by one DPP control (0 where the control
// leaves a lane without a source or the row mask leaves it unwritten).
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ double dpp_move(double v)
{
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), kCtrl, kRowMask, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), kCtrl, kRowMask, 0xf, false);
    return __hiloint2double(hi, lo);
}

// Sum over the 64 lanes of a wavefront by DPP (no LDS): pairs, quads, 8 and
// 16 lanes within each row of 16, then the rows by broadcasts of lanes 15 and
// 31; lane 63 ends with the total, which every lane then reads. The order of
// the additions is fixed, so the bits repeat.
__device__ __forceinline__ double wave_sum(double v)
{
    v += dpp_move<0xb1>(v);        // quad_perm [1,0,3,2]
    v += dpp_move<0x4e>(v);        // quad_perm [2,3,0,1]
    v += dpp_move<0x124>(v);       // row_ror:4
    v += dpp_move<0x128>(v);       // row_ror:8
    v += dpp_move<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_move<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    const int lo = __builtin_amdgcn_readlane(__double2loint(v), 63);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(v), 63);
    return __hiloint2double(hi, lo);
}

// Sum over the block; the result is valid in thread 0.
template <int NT = kBlock>
__device__ __forceinline__ double block_sum(double v)
{
    __shared__ double wsum[NT / kWave];
    v = wave_sum(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) wsum[w] = v;
    __syncthreads();
    double s = 0.0;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 0; i < NT / kWave; ++i) s += wsum[i];
    }
    return s;
}

// Finishes of the device-resident CG iteration (unpreconditioned CG, the
// vector operations of the BS paper's CG list):
//  kStart: rr = r.r; history[0] = rr; convergence threshold tol2 * rr; the
//          history entries after 0 are set to -1 (an iteration that runs
//          overwrites its entry).
//  kSetAlpha: alpha = rr / (p.q).
//  kSetBeta:  rr' = r'.r'; beta = rr' / rr; rr = rr'; history[k+1] = rr';
//          converged when rr' <= threshold (or rr' == 0).
// cg_apply stores the scalars from the reduced sum s (one thread);
// cg_hist_init clears the history (any threads of one block).
enum CgFinish { kStart = 0, kSetAlpha = 1, kSetBeta = 2 };

__device__ __forceinline__ void cg_hist_init(double *hist, int iters, int nthreads)
{
    for (int i = 1 + (int)threadIdx.x; i <= iters; i += nthreads) hist[i] = -1.0;
}

__device__ __forceinline__ void cg_apply(int mode, double s, double *cgs, double *hist, int k, double tol2)
{
    if (mode == kStart) {
        cgs[kRR] = s;
        cgs[kThreshold] = tol2 * s;
        cgs[kDone] = (s == 0.0) ? 1.0 : 0.0;
        hist[0] = s;
    } else if (mode == kSetAlpha) {
        cgs[kAlpha] = cgs[kRR] / s;
    } else {
        cgs[kBeta] = s / cgs[kRR];
        cgs[kRR] = s;
        hist[k + 1] = s;
        if (s == 0.0 || s <= cgs[kThreshold]) cgs[kDone] = 1.0;
    }
}

// One-kernel finish of the vector reductions (norm, dot, fused update), with
// no second launch. Each block publishes its partial with an agent-scope
// atomic store, which on this multi-XCD part writes through to the memory
// side instead of staying in the block's XCD-local L2; waits until that store
// has completed (s_waitcnt vmcnt(0)); then takes a ticket with an agent-scope
// atomic add. The block that draws the last ticket reads every partial back
// with agent-scope atomic loads, which fetch from the memory side and so
// never see a line left in its own L2 by an earlier call, and sums them in
// index order. Partials and tickets are touched only by agent-scope atomics,
// so every value crosses the XCDs coherently; the wait alone orders the
// partial before the ticket, as the memory model's own release sequence does
// for an earlier atomic store. (A release RMW would add an L2 write-back of
// all ordinary stores of the XCD, about 10 us per call at 256-512 blocks.)
// Grids of up to kOneTicket blocks draw from one counter; larger ones count
// first per group of blocks with the same blockIdx mod 8 (the block's XCD),
// each group's counter on its own 256-byte line, so that arrivals do not
// queue on one address (at 512 blocks one counter costs 3 us, grouping 0).
// The last arrival at each counter resets it to zero for the next call. The
// tickets only choose which block finishes: the sum is in a fixed order, so
// results repeat bit for bit.
constexpr unsigned kOneTicket = 256;
constexpr int kTicketStride = 64;                // unsigned ints: 256 bytes
constexpr int kTickets = 9 * kTicketStride;      // [0] the grid, [(1 + g) * stride] group g

enum FinMode { kFinOut = 0, kFinSqrt = 1, kFinCg = 2 };
struct Fin {
    int mode;           // kFinOut: *out = s; kFinSqrt: *out = sqrt(s); kFinCg: cg_apply(cg, s)
    int cg;             // CgFinish
    double *partials;   // one slot per block
    unsigned *tickets;  // kTickets counters, zero between calls
    double *out;
    double *cgs;
    double *hist;
    int k, iters;
    double tol2;
};

// Called by every thread of every block with the block's partial (valid in
// thread 0) and the grid's block count nb; true in the block that is to
// finish.
__device__ __forceinline__ bool last_arrival(double part, const Fin &f, unsigned nb)
{
    __shared__ bool last;
    if (threadIdx.x == 0) {
        __hip_atomic_store(&f.partials[blockIdx.x], part, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // The two single-thread fences emit no instruction. They stop the
        // compiler from moving the store below the wait or the ticket's
        // atomic add above it (relaxed atomics to different addresses could
        // otherwise be reordered), so the program order store -> wait ->
        // ticket that the hardware relies on is also the order in the code.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        bool l;
        if (nb <= kOneTicket) {
            l = __hip_atomic_fetch_add(&f.tickets[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nb - 1;
        } else {
            const unsigned g = blockIdx.x & 7u;
            const unsigned members = nb / 8u + (g < (nb & 7u) ? 1u : 0u);
            unsigned *gc = &f.tickets[(1 + g) * kTicketStride];
            l = false;
            if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == members - 1) {
                __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                l = __hip_atomic_fetch_add(&f.tickets[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 7u;
            }
        }
        if (l) __hip_atomic_store(&f.tickets[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = l;
    }
    __syncthreads();
    return last;
}

// In the finishing block (all kBlock threads): the partials summed in a fixed
// order (each lane a strided run, the wave's DPP sum, the waves in order),
// then stored as the mode says. A lane issues its loads kFinishLoads at a
// time before adding them, so a grid of up to kFinishLoads * kBlock blocks
// costs one round trip to memory, not one per kBlock partials; the lane adds
// its partials in the same order either way (a +0.0 past the end changes no
// bits: the running sum starts at +0.0 and never becomes -0.0).
constexpr int kFinishLoads = 4;
template <int NT = kBlock>
__device__ __forceinline__ void finish_last(const Fin &f, unsigned nb)
{
    __shared__ double wsum[NT / kWave];
    double s = 0.0;
    for (unsigned i0 = threadIdx.x; i0 < nb; i0 += kFinishLoads * NT) {
        double v[kFinishLoads];
#pragma unroll
        for (int k = 0; k < kFinishLoads; ++k) {
            const unsigned i = i0 + k * NT;
            v[k] = i < nb ? __hip_atomic_load(&f.partials[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.0;
        }
#pragma unroll
        for (int k = 0; k < kFinishLoads; ++k) s += v[k];
    }
    s = wave_sum(s);
    if ((threadIdx.x & (kWave - 1)) == 0) wsum[threadIdx.x / kWave] = s;
    if (f.mode == kFinCg && f.cg == kStart) cg_hist_init(f.hist, f.iters, NT);
    __syncthreads();
    if (threadIdx.x != 0) return;
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) t += wsum[i];
    if (f.mode == kFinOut)
        *f.out = t;
    else if (f.mode == kFinSqrt)
        *f.out = std::sqrt(t);
    else
        cg_apply(f.cg, t, f.cgs, f.hist, f.k, f.tol2);
}

template <int NT = kBlock>
__device__ __forceinline__ void finish_block(double part, const Fin &f, unsigned nb)
{
    if (last_arrival(part, f, nb)) finish_last<NT>(f, nb);
}

// Two-kernel reductions (the gather's folded dot, whose grid has one block
// per plan block, and the 8-byte fallbacks): one block sums the nb per-block
// partials in a fixed order and writes the result; nb == 0 stores +0.0. The
// kernel boundary makes the partials visible across XCDs.
//
// finish_sum: the sum over one kFinishBlock-thread block, valid in thread 0:
// each lane a strided run in index order, then the wave's DPP sum, then the
// 16 wave sums in order. A lane issues its loads kFinishBatch at a time, all
// before the adds: the gather's folded dot leaves one partial per plan block
// (55297 at 24^3 order 15), and one load in flight per lane made this sum
// latency-bound (23 us).
constexpr int kFinishBatch = 32;
__device__ __forceinline__ double finish_sum(const double *__restrict__ partials, int nb)
{
    __shared__ double wsum[kFinishBlock / kWave];
    double s = 0.0;
    for (int i0 = threadIdx.x; i0 < nb; i0 += kFinishBatch * kFinishBlock) {
        double v[kFinishBatch];
#pragma unroll
        for (int k = 0; k < kFinishBatch; ++k) {
            const int i = i0 + k * kFinishBlock;
            v[k] = i < nb ? partials[i] : 0.0;
        }
#pragma unroll
        for (int k = 0; k < kFinishBatch; ++k) s += v[k];
    }
    s = wave_sum(s);
    if ((threadIdx.x & (kWave - 1)) == 0) wsum[threadIdx.x / kWave] = s;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 0; i < kFinishBlock / kWave; ++i) t += wsum[i];
    }
    return t;
}

__global__ __launch_bounds__(kFinishBlock) void k_finish(const double *__restrict__ partials, int nb,
                                                         double *__restrict__ out, bool take_sqrt)
{
    const double s = finish_sum(partials, nb);
    if (threadIdx.x == 0) *out = take_sqrt ? std::sqrt(s) : s;
}

// Second stage of the CG iteration's alpha (after the gather's folded p.q).
__global__ __launch_bounds__(kFinishBlock) void k_cg_finish(const double *__restrict__ partials, int nb,
                                                            double *__restrict__ cgs, double *__restrict__ hist,
                                                            int k, int iters, double tol2, int mode)
{
    if (mode == kStart)
        cg_hist_init(hist, iters, kFinishBlock);
    else if (cgs[kDone] != 0.0)
        return;
    const double s = finish_sum(partials, nb);
    if (threadIdx.x == 0) cg_apply(mode, s, cgs, hist, k, tol2);
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

// The body and flags of a Split as plain kernel arguments: bit 0 a head
// element, bit 1 a tail element (which follows the body).
__host__ __device__ inline unsigned ht_of(const Split &s) { return (s.head ? 1u : 0u) | (s.tail >= 0 ? 2u : 0u); }
__device__ inline Split split_ht(int64_t n2, unsigned ht)
{
    const int64_t head = ht & 1u;
    return Split{head, n2, (ht & 2u) ? head + 2 * n2 : -1};
}

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
// The standalone kernels take their arguments as plain scalars and pointers,
// the ones needed first leading: the library is built to preload the leading
// kernel arguments into SGPRs at wave launch (kernarg preload), which spares
// every wave the scalar load of its arguments before its first memory access
// (0.4 us of a 29 us copy). Aggregates cannot be preloaded, nor can the hidden
// grid size behind them: the kernels that end in a reduction finish (an
// aggregate) or have more leading arguments than the preload holds take the
// head/tail flags packed in one word and the grid size as an argument (the
// fused update 0.6 us faster, AXPY and dot 0.15 us).
template <int U, int NT>
__global__ __launch_bounds__(NT) void k_copy(int64_t n2, const double *__restrict__ x, double *__restrict__ y,
                                             int64_t head, int64_t tail)
{
    const Split sp{head, n2, tail};
    const d2 *xv = reinterpret_cast<const d2 *>(x + sp.head);
    d2 *yv = reinterpret_cast<d2 *>(y + sp.head);
    const int64_t stride = (int64_t)gridDim.x * NT * U;
    int64_t i = (int64_t)blockIdx.x * NT * U + threadIdx.x;
    for (; i + (U - 1) * NT < sp.n2; i += stride) {
        d2 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = ld2(xv + i + u * NT);
#pragma unroll
        for (int u = 0; u < U; ++u) st2(yv + i + u * NT, v[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (i + u * NT < sp.n2) st2(yv + i + u * NT, ld2(xv + i + u * NT));
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

// The coefficients come by value (bs_axpy) or from device memory (the
// p = r + beta p step of the device-resident CG iteration).
template <int U, int P>
__device__ __forceinline__ void axpy_body(Split sp, Coef ca, const double *x, Coef cb, double *y,
                                          const double *cgs, unsigned nblk)
{
    if (skipped(cgs)) return;
    const double a = ca.get(), b = cb.get();
    const d2 *xv = reinterpret_cast<const d2 *>(x + sp.head);
    d2 *yv = reinterpret_cast<d2 *>(y + sp.head);
    const int64_t stride = (int64_t)nblk * kBlock * U;
    int64_t i = (int64_t)blockIdx.x * kBlock * U + threadIdx.x;
    for (; i + (U - 1) * kBlock < sp.n2; i += stride) {
        d2 vx[U], vy[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            vx[u] = ldp<P>(xv + i + u * kBlock);
            vy[u] = ldp<P>(yv + i + u * kBlock);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) stp<P>(yv + i + u * kBlock, axpy2(a, vx[u], b, vy[u]));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t k = i + u * kBlock;
        if (k < sp.n2) stp<P>(yv + k, axpy2(a, ldp<P>(xv + k), b, ldp<P>(yv + k)));
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (sp.head) y[0] = a * x[0] + b * y[0];
        if (sp.tail >= 0) y[sp.tail] = a * x[sp.tail] + b * y[sp.tail];
    }
}

template <int U>
__global__ __launch_bounds__(kBlock) void k_axpy(int64_t n2, const double *x, double *y, double a, double b,
                                                 unsigned ht, unsigned nblk)
{
    axpy_body<U, kStream>(split_ht(n2, ht), Coef{a, nullptr}, x, Coef{b, nullptr}, y, nullptr, nblk);
}

// The direction update p = (1 r) + (beta p) of the CG iteration, beta read
// from device memory (streaming policy). Like the standalone kernels, the
// CG iteration's kernels take plain arguments that the preload holds (1-3%
// per iteration at 12^3-32^3 order 7 against aggregate arguments).
template <int U>
__global__ __launch_bounds__(kBlock) void k_axpy_dev(int64_t n2, const double *x, double *y, const double *cgs,
                                                     unsigned ht, unsigned nblk)
{
    axpy_body<U, kStream>(split_ht(n2, ht), Coef{1.0, nullptr}, x, Coef{0.0, cgs + kBeta}, y, cgs, nblk);
}

// The same with the cache-keeping policy.
template <int U>
__global__ __launch_bounds__(kBlock) void k_axpy_keep(int64_t n2, const double *x, double *y, const double *cgs,
                                                      unsigned ht, unsigned nblk)
{
    axpy_body<U, kKeep>(split_ht(n2, ht), Coef{1.0, nullptr}, x, Coef{0.0, cgs + kBeta}, y, cgs, nblk);
}

// ------------------------------------------- pointwise scale y = x / d ----
// The 1/m scaling by the lumped mass ("GPU accelerated spectral finite
// elements on all-hex meshes", coarse-grid correction). Each quotient is one
// correctly rounded IEEE division. y may be x (in place).
template <int U>
__global__ __launch_bounds__(kBlock) void k_scale(int64_t n2, const double *x, const double *d, double *y,
                                                  int64_t head, int64_t tail)
{
    const Split sp{head, n2, tail};
    const d2 *xv = reinterpret_cast<const d2 *>(x + sp.head);
    const d2 *dv = reinterpret_cast<const d2 *>(d + sp.head);
    d2 *yv = reinterpret_cast<d2 *>(y + sp.head);
    const int64_t stride = (int64_t)gridDim.x * kBlock * U;
    int64_t i = (int64_t)blockIdx.x * kBlock * U + threadIdx.x;
    for (; i + (U - 1) * kBlock < sp.n2; i += stride) {
        d2 vx[U], vd[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            vx[u] = ld2(xv + i + u * kBlock);
            vd[u] = ld2(dv + i + u * kBlock);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) st2(yv + i + u * kBlock, vx[u] / vd[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t k = i + u * kBlock;
        if (k < sp.n2) st2(yv + k, ld2(xv + k) / ld2(dv + k));
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (sp.head) y[0] = x[0] / d[0];
        if (sp.tail >= 0) y[sp.tail] = x[sp.tail] / d[sp.tail];
    }
}

__global__ __launch_bounds__(kBlock) void k_scale_scalar(int64_t n, const double *x, const double *d, double *y)
{
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock)
        y[i] = x[i] / d[i];
}

// ------------------------------------------------- BS3 norm, BS4 dot ----
// First stage of both: with kSquare it sums x[i]^2 (y is ignored). The grid
// holds two 256-thread blocks (norm) or one 512-thread block (dot) per CU,
// so the kernel never needs more than two waves per SIMD: the occupancy hint
// lets the compiler keep every load of a lane in flight instead of trading
// registers for waves it will not get. The dot's single block per CU carries
// the same bytes in flight as two smaller ones with half the partials, and
// measured 0.4 us faster at 11.4M doubles; the norm measured no gain from it.
template <int U, bool kSquare, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_dot(
    int64_t n2, const double *__restrict__ x, const double *__restrict__ y, unsigned ht, unsigned nblk, Fin f)
{
    const Split sp = split_ht(n2, ht);
    const d2 *xv = reinterpret_cast<const d2 *>(x + sp.head);
    const d2 *yv = reinterpret_cast<const d2 *>((kSquare ? x : y) + sp.head);
    const int64_t stride = (int64_t)nblk * NT * U;
    int64_t i = (int64_t)blockIdx.x * NT * U + threadIdx.x;
    double acc0 = 0.0, acc1 = 0.0;
    for (; i + (U - 1) * NT < sp.n2; i += stride) {
        d2 vx[U], vy[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            vx[u] = ld2(xv + i + u * NT);
            vy[u] = kSquare ? vx[u] : ld2(yv + i + u * NT);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            acc0 = __builtin_fma(vx[u].x, vy[u].x, acc0);
            acc1 = __builtin_fma(vx[u].y, vy[u].y, acc1);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t k = i + u * NT;
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
    finish_block<NT>(block_sum<NT>(acc0 + acc1), f, nblk);
}

// -------------------------------------------------- BS5 fused CG update ----
// x + (a p) and r - (a q), each product rounded first (contraction is off).
__device__ __forceinline__ d2 plus_ap(d2 x, double a, d2 p)
{
    d2 o;
    o.x = x.x + a * p.x;
    o.y = x.y + a * p.y;
    return o;
}

__device__ __forceinline__ d2 minus_aq(d2 r, double a, d2 q)
{
    d2 o;
    o.x = r.x - a * q.x;
    o.y = r.y - a * q.y;
    return o;
}

// Scalar head and tail elements of the update (one thread), and the block's
// share of r.r to the reduction.
template <int NT = kBlock>
__device__ __forceinline__ void cg_update_finish(Split sp, double a, const double *p, const double *q, double *x,
                                                 double *r, double acc0, double acc1, const Fin &f,
                                                 unsigned nblk)
{
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
    finish_block<NT>(block_sum<NT>(acc0 + acc1), f, nblk);
}

// Two forms of the update, the same bits either way. p, q, x and r are
// distinct arrays (the ABI requires it), so the pointers are
// restrict-qualified: without that the compiler may not move a store of x or
// r past a later load and serialises the lane's loads, which at one block per
// CU costs about a third of the bandwidth.
//
// Two passes in one launch: first x += alpha p over the whole vector, then
// r -= alpha q with the sum of the new r^2. Neither half reads what the other
// writes, so no grid-wide wait sits between them, and each pass keeps three
// streams open (two reads, one write) instead of six, which this memory system
// serves faster when all four arrays come from HBM: 86.4 against 88.7 us at
// 11.4M doubles, the same bytes. The x pass loads U1 pairs per array per lane
// and loop, the r pass U2. One 512-thread block per CU (two waves per SIMD)
// at unroll 1 and 2 took it to 85.4 us; 256 threads at unroll 2 and 4 keep
// the same bytes in flight with half the waves.
template <int U1, int U2, int NT, int P>
__device__ __forceinline__ void cg_update_two_pass(Split sp, Coef ca, const double *__restrict__ p,
                                                   const double *__restrict__ q, double *__restrict__ x,
                                                   double *__restrict__ r, const Fin &f, const double *cgs,
                                                   unsigned nblk)
{
    if (skipped(cgs)) return;
    const double a = ca.get();
    const d2 *pv = reinterpret_cast<const d2 *>(p + sp.head);
    const d2 *qv = reinterpret_cast<const d2 *>(q + sp.head);
    d2 *xv = reinterpret_cast<d2 *>(x + sp.head);
    d2 *rv = reinterpret_cast<d2 *>(r + sp.head);
    {
        const int64_t stride = (int64_t)nblk * NT * U1;
        int64_t i = (int64_t)blockIdx.x * NT * U1 + threadIdx.x;
        for (; i + (U1 - 1) * NT < sp.n2; i += stride) {
            d2 vp[U1], vx[U1];
#pragma unroll
            for (int u = 0; u < U1; ++u) {
                vp[u] = ldp<P>(pv + i + u * NT);
                vx[u] = ldp<P>(xv + i + u * NT);
            }
#pragma unroll
            for (int u = 0; u < U1; ++u) stp<P>(xv + i + u * NT, plus_ap(vx[u], a, vp[u]));
        }
#pragma unroll
        for (int u = 0; u < U1; ++u) {
            const int64_t k = i + u * NT;
            if (k < sp.n2) stp<P>(xv + k, plus_ap(ldp<P>(xv + k), a, ldp<P>(pv + k)));
        }
    }
    double acc0 = 0.0, acc1 = 0.0;
    {
        const int64_t stride = (int64_t)nblk * NT * U2;
        int64_t i = (int64_t)blockIdx.x * NT * U2 + threadIdx.x;
        for (; i + (U2 - 1) * NT < sp.n2; i += stride) {
            d2 vq[U2], vr[U2];
#pragma unroll
            for (int u = 0; u < U2; ++u) {
                vq[u] = ldp<P>(qv + i + u * NT);
                vr[u] = ldp<P>(rv + i + u * NT);
            }
#pragma unroll
            for (int u = 0; u < U2; ++u) {
                const d2 nr = minus_aq(vr[u], a, vq[u]);
                stp<P>(rv + i + u * NT, nr);
                acc0 = __builtin_fma(nr.x, nr.x, acc0);
                acc1 = __builtin_fma(nr.y, nr.y, acc1);
            }
        }
#pragma unroll
        for (int u = 0; u < U2; ++u) {
            const int64_t k = i + u * NT;
            if (k < sp.n2) {
                const d2 nr = minus_aq(ldp<P>(rv + k), a, ldp<P>(qv + k));
                stp<P>(rv + k, nr);
                acc0 = __builtin_fma(nr.x, nr.x, acc0);
                acc1 = __builtin_fma(nr.y, nr.y, acc1);
            }
        }
    }
    cg_update_finish<NT>(sp, a, p, q, x, r, acc0, acc1, f, nblk);
}

// One pass over all four arrays, U pairs of each per lane and loop; PP is the
// policy of the loads of p, PR of the stores of r, P of the other streams.
// Inside a CG iteration p arrives partly in the last-level cache (the scatter
// has just read it with the ordinary policy), and one pass overlaps those hits
// with the HBM streams of q, x and r: 80.9 against 85.9 us for the two passes
// at 11.4M doubles, 353.7 against 361.2 us at 47M.
template <int U, int P, int PP = P, int PR = P>
__device__ __forceinline__ void cg_update_one_pass(Split sp, Coef ca, const double *__restrict__ p,
                                                   const double *__restrict__ q, double *__restrict__ x,
                                                   double *__restrict__ r, const Fin &f, const double *cgs,
                                                   unsigned nblk)
{
    if (skipped(cgs)) return;
    const double a = ca.get();
    const d2 *pv = reinterpret_cast<const d2 *>(p + sp.head);
    const d2 *qv = reinterpret_cast<const d2 *>(q + sp.head);
    d2 *xv = reinterpret_cast<d2 *>(x + sp.head);
    d2 *rv = reinterpret_cast<d2 *>(r + sp.head);
    const int64_t stride = (int64_t)nblk * kBlock * U;
    int64_t i = (int64_t)blockIdx.x * kBlock * U + threadIdx.x;
    double acc0 = 0.0, acc1 = 0.0;
    for (; i + (U - 1) * kBlock < sp.n2; i += stride) {
        d2 vp[U], vq[U], vx[U], vr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            vp[u] = ldp<PP>(pv + i + u * kBlock);
            vq[u] = ldp<P>(qv + i + u * kBlock);
            vx[u] = ldp<P>(xv + i + u * kBlock);
            vr[u] = ldp<P>(rv + i + u * kBlock);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const d2 nr = minus_aq(vr[u], a, vq[u]);
            stp<P>(xv + i + u * kBlock, plus_ap(vx[u], a, vp[u]));
            stp<PR>(rv + i + u * kBlock, nr);
            acc0 = __builtin_fma(nr.x, nr.x, acc0);
            acc1 = __builtin_fma(nr.y, nr.y, acc1);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t k = i + u * kBlock;
        if (k < sp.n2) {
            const d2 nr = minus_aq(ldp<P>(rv + k), a, ldp<P>(qv + k));
            stp<P>(xv + k, plus_ap(ldp<P>(xv + k), a, ldp<PP>(pv + k)));
            stp<PR>(rv + k, nr);
            acc0 = __builtin_fma(nr.x, nr.x, acc0);
            acc1 = __builtin_fma(nr.y, nr.y, acc1);
        }
    }
    cg_update_finish(sp, a, p, q, x, r, acc0, acc1, f, nblk);
}

template <int U1, int U2, int NT>
__global__ __launch_bounds__(NT) void k_cg_update(int64_t n2, const double *__restrict__ p,
                                                  const double *__restrict__ q, double *__restrict__ x,
                                                  double *__restrict__ r, double alpha, unsigned ht, unsigned nblk,
                                                  Fin f)
{
    cg_update_two_pass<U1, U2, NT, kStream>(split_ht(n2, ht), Coef{alpha, nullptr}, p, q, x, r, f, nullptr, nblk);
}

// The same with the cache-keeping policy, for the CG iteration.
template <int U1, int U2, int NT>
__global__ __launch_bounds__(NT) void k_cg_update_keep(int64_t n2, const double *__restrict__ p,
                                                       const double *__restrict__ q, double *__restrict__ x,
                                                       double *__restrict__ r, const double *cgs, unsigned ht,
                                                       unsigned nblk, Fin f)
{
    cg_update_two_pass<U1, U2, NT, kKeep>(split_ht(n2, ht), Coef{0.0, cgs + kAlpha}, p, q, x, r, f, cgs, nblk);
}

// One pass, non-temporal: the CG iteration's update when its vectors do not
// fit in the last-level cache.
template <int U>
__global__ __launch_bounds__(kBlock) void k_cg_update_one_pass(int64_t n2, const double *__restrict__ p,
                                                               const double *__restrict__ q,
                                                               double *__restrict__ x, double *__restrict__ r,
                                                               const double *cgs, unsigned ht, unsigned nblk, Fin f)
{
    cg_update_one_pass<U, kStream>(split_ht(n2, ht), Coef{0.0, cgs + kAlpha}, p, q, x, r, f, cgs, nblk);
}

// The same, for a CG iteration whose vectors do not fit in the last-level
// cache but whose r and p do: p is read and r stored with the ordinary
// policy, so the direction update p = r + beta p that follows finds both
// there.
template <int U>
__global__ __launch_bounds__(kBlock) void k_cg_update_handoff(int64_t n2, const double *__restrict__ p,
                                                               const double *__restrict__ q,
                                                               double *__restrict__ x, double *__restrict__ r,
                                                               const double *cgs, unsigned ht, unsigned nblk, Fin f)
{
    cg_update_one_pass<U, kStream, kKeep, kKeep>(split_ht(n2, ht), Coef{0.0, cgs + kAlpha}, p, q, x, r, f, cgs, nblk);
}

// --------------------------------------------------------- BS7 scatter ----
// Lane t of block b owns the index pairs b*P + t + kBlock*u (u < kScatterPairs,
// P = kBlock*kScatterPairs pairs per block), i.e. local entries 2*pair and
// 2*pair+1: one 8-byte index load, two reads of v_G, one 16-byte store each.
// All index loads of the lane are issued before the reads they feed, and all
// reads before the stores. Full tiles take a path with no bounds tests (they
// would cost the compiler its freedom to keep every load in flight); in the
// last, partial tile a pair past the end is skipped and a pair cut by the end
// goes as one 4-byte load and one 8-byte store.
template <bool kFull, int P>
__device__ __forceinline__ void scatter_tile(int64_t base, int64_t nl, const int32_t *__restrict__ l2g,
                                             const double *__restrict__ vg, double *__restrict__ vl)
{
    i2 id[kScatterPairs];
#pragma unroll
    for (int u = 0; u < kScatterPairs; ++u) {
        const int64_t e = base + 2 * ((int64_t)u * kBlock + threadIdx.x);
        if (kFull || e + 1 < nl) {
            id[u] = ldp<P>(reinterpret_cast<const i2 *>(l2g + e));
        } else {
            id[u].x = e < nl ? l2g[e] : -1;
            id[u].y = -1;
        }
    }
    d2 v[kScatterPairs];
#pragma unroll
    for (int u = 0; u < kScatterPairs; ++u) {
        v[u].x = id[u].x >= 0 ? vg[id[u].x] : 0.0;
        v[u].y = id[u].y >= 0 ? vg[id[u].y] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < kScatterPairs; ++u) {
        const int64_t e = base + 2 * ((int64_t)u * kBlock + threadIdx.x);
        if (kFull || e + 1 < nl)
            stp<P>(reinterpret_cast<d2 *>(vl + e), v[u]);
        else if (e < nl)
            vl[e] = v[u].x;
    }
}

template <int P>
__device__ __forceinline__ void scatter_body(int64_t nl, const int32_t *__restrict__ l2g,
                                             const double *__restrict__ vg, double *__restrict__ vl,
                                             const double *cgs)
{
    if (skipped(cgs)) return;
    constexpr int64_t kTile = 2LL * kBlock * kScatterPairs;  // entries per block
    const int64_t base = (int64_t)blockIdx.x * kTile;
    if (base + kTile <= nl)
        scatter_tile<true, P>(base, nl, l2g, vg, vl);
    else
        scatter_tile<false, P>(base, nl, l2g, vg, vl);
}

__global__ __launch_bounds__(kBlock) void k_scatter(int64_t nl, const int32_t *__restrict__ l2g,
                                                    const double *__restrict__ vg,
                                                    double *__restrict__ vl, const double *cgs)
{
    scatter_body<kStream>(nl, l2g, vg, vl, cgs);
}

// The same with the cache-keeping policy, for the CG iteration.
__global__ __launch_bounds__(kBlock) void k_scatter_keep(int64_t nl, const int32_t *__restrict__ l2g,
                                                         const double *__restrict__ vg,
                                                         double *__restrict__ vl, const double *cgs)
{
    scatter_body<kKeep>(nl, l2g, vg, vl, cgs);
}

// Fallback for index or value pointers without 8/16-byte alignment: 4-byte
// index loads and 8-byte stores, a block's tile of 8 * kBlock consecutive
// entries (lane t: t, t + kBlock, ...) with every index load issued before
// the v_G reads they feed and those before the stores. On the 32^3 order-7
// box: 57.3 us with l2g 4 bytes off, 58.5 us with v_L 8 bytes off, against
// 81.4 and 80.1 us with one entry per lane (16 and 32 entries per lane:
// 61.5-65.8 us; the paired kernel on aligned operands: 54.0 us).
constexpr int kScatterScalarEntries = 8;  // entries per lane of the 8-byte scatter

__global__ __launch_bounds__(kBlock) void k_scatter_scalar(int64_t nl, const int32_t *l2g,
                                                           const double *vg, double *vl)
{
    constexpr int U = kScatterScalarEntries;
    const int64_t i0 = (int64_t)blockIdx.x * U * kBlock + threadIdx.x;
    int32_t g[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = i0 + (int64_t)u * kBlock;
        g[u] = i < nl ? l2g[i] : -1;
    }
    double v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = g[u] >= 0 ? vg[g[u]] : 0.0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = i0 + (int64_t)u * kBlock;
        if (i < nl) vl[i] = v[u];
    }
}

// ---------------------------------------------------------- BS6 gather ----
// Both gather kernels optionally fold a dot product into the same pass: with
// kDot, each lane also accumulates v_G[g] * w[g] over its rows and the block
// writes one partial (the p.q of a CG iteration, q = Z^T Z p, without a
// second read of q). The gathered values are the same bits either way.

// Span kernel (no plan): the rows are cut into fixed spans of kSpanRows,
// and a block sums one span the way the plan kernel below sums a plan block.
// It reads the span's first and end CSR entry from the offsets (one round of
// scalar loads; without a plan nothing else can name them), issues its ids
// (consecutive lanes on consecutive entries) and the two offsets of each of
// its rows at once, stages the v_L values in LDS and, after the one barrier,
// sums each row from LDS in ascending order. A span over kSpanCap entries
// takes the global-memory path. On a box of order N the densest rows, the
// lines through element corners, average 4 (1 + 1/N) entries, so only spans
// lying mostly on such a line overflow: none at 32^3 order 7, whose lines are
// 225 rows long (at most about 1700 entries in a span), and about one span
// in N^2 where lines are longer than a span. Spans go to the XCDs in runs
// of kSpanRun, as plan blocks do, so that neighbouring spans, which read
// neighbouring v_L lines, share an L2. Measured against a row-per-lane
// kernel (one lane per row, its ids and values loaded row by row): 58.9
// against 79.5 us at 32^3 N=7, 207.1 against 270.9 us at 24^3 N=15, 61.8
// against 96.1 us on the tet-split mesh, the same bits; 2-5% behind a plan.
// P is the cache policy of its streams (ids, v_G): the CG iteration takes
// kKeep when its working set fits in the last-level cache (41.6 against
// 42.8 us per iteration on a 32 x 32 x 4-element slab at N=7 without a
// plan).
template <bool kDot, int P>
__global__ __launch_bounds__(kBlock) void k_gather_span(int64_t ng, const int32_t *__restrict__ off,
                                                        const int32_t *__restrict__ ids,
                                                        const double *__restrict__ vl,
                                                        double *__restrict__ vg, const double *cgs,
                                                        const double *__restrict__ w,
                                                        double *__restrict__ partials)
{
    if (skipped(cgs)) return;
    constexpr int K = kSpanCap / kBlock;    // entries per lane
    constexpr int RL = kSpanRows / kBlock;  // rows per lane
    __shared__ double stage[kSpanCap];
    // block b takes span sb: runs of kSpanRun spans per XCD over every whole
    // round of 8 * kSpanRun spans, the spans past the last round in order
    const int64_t nb = (ng + kSpanRows - 1) / kSpanRows, round = 8 * kSpanRun, full = nb / round * round;
    const int64_t b = blockIdx.x, x = b % 8, k = b / 8;
    const int64_t sb = b >= full ? b : ((k / kSpanRun) * 8 + x) * kSpanRun + k % kSpanRun;
    const int64_t r0 = sb * kSpanRows;
    const int64_t r1 = r0 + kSpanRows < ng ? r0 + kSpanRows : ng;
    const int32_t e0 = off[r0], e1 = off[r1];
    const int32_t nr = (int32_t)(r1 - r0), ne = e1 - e0;
    double acc = 0.0;
    if (ne <= kSpanCap) {
        int32_t id[K], oa[RL], ob[RL];
#pragma unroll
        for (int q = 0; q < K; ++q) {
            const int32_t t = threadIdx.x + q * kBlock;
            id[q] = t < ne ? ldp<P>(ids + e0 + t) : -1;
        }
#pragma unroll
        for (int q = 0; q < RL; ++q) {
            const int32_t r = threadIdx.x + q * kBlock;
            oa[q] = r < nr ? off[r0 + r] : 0;
            ob[q] = r < nr ? off[r0 + r + 1] : 0;
        }
        double v[K];
#pragma unroll
        for (int q = 0; q < K; ++q) v[q] = id[q] >= 0 ? vl[id[q]] : 0.0;
#pragma unroll
        for (int q = 0; q < K; ++q) {
            const int32_t t = threadIdx.x + q * kBlock;
            if (t < ne) stage[t] = v[q];
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < RL; ++q) {
            const int32_t r = threadIdx.x + q * kBlock;
            if (r < nr) {
                double sum = 0.0;
                for (int32_t j = oa[q] - e0; j < ob[q] - e0; ++j) sum = sum + stage[j];
                stp<P>(vg + r0 + r, sum);
                if (kDot) acc = __builtin_fma(sum, w[r0 + r], acc);
            }
        }
    } else {
        // offsets reach INT32_MAX at the largest tables: count in 64 bits
        for (int64_t g = r0 + threadIdx.x; g < r1; g += kBlock) {
            double sum = 0.0;
            for (int64_t j = off[g]; j < off[g + 1]; ++j) sum = sum + vl[ids[j]];
            vg[g] = sum;
            if (kDot) acc = __builtin_fma(sum, w[g], acc);
        }
    }
    if (kDot) {
        const double part = block_sum(acc);
        if (threadIdx.x == 0) partials[blockIdx.x] = part;
    }
}

// LDS-staged kernel after the blockStarts scheme of the paper: workgroup s
// takes plan block s, rows r0 .. r1) with CSR entries e0 .. e1), which
// bs_gather_plan caps at kGatherCap rows and kGatherCap entries (a single
// longer row gets a block of its own) and orders for the XCDs. The block
// reads its four plan words with uniform (scalar) loads in one round, so
// each lane can then issue at once its CSR ids (consecutive lanes on
// consecutive entries) and the two offsets of each row it will sum. The v_L
// values the ids name are fetched, staged in LDS, and after the one barrier
// each lane sums its rows from LDS in ascending entry order. (Offsets staged
// in LDS instead, behind a barrier of their own, measured 0.7-2.8% slower;
// the entries loaded from the offsets rather than the plan, 1-4% slower.)
// Blocks over capacity read global memory. Every argument the block needs
// before its first vector load is among the preloaded ones (plan, tables,
// cgs).
template <bool kDot, int P>
__device__ __forceinline__ void gather_plan_body(const int32_t *__restrict__ plan,
                                                 const int32_t *__restrict__ off,
                                                 const int32_t *__restrict__ ids,
                                                 const double *__restrict__ vl,
                                                 double *__restrict__ vg, const double *cgs,
                                                 const double *__restrict__ w,
                                                 double *__restrict__ partials)
{
    if (skipped(cgs)) return;
    constexpr int K = kGatherCap / kBlock;  // entries per lane, and rows per lane at most
    __shared__ double stage[kGatherCap];
    // the block's four plan words in one round of scalar loads, before any
    // test uses them
    const int32_t *q = static_cast<const int32_t *>(__builtin_assume_aligned(plan + 4 * blockIdx.x, 16));
    const int32_t r0 = q[0], r1 = q[1], e0 = q[2], e1 = q[3];
    const int32_t nr = r1 - r0, ne = e1 - e0;
    double acc = 0.0;
    bool staged = false;
    if (nr <= kGatherCap && ne <= kGatherCap) {
        staged = true;
        int32_t id[K], oa[K], ob[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int32_t t = threadIdx.x + k * kBlock;
            id[k] = t < ne ? ldp<P>(ids + e0 + t) : -1;
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int32_t r = threadIdx.x + k * kBlock;
            oa[k] = r < nr ? off[r0 + r] : 0;
            ob[k] = r < nr ? off[r0 + r + 1] : 0;
        }
        double v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = id[k] >= 0 ? vl[id[k]] : 0.0;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int32_t t = threadIdx.x + k * kBlock;
            if (t < ne) stage[t] = v[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int32_t r = threadIdx.x + k * kBlock;
            if (r < nr) {
                double s = 0.0;
                for (int32_t j = oa[k] - e0; j < ob[k] - e0; ++j) s = s + stage[j];
                stp<P>(vg + r0 + r, s);
                if (kDot) acc = __builtin_fma(s, w[r0 + r], acc);
            }
        }
    }
    if (!staged) {
        for (int64_t g = (int64_t)r0 + threadIdx.x; g < r1; g += kBlock) {
            double s = 0.0;
            for (int32_t j = off[g]; j < off[g + 1]; ++j) s = s + vl[ids[j]];
            vg[g] = s;
            if (kDot) acc = __builtin_fma(s, w[g], acc);
        }
    }
    if (kDot) {
        const double part = block_sum(acc);
        if (threadIdx.x == 0) partials[blockIdx.x] = part;
    }
}

template <bool kDot>
__global__ __launch_bounds__(kBlock) void k_gather_plan(const int32_t *__restrict__ plan,
                                                        const int32_t *__restrict__ off,
                                                        const int32_t *__restrict__ ids,
                                                        const double *__restrict__ vl,
                                                        double *__restrict__ vg, const double *cgs,
                                                        const double *__restrict__ w,
                                                        double *__restrict__ partials)
{
    gather_plan_body<kDot, kStream>(plan, off, ids, vl, vg, cgs, w, partials);
}

// The same with the cache-keeping policy, for the CG iteration.
template <bool kDot>
__global__ __launch_bounds__(kBlock) void k_gather_plan_keep(const int32_t *__restrict__ plan,
                                                        const int32_t *__restrict__ off,
                                                        const int32_t *__restrict__ ids,
                                                        const double *__restrict__ vl,
                                                        double *__restrict__ vg, const double *cgs,
                                                        const double *__restrict__ w,
                                                        double *__restrict__ partials)
{
    gather_plan_body<kDot, kKeep>(plan, off, ids, vl, vg, cgs, w, partials);
}

// Scalar (8-byte) versions of the vector ops for operands whose 16-byte
// phases differ. Block b's tile is kScalarUnroll * kBlock consecutive
// elements, lane t taking t, t + kBlock, ...: every load of the tile issued
// before any store or sum (measured at 11.4M doubles, against one element
// per lane per step: AXPY 49.4 against 57.2 us, fused update 104.0 against
// 116.0 us, copy and dot unchanged; the aligned kernels take 43.3 and 85.9).
constexpr int kScalarUnroll = 4;  // elements per lane in flight in the 8-byte kernels

__global__ __launch_bounds__(kBlock) void k_copy_scalar(int64_t n, const double *x, double *y)
{
    constexpr int U = kScalarUnroll;
    const int64_t stride = kBlock, step = (int64_t)gridDim.x * U * kBlock;
    int64_t i = (int64_t)blockIdx.x * U * kBlock + threadIdx.x;
    for (; i + (U - 1) * stride < n; i += step) {
        double v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = x[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) y[i + u * stride] = v[u];
    }
    for (; i < n; i += stride) y[i] = x[i];
}

__global__ __launch_bounds__(kBlock) void k_axpy_scalar(int64_t n, double a, const double *x,
                                                        double b, double *y)
{
    constexpr int U = kScalarUnroll;
    const int64_t stride = kBlock, step = (int64_t)gridDim.x * U * kBlock;
    int64_t i = (int64_t)blockIdx.x * U * kBlock + threadIdx.x;
    for (; i + (U - 1) * stride < n; i += step) {
        double vx[U], vy[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            vx[u] = x[i + u * stride];
            vy[u] = y[i + u * stride];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) y[i + u * stride] = a * vx[u] + b * vy[u];
    }
    for (; i < n; i += stride) y[i] = a * x[i] + b * y[i];
}

__global__ __launch_bounds__(kBlock) void k_dot_scalar(int64_t n, const double *x, const double *y,
                                                       double *partials)
{
    constexpr int U = kScalarUnroll;
    const int64_t stride = kBlock, step = (int64_t)gridDim.x * U * kBlock;
    int64_t i = (int64_t)blockIdx.x * U * kBlock + threadIdx.x;
    double acc = 0.0;
    for (; i + (U - 1) * stride < n; i += step) {
        double vx[U], vy[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            vx[u] = x[i + u * stride];
            vy[u] = y[i + u * stride];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc = __builtin_fma(vx[u], vy[u], acc);
    }
    for (; i < n; i += stride) acc = __builtin_fma(x[i], y[i], acc);
    const double part = block_sum(acc);
    if (threadIdx.x == 0) partials[blockIdx.x] = part;
}

__global__ __launch_bounds__(kBlock) void k_cg_update_scalar(int64_t n, double a, const double *p,
                                                             const double *q, double *x, double *r,
                                                             double *partials)
{
    constexpr int U = kScalarUnroll;
    const int64_t stride = kBlock, step = (int64_t)gridDim.x * U * kBlock;
    int64_t i = (int64_t)blockIdx.x * U * kBlock + threadIdx.x;
    double acc = 0.0;
    for (; i + (U - 1) * stride < n; i += step) {
        double vp[U], vq[U], vx[U], vr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            vp[u] = p[i + u * stride];
            vq[u] = q[i + u * stride];
            vx[u] = x[i + u * stride];
            vr[u] = r[i + u * stride];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            x[i + u * stride] = vx[u] + a * vp[u];
            const double nr = vr[u] - a * vq[u];
            r[i + u * stride] = nr;
            acc = __builtin_fma(nr, nr, acc);
        }
    }
    for (; i < n; i += stride) {
        x[i] = x[i] + a * p[i];
        const double nr = r[i] - a * q[i];
        r[i] = nr;
        acc = __builtin_fma(nr, nr, acc);
    }
    const double part = block_sum(acc);
    if (threadIdx.x == 0) partials[blockIdx.x] = part;
}

// Sets the arrival counters of the one-kernel reductions to zero (the
// allocation-free CG solve clears its static counters this way at the start
// of every call: a kernel, so the call stays capturable in a HIP graph).
__global__ __launch_bounds__(kBlock) void k_zero_tickets(unsigned *tickets)
{
    for (int i = threadIdx.x; i < kTickets; i += kBlock) tickets[i] = 0u;
}

}  // namespace

// =================================================================== ABI ====

struct bs_ctx {
    int device;
    int cus;
    int max_partials;
    double *partials;   // first-stage reduction results, one per block
    unsigned *tickets;  // arrival counters of the one-kernel reductions (kTickets, zero between calls)
    double *cgs;        // device-resident CG scalars (CgSlot)
    hipEvent_t time_start, time_stop;  // armed by bs_ctx_time_next for the next kernel, else null
};

namespace {

inline bool misaligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

inline int launch_status() { return hipGetLastError() == hipSuccess ? BS_OK : BS_EHIP; }

// Every kernel of the operations goes through here. If bs_ctx_time_next has
// armed the context, this launch carries the two events, which the runtime
// sets to the kernel's own start and end, and the context disarms.
template <typename K, typename... Args>
void launch(bs_ctx *c, K kernel, dim3 grid, dim3 block, unsigned shmem, hipStream_t st, Args... args)
{
    if (c->time_start || c->time_stop) {
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, c->time_start, c->time_stop, 0, args...);
        c->time_start = c->time_stop = nullptr;
    } else {
        hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
    }
}

// Grid of a vector kernel with shape s over n2 pairs: the tiles needed, at
// most CUs * blocks_per_cu (when that is set). A reduction's grid is also
// bounded by the partials the context holds; any other grid by 2^22 blocks
// (the kernels loop over whatever a smaller grid leaves).
inline unsigned vector_grid(const bs_ctx *c, int64_t n2, VecShape s, bool reduction)
{
    const int64_t per = (int64_t)s.threads * s.unroll;
    int64_t g = (n2 + per - 1) / per;
    if (s.blocks_per_cu > 0 && g > (int64_t)c->cus * s.blocks_per_cu) g = (int64_t)c->cus * s.blocks_per_cu;
    const int64_t cap = reduction ? (int64_t)c->max_partials : (int64_t)1 << 22;
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    return (unsigned)g;
}

// Grid of an 8-byte kernel: one tile per block, at most 2^22 blocks (the
// kernels loop over whatever a smaller grid leaves), and for a reduction at
// most the partials the context holds.
inline unsigned scalar_grid(const bs_ctx *c, int64_t n, bool reduction = false)
{
    const int64_t per = (int64_t)kBlock * kScalarUnroll;
    int64_t g = (n + per - 1) / per;
    const int64_t cap = reduction ? (int64_t)c->max_partials : (int64_t)1 << 22;
    if (g > cap) g = cap;
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

// Makes a device current for the length of one ABI call and gives the
// calling thread its previous device back when the call returns.
class DeviceScope {
public:
    DeviceScope() = default;
    DeviceScope(const DeviceScope &) = delete;
    DeviceScope &operator=(const DeviceScope &) = delete;
    ~DeviceScope()
    {
        if (switched_) (void)hipSetDevice(prev_);
    }
    int enter(int device)
    {
        if (hipGetDevice(&prev_) != hipSuccess) return BS_EHIP;
        if (prev_ != device) {
            if (hipSetDevice(device) != hipSuccess) return BS_EHIP;
            switched_ = true;
        }
        return BS_OK;
    }
    int enter(const bs_ctx *c) { return c ? enter(c->device) : BS_EINVAL; }

private:
    int prev_ = -1;
    bool switched_ = false;
};

// Do the byte ranges [a, a + na) and [b, b + nb) share memory?
inline bool overlap(const void *a, int64_t na, const void *b, int64_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// Two double[n] operands that are the same array or do not meet at all.
inline bool same_or_apart(const double *a, const double *b, int64_t n)
{
    return a == b || !overlap(a, 8 * n, b, 8 * n);
}

int finish_launch(bs_ctx *c, unsigned nb, double *out, bool take_sqrt, hipStream_t st)
{
    launch(c, k_finish, dim3(1), dim3(kFinishBlock), 0, st, c->partials, (int)nb, out, take_sqrt);
    return launch_status();
}

// How a one-kernel reduction of this context stores its result.
Fin fin_out(const bs_ctx *c, double *out, bool take_sqrt)
{
    Fin f{};
    f.mode = take_sqrt ? kFinSqrt : kFinOut;
    f.partials = c->partials;
    f.tickets = c->tickets;
    f.out = out;
    return f;
}

Fin fin_cg(const bs_ctx *c, int mode, double *hist, int k, int iters, double tol2)
{
    Fin f{};
    f.mode = kFinCg;
    f.cg = mode;
    f.partials = c->partials;
    f.tickets = c->tickets;
    f.cgs = c->cgs;
    f.hist = hist;
    f.k = k;
    f.iters = iters;
    f.tol2 = tol2;
    return f;
}

// Second launch for the two-kernel paths (8-byte fallbacks).
int finish_two_stage(bs_ctx *c, unsigned nb, const Fin &f, hipStream_t st)
{
    if (f.mode == kFinCg) {
        launch(c, k_cg_finish, dim3(1), dim3(kFinishBlock), 0, st, c->partials, (int)nb, c->cgs, f.hist,
               f.k, f.iters, f.tol2, f.cg);
        return launch_status();
    }
    return finish_launch(c, nb, f.out, f.mode == kFinSqrt, st);
}

// norm / dot of n > 0 elements, finished as f says.
int dot_launch(bs_ctx *c, int64_t n, const double *x, const double *y, bool square, const Fin &f, hipStream_t st)
{
    const void *ptrs[2] = {x, square ? x : y};
    int64_t head;
    if (common_head(ptrs, 2, &head)) {
        const Split sp = split_of(n, head);
        if (square) {
            const unsigned g = vector_grid(c, sp.n2, kNormShape, true);
            launch(c, (k_dot<kNormShape.unroll, true, kNormShape.threads>), dim3(g), dim3(kNormShape.threads), 0, st,
                   sp.n2, x, x, ht_of(sp), g, f);
        } else {
            const unsigned g = vector_grid(c, sp.n2, kDotShape, true);
            launch(c, (k_dot<kDotShape.unroll, false, kDotShape.threads>), dim3(g), dim3(kDotShape.threads), 0, st,
                   sp.n2, x, y, ht_of(sp), g, f);
        }
        return launch_status();
    }
    const unsigned nb = scalar_grid(c, n, true);
    launch(c, k_dot_scalar, dim3(nb), dim3(kBlock), 0, st, n, x, y, c->partials);
    if (hipGetLastError() != hipSuccess) return BS_EHIP;
    return finish_two_stage(c, nb, f, st);
}

int reduce_launch(bs_ctx *c, int64_t n, const double *x, const double *y, double *out, bool square,
                  hipStream_t st)
{
    if (n == 0) return finish_launch(c, 0, out, false, st);
    return dot_launch(c, n, x, y, square, fin_out(c, out, square), st);
}

// Gather launch shared by bs_gather, bs_gather_dot and the CG iteration
// (keep: the plan kernel with the cache-keeping policy).
int gather_launch(bs_ctx *c, int64_t ng, const int32_t *off, const int32_t *ids, const double *vl, double *vg,
                  const int32_t *bstart, int64_t nblocks, const double *w, const double *cgs, hipStream_t st,
                  unsigned *nb, bool keep = false)
{
    if (bstart) {
        *nb = (unsigned)nblocks;
        if (w && keep)
            launch(c, k_gather_plan_keep<true>, dim3(*nb), dim3(kBlock), 0, st, bstart, off, ids, vl, vg,
                   cgs, w, c->partials);
        else if (w)
            launch(c, k_gather_plan<true>, dim3(*nb), dim3(kBlock), 0, st, bstart, off, ids, vl, vg, cgs,
                   w, c->partials);
        else
            launch(c, k_gather_plan<false>, dim3(*nb), dim3(kBlock), 0, st, bstart, off, ids, vl, vg,
                   cgs, nullptr, nullptr);
    } else {
        *nb = (unsigned)((ng + kSpanRows - 1) / kSpanRows);
        if (w && keep)
            launch(c, k_gather_span<true, kKeep>, dim3(*nb), dim3(kBlock), 0, st, ng, off, ids, vl, vg, cgs, w,
                   c->partials);
        else if (w)
            launch(c, k_gather_span<true, kStream>, dim3(*nb), dim3(kBlock), 0, st, ng, off, ids, vl, vg, cgs, w,
                   c->partials);
        else
            launch(c, k_gather_span<false, kStream>, dim3(*nb), dim3(kBlock), 0, st, ng, off, ids, vl, vg, cgs,
                   nullptr, nullptr);
    }
    return launch_status();
}

int gather_args(const bs_ctx *c, int64_t n_global, const int32_t *off, const int32_t *ids, const double *v_local,
                double *v_global, const int32_t *block_starts, int64_t n_blocks, bool dot)
{
    if (n_global < 0 || (n_global > 0 && (!off || !ids || !v_local || !v_global))) return BS_EINVAL;
    if (n_global >= INT32_MAX) return BS_ERANGE;
    if (n_global > 0 && (misaligned(off, 4) || misaligned(ids, 4) || misaligned(v_local, 8) ||
                         misaligned(v_global, 8)))
        return BS_EALIGN;
    if (block_starts && n_global > 0) {
        if (n_blocks < 1 || n_blocks > n_global) return BS_EINVAL;
        if (misaligned(block_starts, 16)) return BS_EALIGN;
    }
    // the fused dot writes one partial per block
    const int64_t nb = block_starts ? n_blocks : (n_global + kSpanRows - 1) / kSpanRows;
    if (dot && nb > c->max_partials) return BS_ERANGE;
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

int bs_version(void) { return 300; }

int bs_ctx_create(int device, bs_ctx **out)
{
    if (!out) return BS_EINVAL;
    *out = nullptr;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) return BS_EHIP;
    DeviceScope scope;
    if (scope.enter(device) != BS_OK) return BS_EHIP;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1)
        return BS_EHIP;
    bs_ctx *c = new (std::nothrow) bs_ctx;
    if (!c) return BS_ENOMEM;
    c->device = device;
    c->cus = cus;
    c->max_partials = kMaxPartials;
    c->partials = nullptr;
    c->tickets = nullptr;
    c->cgs = nullptr;
    c->time_start = c->time_stop = nullptr;
    if (hipMalloc(&c->partials, sizeof(double) * kMaxPartials) != hipSuccess ||
        hipMalloc(&c->tickets, sizeof(unsigned) * kTickets) != hipSuccess ||
        hipMalloc(&c->cgs, sizeof(double) * kCgSlots) != hipSuccess) {
        if (c->partials) (void)hipFree(c->partials);
        if (c->tickets) (void)hipFree(c->tickets);
        delete c;
        return BS_ENOMEM;
    }
    // the tickets start at zero; every reduction leaves them at zero
    if (hipMemset(c->tickets, 0, sizeof(unsigned) * kTickets) != hipSuccess) {
        (void)hipFree(c->partials);
        (void)hipFree(c->tickets);
        (void)hipFree(c->cgs);
        delete c;
        return BS_EHIP;
    }
    *out = c;
    return BS_OK;
}

void bs_ctx_destroy(bs_ctx *c)
{
    if (!c) return;
    DeviceScope scope;
    if (scope.enter(c->device) == BS_OK) {
        (void)hipDeviceSynchronize();
        (void)hipFree(c->partials);
        (void)hipFree(c->tickets);
        (void)hipFree(c->cgs);
    }
    delete c;
}

int bs_ctx_time_next(bs_ctx *c, void *start_event, void *stop_event)
{
    if (!c) return BS_EINVAL;
    c->time_start = static_cast<hipEvent_t>(start_event);
    c->time_stop = static_cast<hipEvent_t>(stop_event);
    return BS_OK;
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
    DeviceScope scope;
    if (int s = scope.enter(c)) return s;
    if (n < 0 || (n > 0 && (!x || !y))) return BS_EINVAL;
    if (misaligned(x, 8) || misaligned(y, 8)) return BS_EALIGN;
    if (!same_or_apart(x, y, n)) return BS_EINVAL;
    // a copy onto itself changes nothing (and keeps the kernel's restrict
    // qualifiers honest)
    if (n == 0 || x == y) return BS_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const void *ptrs[2] = {x, y};
    int64_t head;
    if (common_head(ptrs, 2, &head)) {
        const Split sp = split_of(n, head);
        if (sp.n2 <= kCopyLargePairs)
            launch(c, k_copy<kCopyShape.unroll, kCopyShape.threads>, dim3(vector_grid(c, sp.n2, kCopyShape, false)),
                   dim3(kCopyShape.threads), 0, st, sp.n2, x, y, sp.head, sp.tail);
        else
            launch(c, k_copy<kCopyLargeShape.unroll, kCopyLargeShape.threads>,
                   dim3(vector_grid(c, sp.n2, kCopyLargeShape, false)), dim3(kCopyLargeShape.threads), 0, st, sp.n2,
                   x, y, sp.head, sp.tail);
    } else {
        launch(c, k_copy_scalar, dim3(scalar_grid(c, n)), dim3(kBlock), 0, st, n, x, y);
    }
    return launch_status();
}

int bs_axpy(bs_ctx *c, int64_t n, double alpha, const double *x, double beta, double *y, void *stream)
{
    DeviceScope scope;
    if (int s = scope.enter(c)) return s;
    if (n < 0 || (n > 0 && (!x || !y))) return BS_EINVAL;
    if (n == 0) return BS_OK;
    if (misaligned(x, 8) || misaligned(y, 8)) return BS_EALIGN;
    if (!same_or_apart(x, y, n)) return BS_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const void *ptrs[2] = {x, y};
    int64_t head;
    if (common_head(ptrs, 2, &head)) {
        const Split sp = split_of(n, head);
        const unsigned g = vector_grid(c, sp.n2, kAxpyShape, false);
        launch(c, k_axpy<kAxpyShape.unroll>, dim3(g), dim3(kBlock), 0, st, sp.n2, x, y, alpha, beta, ht_of(sp), g);
    } else {
        launch(c, k_axpy_scalar, dim3(scalar_grid(c, n)), dim3(kBlock), 0, st, n, alpha, x, beta, y);
    }
    return launch_status();
}

int bs_scale(bs_ctx *c, int64_t n, const double *x, const double *d, double *y, void *stream)
{
    DeviceScope scope;
    if (int s = scope.enter(c)) return s;
    if (n < 0 || (n > 0 && (!x || !d || !y))) return BS_EINVAL;
    if (n == 0) return BS_OK;
    if (misaligned(x, 8) || misaligned(d, 8) || misaligned(y, 8)) return BS_EALIGN;
    if (!same_or_apart(x, y, n) || !same_or_apart(d, y, n)) return BS_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const void *ptrs[3] = {x, d, y};
    int64_t head;
    if (common_head(ptrs, 3, &head)) {
        const Split sp = split_of(n, head);
        launch(c, k_scale<kAxpyShape.unroll>, dim3(vector_grid(c, sp.n2, kAxpyShape, false)), dim3(kBlock),
               0, st, sp.n2, x, d, y, sp.head, sp.tail);
    } else {
        launch(c, k_scale_scalar, dim3(scalar_grid(c, n)), dim3(kBlock), 0, st, n, x, d, y);
    }
    return launch_status();
}

int bs_norm(bs_ctx *c, int64_t n, const double *x, double *result, void *stream)
{
    DeviceScope scope;
    if (int s = scope.enter(c)) return s;
    if (n < 0 || !result || (n > 0 && !x)) return BS_EINVAL;
    if ((n > 0 && misaligned(x, 8)) || misaligned(result, 8)) return BS_EALIGN;
    return reduce_launch(c, n, x, x, result, true, static_cast<hipStream_t>(stream));
}

int bs_dot(bs_ctx *c, int64_t n, const double *x, const double *y, double *result, void *stream)
{
    DeviceScope scope;
    if (int s = scope.enter(c)) return s;
    if (n < 0 || !result || (n > 0 && (!x || !y))) return BS_EINVAL;
    if ((n > 0 && (misaligned(x, 8) || misaligned(y, 8))) || misaligned(result, 8)) return BS_EALIGN;
    return reduce_launch(c, n, x, y, result, false, static_cast<hipStream_t>(stream));
}

int bs_cg_update(bs_ctx *c, int64_t n, double alpha, const double *p, const double *q, double *x,
                 double *r, double *rr, void *stream)
{
    DeviceScope scope;
    if (int s = scope.enter(c)) return s;
    if (n < 0 || !rr || (n > 0 && (!p || !q || !x || !r))) return BS_EINVAL;
    if ((n > 0 && (misaligned(p, 8) || misaligned(q, 8) || misaligned(x, 8) || misaligned(r, 8))) ||
        misaligned(rr, 8))
        return BS_EALIGN;
    // x and r are written through restrict pointers: neither may meet the
    // other or p, q (p and q are only read and may be the same array)
    const int64_t nbytes = 8 * n;
    if (overlap(x, nbytes, r, nbytes) || overlap(x, nbytes, p, nbytes) || overlap(x, nbytes, q, nbytes) ||
        overlap(r, nbytes, p, nbytes) || overlap(r, nbytes, q, nbytes))
        return BS_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (n == 0) return finish_launch(c, 0, rr, false, st);
    const void *ptrs[4] = {p, q, x, r};
    int64_t head;
    if (common_head(ptrs, 4, &head)) {
        const Split sp = split_of(n, head);
        const unsigned g = vector_grid(c, sp.n2, kCgShape, true);
        launch(c, k_cg_update<kCgShape.unroll, kCgRUnroll, kCgShape.threads>, dim3(g), dim3(kCgShape.threads), 0, st,
               sp.n2, p, q, x, r, alpha, ht_of(sp), g, fin_out(c, rr, false));
        return launch_status();
    }
    const unsigned nb = scalar_grid(c, n, true);
    launch(c, k_cg_update_scalar, dim3(nb), dim3(kBlock), 0, st, n, alpha, p, q, x, r, c->partials);
    if (hipGetLastError() != hipSuccess) return BS_EHIP;
    return finish_launch(c, nb, rr, false, st);
}

int bs_scatter(bs_ctx *c, int64_t n_local, const int32_t *l2g, const double *v_global, double *v_local,
               void *stream)
{
    DeviceScope scope;
    if (int s = scope.enter(c)) return s;
    if (n_local < 0 || (n_local > 0 && (!l2g || !v_global || !v_local))) return BS_EINVAL;
    if (n_local > INT32_MAX) return BS_ERANGE;
    if (n_local == 0) return BS_OK;
    if (misaligned(l2g, 4) || misaligned(v_global, 8) || misaligned(v_local, 8)) return BS_EALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!misaligned(l2g, 8) && !misaligned(v_local, 16)) {
        const int64_t per = 2LL * kBlock * kScatterPairs;
        const int64_t nb = (n_local + per - 1) / per;
        launch(c, k_scatter, dim3((unsigned)nb), dim3(kBlock), 0, st, n_local, l2g, v_global, v_local,
               nullptr);
    } else {
        const int64_t per = (int64_t)kBlock * kScatterScalarEntries;
        const int64_t nb = (n_local + per - 1) / per;
        launch(c, k_scatter_scalar, dim3((unsigned)nb), dim3(kBlock), 0, st, n_local, l2g, v_global,
               v_local);
    }
    return launch_status();
}

int bs_gather(bs_ctx *c, int64_t n_global, const int32_t *off, const int32_t *ids, const double *v_local,
              double *v_global, const int32_t *block_starts, int64_t n_blocks, void *stream)
{
    DeviceScope scope;
    if (int s = scope.enter(c)) return s;
    if (int s = gather_args(c, n_global, off, ids, v_local, v_global, block_starts, n_blocks, false)) return s;
    if (n_global == 0) return BS_OK;
    unsigned nb;
    return gather_launch(c, n_global, off, ids, v_local, v_global, block_starts, n_blocks, nullptr, nullptr,
                         static_cast<hipStream_t>(stream), &nb);
}

int bs_gather_dot(bs_ctx *c, int64_t n_global, const int32_t *off, const int32_t *ids, const double *v_local,
                  double *v_global, const int32_t *block_starts, int64_t n_blocks, const double *w,
                  double *result, void *stream)
{
    DeviceScope scope;
    if (int s = scope.enter(c)) return s;
    if (!result || (n_global > 0 && !w)) return BS_EINVAL;
    if (int s = gather_args(c, n_global, off, ids, v_local, v_global, block_starts, n_blocks, true)) return s;
    if (misaligned(result, 8) || (n_global > 0 && misaligned(w, 8))) return BS_EALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (n_global == 0) return finish_launch(c, 0, result, false, st);
    unsigned nb;
    if (int s = gather_launch(c, n_global, off, ids, v_local, v_global, block_starts, n_blocks, w, nullptr, st,
                              &nb))
        return s;
    return finish_launch(c, nb, result, false, st);
}

}  // extern "C"

namespace {

// The device-resident CG iteration on the scratch of `c` (a context, or the
// static scratch of bs_cg_solve_static, which asks for its ticket counters to
// be cleared first). The device of `c` is current.
int cg_solve_run(bs_ctx *c, int64_t n_global, int64_t n_local, const int32_t *l2g, const int32_t *off,
                 const int32_t *ids, const int32_t *block_starts, int64_t n_blocks, double *x, double *r, double *p,
                 double *q, double *p_local, int iters, double tol, double *rr_hist, void *stream,
                 bool zero_tickets)
{
    if (n_global < 1 || n_local < 1 || iters < 0 || !(tol >= 0.0) || !l2g || !x || !r || !p || !q || !p_local ||
        !rr_hist)
        return BS_EINVAL;
    if (n_local > INT32_MAX) return BS_ERANGE;
    if (int s = gather_args(c, n_global, off, ids, p_local, q, block_starts, n_blocks, true)) return s;
    const void *vec[6] = {x, r, p, q, p_local, rr_hist};
    for (const void *v : vec)
        if (misaligned(v, 16) && v != rr_hist) return BS_EALIGN;
    if (misaligned(rr_hist, 8) || misaligned(l2g, 8)) return BS_EALIGN;
    {
        // every vector of the iteration is written at some step: no two may meet
        const void *arr[5] = {x, r, p, q, p_local};
        const int64_t len[5] = {8 * n_global, 8 * n_global, 8 * n_global, 8 * n_global, 8 * n_local};
        for (int i = 0; i < 5; ++i)
            for (int j = i + 1; j < 5; ++j)
                if (overlap(arr[i], len[i], arr[j], len[j])) return BS_EINVAL;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Split sp = split_of(n_global, 0);
    const double *cgs = c->cgs;
    if (zero_tickets) {
        launch(c, k_zero_tickets, dim3(1), dim3(kBlock), 0, st, c->tickets);
        if (hipGetLastError() != hipSuccess) return BS_EHIP;
    }
    // rr0 = r.r, history, threshold
    if (int s = dot_launch(c, n_global, r, r, true, fin_cg(c, kStart, rr_hist, 0, iters, tol * tol), st)) return s;
    unsigned nb;
    const int64_t sc_per = 2LL * kBlock * kScatterPairs;
    const unsigned sc_nb = (unsigned)((n_local + sc_per - 1) / sc_per);
    const unsigned cg_nb = vector_grid(c, sp.n2, kCgShape, true);
    const unsigned cg1_nb = vector_grid(c, sp.n2, kCgOnePassShape, true);
    const unsigned ax_nb = vector_grid(c, sp.n2, kAxpyShape, false);
    // Kernels of the iteration hand x, r, p, q and p_local to each other and
    // read the tables every iteration. When all of it fits in the last-level
    // cache, the cache-keeping kernels leave it there for the next kernel;
    // larger working sets stream non-temporally like the standalone
    // operations (measured: 7-12% faster per iteration up to ~190 MB, equal
    // near 320 MB, 11% slower at 680 MB with the keeping policy).
    const int64_t working_set = 8 * (4 * n_global + n_local) + 4 * (2 * n_local + n_global + 1) +
                                (block_starts ? 16 * n_blocks : 0);
    const bool keep = working_set <= kCacheResidentBytes;
    // Otherwise, while r and p alone fit, the update hands them to the
    // direction update through the cache (1-3% per iteration at 24^3-32^3,
    // order 7).
    const bool handoff = !keep && 16 * n_global <= kHandoffBytes;
    for (int k = 0; k < iters; ++k) {
        // q = Z^T Z p and p.q in the gather's pass; alpha = rr / p.q
        if (keep)
            launch(c, k_scatter_keep, dim3(sc_nb), dim3(kBlock), 0, st, n_local, l2g, p, p_local, cgs);
        else
            launch(c, k_scatter, dim3(sc_nb), dim3(kBlock), 0, st, n_local, l2g, p, p_local, cgs);
        if (int s = gather_launch(c, n_global, off, ids, p_local, q, block_starts, n_blocks, p, cgs, st, &nb, keep))
            return s;
        launch(c, k_cg_finish, dim3(1), dim3(kFinishBlock), 0, st, c->partials, (int)nb, c->cgs,
               rr_hist, k, iters, 0.0, (int)kSetAlpha);
        // x += alpha p, r -= alpha q, r.r; beta = rr' / rr (the update's last block).
        // Two passes when the iteration is cache-resident; otherwise one pass,
        // which overlaps the cached part of p (left by the scatter) with HBM.
        if (keep)
            launch(c, k_cg_update_keep<kCgShape.unroll, kCgRUnroll, kCgShape.threads>, dim3(cg_nb),
                   dim3(kCgShape.threads), 0, st, sp.n2, p, q, x, r, cgs, ht_of(sp), cg_nb,
                   fin_cg(c, kSetBeta, rr_hist, k, iters, 0.0));
        else if (handoff)
            launch(c, k_cg_update_handoff<kCgOnePassShape.unroll>, dim3(cg1_nb), dim3(kBlock), 0, st, sp.n2, p, q,
                   x, r, cgs, ht_of(sp), cg1_nb, fin_cg(c, kSetBeta, rr_hist, k, iters, 0.0));
        else
            launch(c, k_cg_update_one_pass<kCgOnePassShape.unroll>, dim3(cg1_nb), dim3(kBlock), 0, st, sp.n2, p,
                   q, x, r, cgs, ht_of(sp), cg1_nb, fin_cg(c, kSetBeta, rr_hist, k, iters, 0.0));
        // p = (1 r) + (beta p)
        if (keep || handoff)
            launch(c, k_axpy_keep<kAxpyShape.unroll>, dim3(ax_nb), dim3(kBlock), 0, st, sp.n2, r, p, cgs, ht_of(sp),
                   ax_nb);
        else
            launch(c, k_axpy_dev<kAxpyShape.unroll>, dim3(ax_nb), dim3(kBlock), 0, st, sp.n2, r, p, cgs, ht_of(sp),
                   ax_nb);
        if (hipGetLastError() != hipSuccess) return BS_EHIP;
    }
    return BS_OK;
}

// ------------------------------------------------ allocation-free solve ----
// Scratch of bs_cg_solve_static: the ticket counters, the CG scalars and up
// to kStaticPartials reduction partials, in one static device array. Each GPU
// the library runs on holds its own copy for the life of the process; its
// address there is taken once per device with hipGetSymbolAddress (in host
// code the array's name is not a device address).
constexpr int kStaticPartials = 1 << 17;  // 1 MiB: gathers of up to 131072 blocks
constexpr int kStaticTicketDoubles = kTickets * (int)sizeof(unsigned) / (int)sizeof(double);
constexpr int kStaticCgDoubles = 32;  // kCgSlots doubles, padded to 256 bytes
constexpr int kStaticDoubles = kStaticTicketDoubles + kStaticCgDoubles + kStaticPartials;
static_assert(kTickets * sizeof(unsigned) % 256 == 0, "tickets fill whole 256-byte lines");
static_assert(kCgSlots <= kStaticCgDoubles, "CG scalars fit their slot");

}  // namespace

static __device__ __align__(256) double scratch[kStaticDoubles];

namespace {

constexpr int kMaxStaticDevices = 64;
struct StaticScratch {
    double *base = nullptr;  // device address of `scratch` on this device
    int cus = 0;
};
StaticScratch g_static[kMaxStaticDevices];
std::mutex g_static_mutex;

// Set-up on first use on a device (the device is current): its copy's
// address and its compute-unit count. Allocates nothing.
int static_scratch(int device, StaticScratch *out)
{
    if (device < 0 || device >= kMaxStaticDevices) return BS_EINVAL;
    std::lock_guard<std::mutex> lock(g_static_mutex);
    StaticScratch &s = g_static[device];
    if (!s.base) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1)
            return BS_EHIP;
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return BS_EHIP;
        s.cus = cus;
        s.base = static_cast<double *>(ptr);
    }
    *out = s;
    return BS_OK;
}

}  // namespace

extern "C" {

int bs_cg_solve(bs_ctx *c, int64_t n_global, int64_t n_local, const int32_t *l2g, const int32_t *off,
                const int32_t *ids, const int32_t *block_starts, int64_t n_blocks, double *x, double *r,
                double *p, double *q, double *p_local, int iters, double tol, double *rr_hist, void *stream)
{
    DeviceScope scope;
    if (int s = scope.enter(c)) return s;
    return cg_solve_run(c, n_global, n_local, l2g, off, ids, block_starts, n_blocks, x, r, p, q, p_local, iters,
                        tol, rr_hist, stream, false);
}

int bs_cg_solve_static(int64_t n_global, int64_t n_local, const int32_t *l2g, const int32_t *off,
                       const int32_t *ids, const int32_t *block_starts, int64_t n_blocks, double *x, double *r,
                       double *p, double *q, double *p_local, int iters, double tol, double *rr_hist,
                       void *stream)
{
    // the checks that need no device first, so that they fail without a HIP call
    if (n_global < 1 || n_local < 1 || iters < 0 || !(tol >= 0.0) || !l2g || !off || !ids || !x || !r || !p || !q ||
        !p_local || !rr_hist)
        return BS_EINVAL;
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) return BS_EHIP;
    StaticScratch ss;
    if (int s = static_scratch(device, &ss)) return s;
    // a context on the stack whose scratch is this device's static array
    bs_ctx c{};
    c.device = device;
    c.cus = ss.cus;
    c.max_partials = kStaticPartials;
    c.tickets = reinterpret_cast<unsigned *>(ss.base);
    c.cgs = ss.base + kStaticTicketDoubles;
    c.partials = c.cgs + kStaticCgDoubles;
    c.time_start = c.time_stop = nullptr;
    return cg_solve_run(&c, n_global, n_local, l2g, off, ids, block_starts, n_blocks, x, r, p, q, p_local, iters,
                        tol, rr_hist, stream, true);
}

}  // extern "C"
