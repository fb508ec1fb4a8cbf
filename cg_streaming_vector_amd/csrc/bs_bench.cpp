// bs_bench.cpp -- host-timed launch loop for the streaming operations.
//
// The BS paper times each test on the host around a run of back-to-back
// launches of the kernel ("Portable high-order finite element kernels I",
// arXiv 2009.10917, the performance model: T(B) = T0 + B / W_max, eq. 8,
// where T0 is the fixed cost of a launch). Doing the loop here, in C++, keeps
// interpreter overhead out of T0: what remains is the runtime's launch path
// and the kernels themselves.

#include <chrono>

#include <hip/hip_runtime.h>

#include "bs.h"

extern "C" int bs_bench_loop(bs_ctx *ctx, int op, int64_t n, double alpha, double beta, int64_t n_blocks,
                             int n_sets, void *const *sets, double *result, int reps, void *stream,
                             double *seconds)
{
    if (!ctx || !sets || !seconds || n_sets < 1 || reps < 1 || n < 0) return BS_EINVAL;
    if (op < BS_OP_COPY || op > BS_OP_GATHER) return BS_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipStreamSynchronize(st) != hipSuccess) return BS_EHIP;
    const auto t0 = std::chrono::steady_clock::now();
    for (int rep = 0; rep < reps; ++rep) {
        void *const *s = sets + BS_BENCH_SET * (rep % n_sets);
        double *a = static_cast<double *>(s[0]), *b = static_cast<double *>(s[1]);
        double *c = static_cast<double *>(s[2]), *d = static_cast<double *>(s[3]);
        int rc = BS_OK;
        switch (op) {
        case BS_OP_COPY: rc = bs_copy(ctx, n, a, b, stream); break;
        case BS_OP_AXPY: rc = bs_axpy(ctx, n, alpha, a, beta, b, stream); break;
        case BS_OP_NORM: rc = bs_norm(ctx, n, a, result, stream); break;
        case BS_OP_DOT: rc = bs_dot(ctx, n, a, b, result, stream); break;
        case BS_OP_CG_UPDATE: rc = bs_cg_update(ctx, n, alpha, a, b, c, d, result, stream); break;
        case BS_OP_SCALE: rc = bs_scale(ctx, n, a, b, c, stream); break;
        case BS_OP_SCATTER:
            rc = bs_scatter(ctx, n, static_cast<const int32_t *>(s[0]), b, c, stream);
            break;
        case BS_OP_GATHER:
            rc = bs_gather(ctx, n, static_cast<const int32_t *>(s[0]), static_cast<const int32_t *>(s[1]), c, d,
                           static_cast<const int32_t *>(s[4]), n_blocks, stream);
            break;
        }
        if (rc != BS_OK) {
            (void)hipStreamSynchronize(st);
            return rc;
        }
    }
    if (hipStreamSynchronize(st) != hipSuccess) return BS_EHIP;
    *seconds = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    return BS_OK;
}
