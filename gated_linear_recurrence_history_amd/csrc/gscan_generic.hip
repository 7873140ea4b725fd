// The scan for the shapes outside the fused kernels' envelope (SH2 a multiple
// of 16 up to 1024 that is not a multiple of 64, or beyond 512), in the
// structure of the design spec "Custom Kernel Optimization - cuBLAS
// Projections + Batch-Parallel Scans", Design 1: the projections of
// Forward Step 1 written to a scratch buffer (split-bf16 products on the
// matrix cores, both projections in one launch: gscan_proj2_kernel), then
// the lightweight scan with one thread per (sample, state); for the
// backward, the replayed projections, the reverse scan (the per-sample
// adjoint pass shared with the general kernel) and the weight-gradient
// contractions of Backward Step 3 into per-slab partials (the split
// backward's contraction loop with ragged tiles, both contractions in one
// launch: gscan_gen_contract_kernel), summed by the fixed-order reduction.
#include <cstdint>

#include "gscan_internal.h"

namespace gscan {
namespace {

constexpr int kGenThreads = 256;

// Forward Step 2, one thread per (sample b, state s): x = 0, then x =
// sigmoid(A + a_shift) * x + Bv over the K rows of the sample (ab holds
// A | Bv per row, [B*K][2D]); context = C * x_K.
__global__ void __launch_bounds__(kGenThreads)
gscan_gen_fwd_scan_kernel(const float *__restrict__ ab, const float *__restrict__ cv, int64_t B,
                          int64_t K, int D, float a_shift, CtxOut out)
{
    const int64_t n = B * D;
    for (int64_t e = (int64_t)blockIdx.x * kGenThreads + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * kGenThreads) {
        const int64_t b = e / D;
        const int s = (int)(e % D);
        const float *row = ab + b * K * 2 * D;
        float x = 0.f;
        // steps in chunks of kC whose loads all go out before the chunk's
        // arithmetic, so that they are in flight together
        constexpr int kC = 8;
        for (int64_t t0 = 0; t0 < K; t0 += kC) {
            const int n = K - t0 < kC ? (int)(K - t0) : kC;
            float av[kC], bv[kC];
#pragma unroll
            for (int u = 0; u < kC; ++u) {
                if (u < n) {
                    av[u] = row[(t0 + u) * 2 * D + s];
                    bv[u] = row[(t0 + u) * 2 * D + D + s];
                }
            }
#pragma unroll
            for (int u = 0; u < kC; ++u) {
                if (u < n) {
                    const float g = __builtin_amdgcn_rcpf(1.0f + __expf(-(av[u] + a_shift)));
                    x = g * x + bv[u];
                }
            }
        }
        const float v = cv[b * D + s] * x;
        if (out.ctx) out.ctx[b * D + s] = v;
        if (out.enr) {
            float *p = out.enr + b * out.ld + s;
            *p = *p + v;
        }
    }
}

hipError_t gen_forward(const Plan &p, const void *hh, const void *hs2, const float *WA,
                       const float *WB, const float *WC, float a_shift, const CtxOut &ctx,
                       float *ab, float *cv, hipStream_t st)
{
    hipError_t e = launch_proj_ab_c(p.dtype, hh, hs2, WA, WB, WC, p.B * p.K, p.B, p.SH2, p.D, ab,
                                    cv, st);
    if (e != hipSuccess) return e;
    const int64_t n = p.B * p.D;
    const int64_t blocks = (n + kGenThreads - 1) / kGenThreads;
    hipLaunchKernelGGL(gscan_gen_fwd_scan_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)),
                       dim3(kGenThreads), 0, st, ab, cv, p.B, p.K, (int)p.D, a_shift, ctx);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gen_forward(const Plan &p, const void *hh, const void *hs2, const float *WA,
                              const float *WB, const float *WC, float a_shift, const CtxOut &ctx,
                              float *ab, float *cv, hipStream_t st)
{
    return gen_forward(p, hh, hs2, WA, WB, WC, a_shift, ctx, ab, cv, st);
}

hipError_t launch_gen_partials(const Plan &p, const void *hh, const void *hs2, const float *WA,
                               const float *WB, const float *WC, float a_shift,
                               const float *dctx, float *part, float *ab, float *cv,
                               hipStream_t st)
{
    // replayed projections, the exact adjoints in place, then the
    // contractions of Backward Step 3 into the slab partials
    hipError_t e = launch_proj_ab_c(p.dtype, hh, hs2, WA, WB, WC, p.B * p.K, p.B, p.SH2, p.D, ab,
                                    cv, st);
    if (e == hipSuccess) e = launch_adjoint(p, ab, cv, dctx, a_shift, st);
    if (e == hipSuccess) e = launch_gen_contract(p, hh, hs2, ab, cv, part, st);
    return e;
}

}  // namespace gscan
