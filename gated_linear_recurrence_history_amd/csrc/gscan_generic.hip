// The scan for the shapes outside the fused kernels' envelope (SH2 a multiple
// of 16 up to 1024 that is not a multiple of 64, or beyond 512), in the
// structure of the design spec "Custom Kernel Optimization - cuBLAS
// Projections + Batch-Parallel Scans", Design 1: the projections of
// Forward Step 1 materialised in a scratch buffer, then the lightweight
// scan with one thread per (sample, state); for the backward, the replayed
// projections, the reverse scan (the per-sample adjoint pass shared with
// the general kernel) and the weight-gradient contractions of Backward
// Step 3 into per-slab partials, summed by the fixed-order reduction.
// Plain fp32 fused multiply-adds in a fixed order throughout (no split
// products): these shapes trade speed for reach.
#include <cstdint>

#include "gscan_internal.h"

namespace gscan {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kGenThreads = 256;
constexpr int kGenTile = 64;  // output tile edge (rows x outputs, or i x o)
constexpr int kGenK = 16;     // contraction chunk staged per round

template <typename T> __device__ __forceinline__ float widen(T v);
template <> __device__ __forceinline__ float widen<float>(float v) { return v; }
template <> __device__ __forceinline__ float widen<uint16_t>(uint16_t v)
{
    return __uint_as_float((uint32_t)v << 16);
}

// out[r][o] = sum_k X[r][k] * Wk(k, o) for r < R, o < NO, k < KC, where
// Wk(k, o) = W1[k][o] (row pitch D1) for o < D1, else W2[k][o - D1]:
// [A | Bv] = h_history [W_A | W_B] and C = h_s2 W_C.  A workgroup computes
// a 64 x 64 tile (4 x 4 per thread), the k index in chunks of 16 through
// LDS, in increasing k order.  Row tiles are walked grid-stride.
template <typename TIn>
__global__ void __launch_bounds__(kGenThreads)
gscan_gen_proj_kernel(const TIn *__restrict__ X, const float *__restrict__ W1,
                      const float *__restrict__ W2, int64_t R, int KC, int D1, int NO,
                      float *__restrict__ out)
{
    __shared__ float xs[kGenK][kGenTile + 4];
    __shared__ float ws[kGenK][kGenTile + 4];
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    const int o0 = blockIdx.y * kGenTile;
    const int64_t tiles = (R + kGenTile - 1) / kGenTile;
    for (int64_t rt = blockIdx.x; rt < tiles; rt += gridDim.x) {
        const int64_t r0 = rt * kGenTile;
        float acc[4][4] = {};
        for (int k0 = 0; k0 < KC; k0 += kGenK) {
            // stage X[r0 .. +64][k0 .. +16] (as [k][r]) and W[k0 .. +16][o0 .. +64]
#pragma unroll
            for (int u = 0; u < kGenK * kGenTile / kGenThreads; ++u) {
                const int e = tid + kGenThreads * u;
                const int rr = e / kGenK, kk = e % kGenK;
                const int64_t r = r0 + rr;
                xs[kk][rr] = r < R ? widen<TIn>(X[r * KC + k0 + kk]) : 0.f;
                const int oo = e % kGenTile, kw = e / kGenTile;
                const int o = o0 + oo;
                const int k = k0 + kw;
                float w = 0.f;
                if (o < NO) w = o < D1 ? W1[(int64_t)k * D1 + o] : W2[(int64_t)k * (NO - D1) + (o - D1)];
                ws[kw][oo] = w;
            }
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < kGenK; ++kk) {
                float a[4], b[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    a[j] = xs[kk][4 * ty + j];
                    b[j] = ws[kk][4 * tx + j];
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int l = 0; l < 4; ++l) acc[j][l] = fmaf(a[j], b[l], acc[j][l]);
            }
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t r = r0 + 4 * ty + j;
            if (r >= R) continue;
#pragma unroll
            for (int l = 0; l < 4; ++l) {
                const int o = o0 + 4 * tx + l;
                if (o < NO) out[r * NO + o] = acc[j][l];
            }
        }
    }
}

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
        for (int64_t t = 0; t < K; ++t) {
            const float a = row[t * 2 * D + s] + a_shift;
            const float g = __builtin_amdgcn_rcpf(1.0f + __expf(-a));
            x = g * x + row[t * 2 * D + D + s];
        }
        const float v = cv[b * D + s] * x;
        if (out.ctx) out.ctx[b * D + s] = v;
        if (out.enr) {
            float *p = out.enr + b * out.ld + s;
            *p = *p + v;
        }
    }
}

// Backward Step 3 for one slab of rows: part[slab][which0 + o / D][i][o % D]
// = sum over the slab's rows r (in increasing order) of X[r][i] * Y[r][o],
// i < SH2, o < NO.  A workgroup computes a 64 x 64 (i, o) tile, the rows in
// chunks of 16 through LDS.
template <typename TIn>
__global__ void __launch_bounds__(kGenThreads)
gscan_gen_contract_kernel(const TIn *__restrict__ X, const float *__restrict__ Y, int64_t rows,
                          int64_t rows_per_slab, int SH2, int NO, int D, int which0,
                          float *__restrict__ part)
{
    __shared__ float xs[kGenK][kGenTile + 4];
    __shared__ float ys[kGenK][kGenTile + 4];
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    const int64_t slab = blockIdx.x;
    const int i0 = blockIdx.y * kGenTile, o0 = blockIdx.z * kGenTile;
    const int64_t rb = slab * rows_per_slab;
    const int64_t re = rb + rows_per_slab < rows ? rb + rows_per_slab : rows;
    float acc[4][4] = {};
    for (int64_t r0 = rb; r0 < re; r0 += kGenK) {
#pragma unroll
        for (int u = 0; u < kGenK * kGenTile / kGenThreads; ++u) {
            const int e = tid + kGenThreads * u;
            const int kk = e / kGenTile, cc = e % kGenTile;
            const int64_t r = r0 + kk;
            const bool rv = r < re;
            const int i = i0 + cc, o = o0 + cc;
            xs[kk][cc] = rv && i < SH2 ? widen<TIn>(X[r * SH2 + i]) : 0.f;
            ys[kk][cc] = rv && o < NO ? Y[r * NO + o] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kGenK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                a[j] = xs[kk][4 * ty + j];
                b[j] = ys[kk][4 * tx + j];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int l = 0; l < 4; ++l) acc[j][l] = fmaf(a[j], b[l], acc[j][l]);
        }
        __syncthreads();
    }
    float *P = part + slab * 3 * (int64_t)SH2 * D;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = i0 + 4 * ty + j;
        if (i >= SH2) continue;
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            const int o = o0 + 4 * tx + l;
            if (o >= NO) continue;
            const int which = which0 + o / D, s = o % D;
            P[((int64_t)which * SH2 + i) * D + s] = acc[j][l];
        }
    }
}

template <typename TIn>
hipError_t proj(const TIn *X, const float *W1, const float *W2, int64_t R, int64_t KC, int64_t D1,
                int64_t NO, float *out, hipStream_t st)
{
    if (R <= 0) return hipSuccess;
    const int64_t tiles = (R + kGenTile - 1) / kGenTile;
    const unsigned gx = (unsigned)(tiles < 16384 ? tiles : 16384);
    const dim3 grid(gx, (unsigned)((NO + kGenTile - 1) / kGenTile));
    hipLaunchKernelGGL((gscan_gen_proj_kernel<TIn>), grid, dim3(kGenThreads), 0, st, X, W1, W2, R,
                       (int)KC, (int)D1, (int)NO, out);
    return hipGetLastError();
}

template <typename TIn>
hipError_t gen_forward(const Plan &p, const TIn *hh, const TIn *hs2, const float *WA,
                       const float *WB, const float *WC, float a_shift, const CtxOut &ctx,
                       float *ab, float *cv, hipStream_t st)
{
    hipError_t e = proj<TIn>(hh, WA, WB, p.B * p.K, p.SH2, p.D, 2 * p.D, ab, st);
    if (e == hipSuccess) e = proj<TIn>(hs2, WC, nullptr, p.B, p.SH2, p.D, p.D, cv, st);
    if (e != hipSuccess) return e;
    const int64_t n = p.B * p.D;
    const int64_t blocks = (n + kGenThreads - 1) / kGenThreads;
    hipLaunchKernelGGL(gscan_gen_fwd_scan_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)),
                       dim3(kGenThreads), 0, st, ab, cv, p.B, p.K, (int)p.D, a_shift, ctx);
    return hipGetLastError();
}

template <typename TIn>
hipError_t gen_partials(const Plan &p, const TIn *hh, const TIn *hs2, const float *WA,
                        const float *WB, const float *WC, float a_shift, const float *dctx,
                        float *part, float *ab, float *cv, hipStream_t st)
{
    // replayed projections, then the exact adjoints in place
    hipError_t e = proj<TIn>(hh, WA, WB, p.B * p.K, p.SH2, p.D, 2 * p.D, ab, st);
    if (e == hipSuccess) e = proj<TIn>(hs2, WC, nullptr, p.B, p.SH2, p.D, p.D, cv, st);
    if (e == hipSuccess) e = launch_adjoint(p, ab, cv, dctx, a_shift, st);
    if (e != hipSuccess) return e;
    const int64_t slabs = p.gen_slabs;
    const int64_t rows = p.B * p.K;
    const int64_t rps = ((rows + slabs - 1) / slabs + kGenK - 1) / kGenK * kGenK;
    const int64_t rpsc = ((p.B + slabs - 1) / slabs + kGenK - 1) / kGenK * kGenK;
    const unsigned gi = (unsigned)((p.SH2 + kGenTile - 1) / kGenTile);
    hipLaunchKernelGGL((gscan_gen_contract_kernel<TIn>),
                       dim3((unsigned)slabs, gi, (unsigned)((2 * p.D + kGenTile - 1) / kGenTile)),
                       dim3(kGenThreads), 0, st, hh, (const float *)ab, rows, rps, (int)p.SH2,
                       (int)(2 * p.D), (int)p.D, 0, part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((gscan_gen_contract_kernel<TIn>),
                       dim3((unsigned)slabs, gi, (unsigned)((p.D + kGenTile - 1) / kGenTile)),
                       dim3(kGenThreads), 0, st, hs2, (const float *)cv, p.B, rpsc, (int)p.SH2,
                       (int)p.D, (int)p.D, 2, part);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gen_forward(const Plan &p, const void *hh, const void *hs2, const float *WA,
                              const float *WB, const float *WC, float a_shift, const CtxOut &ctx,
                              float *ab, float *cv, hipStream_t st)
{
    if (p.dtype == 1)
        return gen_forward<uint16_t>(p, static_cast<const uint16_t *>(hh),
                                     static_cast<const uint16_t *>(hs2), WA, WB, WC, a_shift, ctx,
                                     ab, cv, st);
    return gen_forward<float>(p, static_cast<const float *>(hh), static_cast<const float *>(hs2),
                              WA, WB, WC, a_shift, ctx, ab, cv, st);
}

hipError_t launch_gen_partials(const Plan &p, const void *hh, const void *hs2, const float *WA,
                               const float *WB, const float *WC, float a_shift,
                               const float *dctx, float *part, float *ab, float *cv,
                               hipStream_t st)
{
    if (p.dtype == 1)
        return gen_partials<uint16_t>(p, static_cast<const uint16_t *>(hh),
                                      static_cast<const uint16_t *>(hs2), WA, WB, WC, a_shift,
                                      dctx, part, ab, cv, st);
    return gen_partials<float>(p, static_cast<const float *>(hh), static_cast<const float *>(hs2),
                               WA, WB, WC, a_shift, dctx, part, ab, cv, st);
}

}  // namespace gscan
