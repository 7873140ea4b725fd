// Gated temporal scan, forward and backward, for gfx950 (MI355X).
//
// Operation: foxhunt design spec "Custom Kernel Optimization - cuBLAS
// Projections + Batch-Parallel Scans", Design 1 "Mamba2 Scan":
//   Forward Step 1  A = h_history @ W_A (+a_shift), Bv = h_history @ W_B,
//                   C = h_s2 @ W_C
//   Forward Step 2  x <- sigmoid(A_t) * x + Bv_t for t = 0..K-1 from x = 0;
//                   context = C * x_K
//   Backward Steps 1-3  replay, reverse scan, and the weight gradients
//                   dW_A = h^T @ dL/dA, dW_B = h^T @ dL/dBv, dW_C = h_s2^T @ dL/dC.
//
// The page's design materialises A/Bv/C and the gate gradients in HBM
// between six library GEMMs and two scan kernels.  Here one kernel per pass
// streams h_history once: the projections are MFMA tiles whose results
// never leave registers, the scan runs on the MFMA output layout, and the
// backward contracts the gradients on chip into per-workgroup partials that
// a second small kernel sums in a fixed order (no floating-point atomics).
//
// Work decomposition
//   workgroup = 4 wavefronts = one "group" of 16 samples x one 16-state slice
//   of D.  The weight slice [SH2 x (16 A | 16 B | 16 C)] is staged in LDS in
//   MFMA operand order.  MFMA v_mfma_f32_16x16x4_f32: for a 16-row block of
//   h_history, lane l holds row (l % 16) and eight consecutive columns
//   32q + 8(l/16) + e of every 32-column unit q; the contraction order over
//   SH2 is a permutation applied identically to h and W, so 16-byte loads
//   feed the A operand directly.  The 16x16 result gives lane l the state
//   s = l % 16 for rows 4(l/16) + j, j = 0..3.
//
// Scan on that layout: every row is an affine map of the state,
//   x -> g*x + b          (t > 0)
//   x -> b   (a reset)    (t = 0, since x_0 = 0),
// composed exactly with an explicit reset flag so a non-finite value never
// leaks from one sample into the next.  Lanes compose their four rows,
// lane groups (l/16) combine with two shuffle steps, wavefronts through LDS.
// The backward runs the same construction on the reverse adjoint
//   mu_{r-1} = g_r * mu_r (t_r > 0),   mu_{r-1} = lambda_K(previous sample) (t_r = 0).
#include <cstdint>

#include "gscan_internal.h"

namespace gscan {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma(float a, float b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f4 zero4()
{
    f4 z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

// ---------------------------------------------------------------- input loads
template <typename T> struct In;

template <> struct In<float> {
    // eight consecutive columns starting at p (16-byte aligned)
    static __device__ __forceinline__ void load8(const float *p, float (&v)[8])
    {
        const f4 a = *reinterpret_cast<const f4 *>(p);
        const f4 b = *reinterpret_cast<const f4 *>(p + 4);
        v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
        v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
    }
    static __device__ __forceinline__ f4 load4(const float *p)
    {
        return *reinterpret_cast<const f4 *>(p);
    }
};

// bfloat16 storage: widening is exact (the value's bits are the top half of a float)
template <> struct In<uint16_t> {
    static __device__ __forceinline__ float lo(uint32_t u) { return __uint_as_float(u << 16); }
    static __device__ __forceinline__ float hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
    static __device__ __forceinline__ void load8(const uint16_t *p, float (&v)[8])
    {
        const uint4 u = *reinterpret_cast<const uint4 *>(p);
        v[0] = lo(u.x); v[1] = hi(u.x); v[2] = lo(u.y); v[3] = hi(u.y);
        v[4] = lo(u.z); v[5] = hi(u.z); v[6] = lo(u.w); v[7] = hi(u.w);
    }
    static __device__ __forceinline__ f4 load4(const uint16_t *p)
    {
        const uint2 u = *reinterpret_cast<const uint2 *>(p);
        f4 r;
        r[0] = lo(u.x); r[1] = hi(u.x); r[2] = lo(u.y); r[3] = hi(u.y);
        return r;
    }
};

// ------------------------------------------------------------ affine state maps
// x -> r ? c : m*x + c
struct Aff {
    float m, c;
    int r;
};

__device__ __forceinline__ Aff aff_id()
{
    Aff a = {1.f, 0.f, 0};
    return a;
}

// apply `earlier` first, then `later`
__device__ __forceinline__ Aff compose(const Aff &later, const Aff &earlier)
{
    Aff o;
    o.r = later.r | earlier.r;
    o.m = later.r ? later.m : later.m * earlier.m;
    o.c = later.r ? later.c : later.m * earlier.c + later.c;
    return o;
}

__device__ __forceinline__ float apply(const Aff &a, float x)
{
    return a.r ? a.c : a.m * x + a.c;
}

__device__ __forceinline__ Aff shfl_aff(const Aff &a, int src)
{
    Aff o;
    o.m = __shfl(a.m, src);
    o.c = __shfl(a.c, src);
    o.r = __shfl(a.r, src);
    return o;
}

// Prefix over the four lane groups g = lane/16 (ascending): returns the
// composite of groups < g (exclusive) and of all four groups (total).
__device__ __forceinline__ void scan_up(const Aff &mine, int lane, Aff &excl, Aff &total)
{
    const int kg = lane >> 4;
    Aff p = shfl_aff(mine, lane - 16 < 0 ? lane : lane - 16);
    if (kg < 1) p = aff_id();
    const Aff s1 = compose(mine, p);
    Aff q = shfl_aff(s1, lane - 32 < 0 ? lane : lane - 32);
    if (kg < 2) q = aff_id();
    const Aff s2 = compose(s1, q);  // inclusive prefix
    Aff e = shfl_aff(s2, lane - 16 < 0 ? lane : lane - 16);
    if (kg < 1) e = aff_id();
    excl = e;
    total = shfl_aff(s2, 48 + (lane & 15));
}

// Suffix over the lane groups (descending: group 3 applied first).
__device__ __forceinline__ void scan_down(const Aff &mine, int lane, Aff &excl, Aff &total)
{
    const int kg = lane >> 4;
    Aff p = shfl_aff(mine, lane + 16 > 63 ? lane : lane + 16);
    if (kg > 2) p = aff_id();
    const Aff s1 = compose(mine, p);
    Aff q = shfl_aff(s1, lane + 32 > 63 ? lane : lane + 32);
    if (kg > 1) q = aff_id();
    const Aff s2 = compose(s1, q);  // inclusive suffix
    Aff e = shfl_aff(s2, lane + 16 > 63 ? lane : lane + 16);
    if (kg > 2) e = aff_id();
    excl = e;
    total = shfl_aff(s2, lane & 15);
}

__device__ __forceinline__ float sigmoid(float a)
{
    return __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// --------------------------------------------------------------- weight slice
// LDS image of [W_A | W_B | W_C][:, s0 .. s0+16) in MFMA B-operand order:
// entry ((q*3 + w)*2 + half)*64 + lane holds, for state s0 + lane%16,
// the four rows 32q + 8(lane/16) + 4*half + {0..3} of weight w.
template <int NQ>
__device__ __forceinline__ void stage_weights(f4 *Wl, const float *__restrict__ WA,
                                              const float *__restrict__ WB,
                                              const float *__restrict__ WC, int D, int s0)
{
    for (int idx = threadIdx.x; idx < NQ * 3 * 2 * kWave; idx += kThreads) {
        const int ln = idx & 63;
        int rest = idx >> 6;
        const int half = rest & 1;
        rest >>= 1;
        const int w = rest % 3;
        const int q = rest / 3;
        const int k0 = 32 * q + 8 * (ln >> 4) + 4 * half;
        const int s = s0 + (ln & 15);
        const float *W = w == 0 ? WA : (w == 1 ? WB : WC);
        f4 v;
        v[0] = W[(k0 + 0) * D + s];
        v[1] = W[(k0 + 1) * D + s];
        v[2] = W[(k0 + 2) * D + s];
        v[3] = W[(k0 + 3) * D + s];
        Wl[idx] = v;
    }
}

__device__ __forceinline__ const f4 &wop(const f4 *Wl, int q, int w, int half, int lane)
{
    return Wl[((q * 3 + w) * 2 + half) * kWave + lane];
}

// A|Bv projection of one 16-row block: `rowp` is this lane's row (row l%16).
template <typename TIn, int NQ>
__device__ __forceinline__ void project_block(const TIn *__restrict__ rowp, const f4 *Wl, int lane,
                                              f4 &aA, f4 &aB)
{
    const int kg = lane >> 4;
    float hv[NQ][8];
#pragma unroll
    for (int q = 0; q < NQ; ++q) In<TIn>::load8(rowp + 32 * q + 8 * kg, hv[q]);
    aA = zero4();
    aB = zero4();
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const f4 wa = wop(Wl, q, 0, half, lane);
            const f4 wb = wop(Wl, q, 1, half, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                aA = mfma(hv[q][4 * half + e], wa[e], aA);
                aB = mfma(hv[q][4 * half + e], wb[e], aB);
            }
        }
    }
}

// C projection partial over the 32-column units q = wave, wave+4, ... for the
// group's 16 samples (row l%16 = sample).
template <typename TIn, int NQ>
__device__ __forceinline__ f4 project_c_partial(const TIn *__restrict__ rowp, const f4 *Wl,
                                                int lane, int wave)
{
    const int kg = lane >> 4;
    f4 acc = zero4();
    for (int q = wave; q < NQ; q += kWaves) {
        float hv[8];
        In<TIn>::load8(rowp + 32 * q + 8 * kg, hv);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const f4 wc = wop(Wl, q, 2, half, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = mfma(hv[4 * half + e], wc[e], acc);
        }
    }
    return acc;
}

__device__ __forceinline__ void decode_block(int slices, int64_t &g, int &slice)
{
    const int64_t id = blockIdx.x;
    const int xcd = (int)(id % kXcds);
    const int64_t rest = id / kXcds;
    slice = (int)(rest % slices);
    g = (rest / slices) * kXcds + xcd;
}

// ============================================================== forward kernel
// Each wavefront owns four samples of the group and walks their rows in
// 16-row blocks, carrying the state across blocks.
template <typename TIn, int NQ>
__global__ void __launch_bounds__(kThreads)
gscan_fwd_kernel(const TIn *__restrict__ hh, const TIn *__restrict__ hs2,
                 const float *__restrict__ WA, const float *__restrict__ WB,
                 const float *__restrict__ WC, int64_t B, int K, int D, int slices,
                 int64_t groups, float a_shift, float *__restrict__ ctx)
{
    constexpr int SH2 = NQ * 32;
    __shared__ f4 Wl[NQ * 6 * kWave];
    __shared__ float cvp[kWaves][16][16];

    int64_t g;
    int slice;
    decode_block(slices, g, slice);
    if (g >= groups) return;
    const int s0 = slice * kSlice;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kg = lane >> 4, ln = lane & 15;

    stage_weights<NQ>(Wl, WA, WB, WC, D, s0);
    __syncthreads();

    const int64_t b0 = g * kGroupSamples;
    const int nb = (int)(B - b0 < kGroupSamples ? B - b0 : kGroupSamples);
    {
        const int sl = ln < nb ? ln : nb - 1;
        const f4 cp = project_c_partial<TIn, NQ>(hs2 + (b0 + sl) * SH2, Wl, lane, wave);
#pragma unroll
        for (int j = 0; j < 4; ++j) cvp[wave][4 * kg + j][ln] = cp[j];
    }
    __syncthreads();

    const int lr_begin = 4 * wave * K;
    const int lr_end = (4 * wave + 4 < nb ? 4 * wave + 4 : nb) * K;
    if (lr_begin >= lr_end) return;
    const int64_t R0 = b0 * K;
    float xc = 0.f;
    for (int lr0 = lr_begin; lr0 < lr_end; lr0 += kBlockRows) {
        const int myr = lr0 + ln < lr_end ? lr0 + ln : lr_end - 1;
        f4 aA, aB;
        project_block<TIn, NQ>(hh + (R0 + myr) * SH2, Wl, lane, aA, aB);

        Aff map[4];
        Aff F = aff_id();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = lr0 + 4 * kg + j;
            const int t = r % K;
            Aff m;
            if (r >= lr_end) {
                m = aff_id();
            } else {
                m.m = sigmoid(aA[j] + a_shift);
                m.c = aB[j];
                m.r = t == 0;
            }
            map[j] = m;
            F = compose(m, F);
        }
        Aff excl, total;
        scan_up(F, lane, excl, total);
        float x = apply(excl, xc);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x = apply(map[j], x);
            const int r = lr0 + 4 * kg + j;
            if (r < lr_end && r % K == K - 1) {
                const int bl = r / K;
                const float cv = cvp[0][bl][ln] + cvp[1][bl][ln] + cvp[2][bl][ln] + cvp[3][bl][ln];
                ctx[(b0 + bl) * D + s0 + ln] = cv * x;
            }
        }
        xc = apply(total, xc);
    }
}

// ============================================================= backward kernel
// Persistent over groups.  Rows of a group are processed in 64-row chunks,
// wavefront w projecting block w of the chunk.  After the forward and
// reverse scans (wavefronts combined through LDS), dL/dA and dL/dBv of the
// chunk go to LDS and every wavefront contracts all 64 rows against its own
// 64-column superblocks of SH2 (the "i split"), so each wavefront keeps only
// SH2/8 gradient accumulators.
//
// A sample that continues past the chunk end (K not dividing the chunk)
// needs the gates of later chunks.  Its rows' adjoints are computed with the
// future gates set to 1 and summed into an "open" accumulator; when the next
// chunk's gates of that sample are known the open accumulator is scaled by
// their product (per state) and the new rows are added (Horner's scheme),
// and once the sample ends the open accumulator is folded into the closed one.
// 64-column superblocks of SH2, and how many of them one wavefront owns
constexpr int nsb_of(int nq) { return nq * 32 / 64; }
constexpr int sbw_of(int nq) { return (nsb_of(nq) + kWaves - 1) / kWaves; }

// acc{A,B}[sbi][c] += sum over chunk rows r in [lo, hi) of h[r, i] (x) d{A,B}[r, s]
// for i = 64*ib + 4*(4*(l/16) + jj) + c  (ib = wave + 4*sbi), s = l%16.
template <typename TIn, int NQ>
__device__ __forceinline__ void contract_rows(
    f4 (&accA)[sbw_of(NQ)][4], f4 (&accB)[sbw_of(NQ)][4],
    const TIn *__restrict__ hh, int64_t R0, int cb, int NR, int lo, int hi,
    const f4 (*dab)[2][kWave], int wave, int lane)
{
    constexpr int SH2 = NQ * 32;
    constexpr int NSB = nsb_of(NQ);
    constexpr int SBW = sbw_of(NQ);
    const int kg = lane >> 4, ln = lane & 15;
#pragma unroll
    for (int sbi = 0; sbi < SBW; ++sbi) {
        const int ib = wave + kWaves * sbi;
        if (ib >= NSB) break;
#pragma unroll
        for (int wb = 0; wb < kWaves; ++wb) {
            const f4 dA4 = dab[wb][0][lane];
            const f4 dB4 = dab[wb][1][lane];
            f4 hv[4];
#pragma unroll
            for (int jp = 0; jp < 4; ++jp) {
                const int r = cb + kBlockRows * wb + 4 * kg + jp;
                const int rc = r < NR ? r : NR - 1;
                hv[jp] = In<TIn>::load4(hh + (R0 + rc) * SH2 + 64 * ib + 4 * ln);
            }
#pragma unroll
            for (int jp = 0; jp < 4; ++jp) {
                const int r = cb + kBlockRows * wb + 4 * kg + jp;
                const bool in = r >= lo && r < hi;
                const float da = in ? dA4[jp] : 0.f;
                const float db = in ? dB4[jp] : 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    accA[sbi][c] = mfma(hv[jp][c], da, accA[sbi][c]);
                    accB[sbi][c] = mfma(hv[jp][c], db, accB[sbi][c]);
                }
            }
        }
    }
}

template <typename TIn, int NQ>
__global__ void __launch_bounds__(kThreads)
gscan_bwd_kernel(const TIn *__restrict__ hh, const TIn *__restrict__ hs2,
                 const float *__restrict__ WA, const float *__restrict__ WB,
                 const float *__restrict__ WC, int64_t B, int K, int D, int slices,
                 int64_t groups, int64_t nrows, float a_shift, const float *__restrict__ dctx,
                 float *__restrict__ part)
{
    constexpr int SH2 = NQ * 32;
    constexpr int NSB = nsb_of(NQ);
    constexpr int SBW = sbw_of(NQ);
    __shared__ f4 Wl[NQ * 6 * kWave];
    __shared__ float cvp[kWaves][16][16];
    __shared__ float lamK[16][16];   // d_context * C  (dL/dx_K)
    __shared__ float dctl[16][16];   // d_context slice
    __shared__ float dCl[16][16];    // dL/dC = d_context * x_K
    __shared__ float fsum[2][kWaves][3][16];
    __shared__ float rsum[2][kWaves][3][16];
    __shared__ f4 dab[2][kWaves][2][kWave];
    __shared__ float gprev[2][16];

    int64_t rho;
    int slice;
    decode_block(slices, rho, slice);
    const int s0 = slice * kSlice;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int kg = lane >> 4, ln = lane & 15;

    f4 accAc[SBW][4], accAo[SBW][4], accBc[SBW][4], accBo[SBW][4], accC[SBW][4];
#pragma unroll
    for (int i = 0; i < SBW; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            accAc[i][c] = zero4();
            accAo[i][c] = zero4();
            accBc[i][c] = zero4();
            accBo[i][c] = zero4();
            accC[i][c] = zero4();
        }

    stage_weights<NQ>(Wl, WA, WB, WC, D, s0);

    for (int64_t g = rho; g < groups; g += nrows) {
        __syncthreads();  // weights staged / previous group's LDS reads done
        const int64_t b0 = g * kGroupSamples;
        const int nb = (int)(B - b0 < kGroupSamples ? B - b0 : kGroupSamples);
        {
            const int sl = ln < nb ? ln : nb - 1;
            const f4 cp = project_c_partial<TIn, NQ>(hs2 + (b0 + sl) * SH2, Wl, lane, wave);
#pragma unroll
            for (int j = 0; j < 4; ++j) cvp[wave][4 * kg + j][ln] = cp[j];
        }
        __syncthreads();
        {
            const int bl = tid >> 4, s = tid & 15;
            const float cv = cvp[0][bl][s] + cvp[1][bl][s] + cvp[2][bl][s] + cvp[3][bl][s];
            const float d = bl < nb ? dctx[(b0 + bl) * D + s0 + s] : 0.f;
            dctl[bl][s] = d;
            lamK[bl][s] = d * cv;
        }
        __syncthreads();

        const int64_t R0 = b0 * K;
        const int NR = nb * K;
        const int nch = (NR + kChunkRows - 1) / kChunkRows;
        float xc = 0.f;
        for (int c = 0; c < nch; ++c) {
            const int buf = c & 1;
            const int cb = c * kChunkRows;
            const int ce = cb + kChunkRows < NR ? cb + kChunkRows : NR;
            const int lr0 = cb + kBlockRows * wave;
            const int myr = lr0 + ln < NR ? lr0 + ln : NR - 1;
            f4 aA, aB;
            project_block<TIn, NQ>(hh + (R0 + myr) * SH2, Wl, lane, aA, aB);

            // per-row maps (forward state and reverse adjoint)
            Aff fm[4], rm[4];
            float gate[4];
            Aff F = aff_id();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = lr0 + 4 * kg + j;
                const int bl = r / K;
                const int t = r - bl * K;
                const float gt = sigmoid(aA[j] + a_shift);
                gate[j] = gt;
                if (r >= ce) {
                    fm[j] = aff_id();
                    rm[j] = aff_id();
                } else {
                    fm[j].m = gt;
                    fm[j].c = aB[j];
                    fm[j].r = t == 0;
                    rm[j].m = gt;
                    rm[j].c = (t == 0 && bl > 0) ? lamK[bl - 1][ln] : 0.f;
                    rm[j].r = t == 0;
                }
                F = compose(fm[j], F);
            }
            Aff R = aff_id();
#pragma unroll
            for (int j = 3; j >= 0; --j) R = compose(rm[j], R);
            Aff Fx, Ft, Rx, Rt;
            scan_up(F, lane, Fx, Ft);
            scan_down(R, lane, Rx, Rt);
            if (kg == 0) {
                fsum[buf][wave][0][ln] = Ft.m;
                fsum[buf][wave][1][ln] = Ft.c;
                fsum[buf][wave][2][ln] = (float)Ft.r;
                rsum[buf][wave][0][ln] = Rt.m;
                rsum[buf][wave][1][ln] = Rt.c;
                rsum[buf][wave][2][ln] = (float)Rt.r;
            }
            __syncthreads();

            // carries across wavefronts
            float xin = xc, xnext = xc, gpre = 1.f, gall = 1.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                Aff a;
                a.m = fsum[buf][w][0][ln];
                a.c = fsum[buf][w][1][ln];
                a.r = fsum[buf][w][2][ln] != 0.f;
                if (w < wave) {
                    xin = apply(a, xin);
                    gpre *= a.m;
                }
                xnext = apply(a, xnext);
                gall *= a.m;
            }
            const int bl_top = (ce - 1) / K;
            float mu = lamK[bl_top][ln];
#pragma unroll
            for (int w = kWaves - 1; w >= 0; --w) {
                if (w > wave) {
                    Aff a;
                    a.m = rsum[buf][w][0][ln];
                    a.c = rsum[buf][w][1][ln];
                    a.r = rsum[buf][w][2][ln] != 0.f;
                    mu = apply(a, mu);
                }
            }

            // the sample open at the chunk start (if any) and where it ends
            const bool has_prev = (cb % K) != 0;
            const int prev_end = (cb / K + 1) * K - 1;  // its last local row

            // forward walk: state before each row, dL/dC at sample ends,
            // gate product of the open sample
            float x = apply(Fx, xin);
            float grun = Fx.m * gpre;
            float xbef[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = lr0 + 4 * kg + j;
                const int bl = r / K;
                const int t = r - bl * K;
                xbef[j] = t == 0 ? 0.f : x;
                x = apply(fm[j], x);
                grun *= fm[j].m;
                if (r < ce && t == K - 1) dCl[bl][ln] = dctl[bl][ln] * x;
                if (has_prev && r == prev_end) gprev[buf][ln] = grun;
            }
            // reverse walk: adjoint of each row's output state
            float m_in = apply(Rx, mu);
            f4 dA4, dB4;
#pragma unroll
            for (int j = 3; j >= 0; --j) {
                const int r = lr0 + 4 * kg + j;
                const bool v = r < ce;
                const float gt = gate[j];
                dB4[j] = v ? m_in : 0.f;
                dA4[j] = v ? m_in * xbef[j] * (gt * (1.f - gt)) : 0.f;
                m_in = apply(rm[j], m_in);
            }
            dab[buf][wave][0][lane] = dA4;
            dab[buf][wave][1][lane] = dB4;
            __syncthreads();

            // weight-gradient contraction of the chunk
            const bool top_open = (bl_top + 1) * K > ce;
            const int rN = top_open ? bl_top * K : ce;  // rows >= rN continue past the chunk
            if (!has_prev && !top_open) {
                contract_rows<TIn, NQ>(accAc, accBc, hh, R0, cb, NR, cb, ce, dab[buf], wave, lane);
            } else {
                if (has_prev) {
                    const float gs = prev_end < ce ? gprev[buf][ln] : gall;
#pragma unroll
                    for (int i = 0; i < SBW; ++i)
#pragma unroll
                        for (int cc = 0; cc < 4; ++cc) {
                            accAo[i][cc] *= gs;
                            accBo[i][cc] *= gs;
                        }
                }
                if (rN > cb) {
                    contract_rows<TIn, NQ>(accAo, accBo, hh, R0, cb, NR, cb, rN, dab[buf], wave,
                                           lane);
#pragma unroll
                    for (int i = 0; i < SBW; ++i)
#pragma unroll
                        for (int cc = 0; cc < 4; ++cc) {
                            accAc[i][cc] += accAo[i][cc];
                            accBc[i][cc] += accBo[i][cc];
                            accAo[i][cc] = zero4();
                            accBo[i][cc] = zero4();
                        }
                }
                if (rN < ce)
                    contract_rows<TIn, NQ>(accAo, accBo, hh, R0, cb, NR, rN, ce, dab[buf], wave,
                                           lane);
            }
            xc = xnext;
        }

        // dW_C rows of this group: h_s2^T @ dL/dC (dCl complete after the last barrier)
#pragma unroll
        for (int sbi = 0; sbi < SBW; ++sbi) {
            const int ib = wave + kWaves * sbi;
            if (ib >= NSB) break;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int bl = 4 * a + kg;
                const int blc = bl < nb ? bl : nb - 1;
                const f4 hv = In<TIn>::load4(hs2 + (b0 + blc) * SH2 + 64 * ib + 4 * ln);
                const float dc = bl < nb ? dCl[bl][ln] : 0.f;
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) accC[sbi][cc] = mfma(hv[cc], dc, accC[sbi][cc]);
            }
        }
    }

    // this workgroup's partial: part[rho][which][i][s]
    float *P = part + rho * 3 * (int64_t)SH2 * D;
#pragma unroll
    for (int sbi = 0; sbi < SBW; ++sbi) {
        const int ib = wave + kWaves * sbi;
        if (ib >= NSB) break;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int i = 64 * ib + 4 * (4 * kg + jj) + cc;
                const int64_t o = (int64_t)i * D + s0 + ln;
                P[o] = accAc[sbi][cc][jj];
                P[(int64_t)SH2 * D + o] = accBc[sbi][cc][jj];
                P[2 * (int64_t)SH2 * D + o] = accC[sbi][cc][jj];
            }
    }
}

// ================================================= phase 2: partial reduction
// out[o] = sum over rho (fixed order: four interleaved lanes of partials,
// then their sum) of part[rho][o], o over the 3*SH2*D gradient entries.
__global__ void __launch_bounds__(kThreads)
gscan_reduce_kernel(const float *__restrict__ part, int64_t nrows, int64_t wsz,
                    float *__restrict__ dWA, float *__restrict__ dWB, float *__restrict__ dWC)
{
    __shared__ double red[4][64];
    const int t = threadIdx.x;
    const int seg = t >> 6;
    const int64_t o = (int64_t)blockIdx.x * 64 + (t & 63);
    const int64_t per = 3 * wsz;
    double s = 0.0;
    if (o < per)
        for (int64_t r = seg; r < nrows; r += 4) s += (double)part[r * per + o];
    red[seg][t & 63] = s;
    __syncthreads();
    if (seg == 0 && o < per) {
        const double v = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
        const int64_t which = o / wsz, e = o - which * wsz;
        float *out = which == 0 ? dWA : (which == 1 ? dWB : dWC);
        out[e] = (float)v;
    }
}

// ----------------------------------------------------------------- dispatch
template <typename TIn, int NQ>
hipError_t fwd_launch(const Plan &p, const void *hh, const void *hs2, const float *WA,
                      const float *WB, const float *WC, float a_shift, float *ctx,
                      hipStream_t st)
{
    hipLaunchKernelGGL((gscan_fwd_kernel<TIn, NQ>), dim3((unsigned)p.fwd_grid), dim3(kThreads), 0,
                       st, static_cast<const TIn *>(hh), static_cast<const TIn *>(hs2), WA, WB,
                       WC, p.B, (int)p.K, (int)p.D, p.slices, p.groups, a_shift, ctx);
    return hipGetLastError();
}

template <typename TIn, int NQ>
hipError_t bwd_launch(const Plan &p, const void *hh, const void *hs2, const float *WA,
                      const float *WB, const float *WC, float a_shift, const float *dctx,
                      float *part, hipStream_t st)
{
    hipLaunchKernelGGL((gscan_bwd_kernel<TIn, NQ>), dim3((unsigned)p.bwd_grid), dim3(kThreads), 0,
                       st, static_cast<const TIn *>(hh), static_cast<const TIn *>(hs2), WA, WB,
                       WC, p.B, (int)p.K, (int)p.D, p.slices, p.groups, p.bwd_rows, a_shift,
                       dctx, part);
    return hipGetLastError();
}

template <typename TIn>
hipError_t fwd_by_nq(const Plan &p, const void *hh, const void *hs2, const float *WA,
                     const float *WB, const float *WC, float a, float *ctx, hipStream_t st)
{
    switch (p.nq) {
    case 2: return fwd_launch<TIn, 2>(p, hh, hs2, WA, WB, WC, a, ctx, st);
    case 4: return fwd_launch<TIn, 4>(p, hh, hs2, WA, WB, WC, a, ctx, st);
    case 6: return fwd_launch<TIn, 6>(p, hh, hs2, WA, WB, WC, a, ctx, st);
    case 8: return fwd_launch<TIn, 8>(p, hh, hs2, WA, WB, WC, a, ctx, st);
    case 10: return fwd_launch<TIn, 10>(p, hh, hs2, WA, WB, WC, a, ctx, st);
    case 12: return fwd_launch<TIn, 12>(p, hh, hs2, WA, WB, WC, a, ctx, st);
    case 14: return fwd_launch<TIn, 14>(p, hh, hs2, WA, WB, WC, a, ctx, st);
    case 16: return fwd_launch<TIn, 16>(p, hh, hs2, WA, WB, WC, a, ctx, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename TIn>
hipError_t bwd_by_nq(const Plan &p, const void *hh, const void *hs2, const float *WA,
                     const float *WB, const float *WC, float a, const float *dctx, float *part,
                     hipStream_t st)
{
    switch (p.nq) {
    case 2: return bwd_launch<TIn, 2>(p, hh, hs2, WA, WB, WC, a, dctx, part, st);
    case 4: return bwd_launch<TIn, 4>(p, hh, hs2, WA, WB, WC, a, dctx, part, st);
    case 6: return bwd_launch<TIn, 6>(p, hh, hs2, WA, WB, WC, a, dctx, part, st);
    case 8: return bwd_launch<TIn, 8>(p, hh, hs2, WA, WB, WC, a, dctx, part, st);
    case 10: return bwd_launch<TIn, 10>(p, hh, hs2, WA, WB, WC, a, dctx, part, st);
    case 12: return bwd_launch<TIn, 12>(p, hh, hs2, WA, WB, WC, a, dctx, part, st);
    case 14: return bwd_launch<TIn, 14>(p, hh, hs2, WA, WB, WC, a, dctx, part, st);
    case 16: return bwd_launch<TIn, 16>(p, hh, hs2, WA, WB, WC, a, dctx, part, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool make_plan(int64_t B, int64_t K, int64_t SH2, int64_t D, int dtype, Plan *p)
{
    if (B < 1 || K < 1 || SH2 < 64 || SH2 > kMaxSH2 || SH2 % 64 != 0 || D < kSlice ||
        D > kMaxD || D % kSlice != 0 || (dtype != 0 && dtype != 1))
        return false;
    // local row indices (16 samples x K) and global row counts stay in range
    if (K > (int64_t(1) << 26) || B > (int64_t(1) << 40) || B * K > (int64_t(1) << 46))
        return false;
    Plan q;
    q.B = B;
    q.K = K;
    q.SH2 = SH2;
    q.D = D;
    q.dtype = dtype;
    q.nq = (int)(SH2 / 32);
    q.slices = (int)(D / kSlice);
    q.groups = (B + kGroupSamples - 1) / kGroupSamples;
    q.fwd_rows = (q.groups + kXcds - 1) / kXcds * kXcds;
    q.fwd_grid = q.fwd_rows * q.slices;
    // backward: about two resident workgroups per CU when the weight slice
    // leaves room for two in LDS, one otherwise (256 CUs)
    const int64_t target = q.nq <= 8 ? 512 : 256;
    int64_t cap = target / q.slices / kXcds * kXcds;
    if (cap < kXcds) cap = kXcds;
    q.bwd_rows = q.fwd_rows < cap ? q.fwd_rows : cap;
    q.bwd_grid = q.bwd_rows * q.slices;
    const int64_t wsz = SH2 * D;
    q.red_grid = (3 * wsz + 63) / 64;
    q.ws_bytes = (size_t)(q.bwd_rows * 3 * wsz * 4);
    if (q.fwd_grid > 0x7fffffff || q.bwd_grid > 0x7fffffff) return false;
    *p = q;
    return true;
}

hipError_t launch_forward(const Plan &p, const void *hh, const void *hs2, const float *WA,
                          const float *WB, const float *WC, float a_shift, float *ctx,
                          hipStream_t st)
{
    if (p.dtype == 1) return fwd_by_nq<uint16_t>(p, hh, hs2, WA, WB, WC, a_shift, ctx, st);
    return fwd_by_nq<float>(p, hh, hs2, WA, WB, WC, a_shift, ctx, st);
}

hipError_t launch_backward_partials(const Plan &p, const void *hh, const void *hs2,
                                    const float *WA, const float *WB, const float *WC,
                                    float a_shift, const float *dctx, float *part, hipStream_t st)
{
    return p.dtype == 1 ? bwd_by_nq<uint16_t>(p, hh, hs2, WA, WB, WC, a_shift, dctx, part, st)
                        : bwd_by_nq<float>(p, hh, hs2, WA, WB, WC, a_shift, dctx, part, st);
}

hipError_t launch_backward_reduce(const Plan &p, const float *part, float *dWA, float *dWB,
                                  float *dWC, hipStream_t st)
{
    hipLaunchKernelGGL(gscan_reduce_kernel, dim3((unsigned)p.red_grid), dim3(kThreads), 0, st,
                       part, p.bwd_rows, p.SH2 * p.D, dWA, dWB, dWC);
    return hipGetLastError();
}

}  // namespace gscan
