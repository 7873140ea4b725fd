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
// Arithmetic.  Products of h with W (projections) and of h with dL/dA, dL/dBv
// (weight gradients) run on bf16 MFMA with a two-term split of each fp32
// operand, x = hi + lo with hi = bf16(x) and lo = bf16(x - hi) (both round to
// nearest even), keeping hi*hi + hi*lo + lo*hi and accumulating in fp32.
// The dropped terms are below 2^-16 of each product.  bf16 inputs are exact
// in hi, so their lo term vanishes and is skipped.  dW_C, the only contraction
// over samples rather than rows, uses the same split products in the
// per-block backward kernel and fp32 MFMA (16x16x4) in the general one.
//
// Work decomposition
//   workgroup = 4 wavefronts = one "group" of 16 samples x one 16-state slice
//   of D.  The weight slice [SH2 x (16 A | 16 B | 16 C)] is split into bf16
//   hi/lo and staged in LDS in MFMA operand order.  For MFMA
//   v_mfma_f32_16x16x32_bf16 on a 16-row block of h_history, lane l holds row
//   l % 16 and the eight consecutive columns 32q + 8(l/16) + e of every
//   32-column unit q; the contraction order over SH2 is a permutation applied
//   identically to h and W, so 16-byte row loads feed the operand directly.
//   The 16x16 result gives lane l the state s = l % 16 for rows 4(l/16) + j.
//
// Scan on that layout: every row is an affine map of the state,
//   x -> g*x + b          (t > 0)
//   x -> b   (a reset)    (t = 0, since x_0 = 0),
// composed exactly with an explicit reset flag so a non-finite value never
// leaks from one sample into the next.  Lanes compose their four rows,
// lane groups (l/16) combine with two shuffle steps, wavefronts through LDS.
// The backward runs the same construction on the reverse adjoint
//   mu_{r-1} = g_r * mu_r (t_r > 0),   mu_{r-1} = lambda_K(previous sample) (t_r = 0).
//
// Kernels in this file (the launch plan, make_plan, picks among them):
//   gscan_fwd_kernel, gscan_fwd_persist_kernel  forward, one group x one slice
//   gscan_fwd_ms_kernel      forward, two groups x S slices sharing each split row
//   gscan_fwd_rows_kernel, gscan_bwd_rows_kernel  the per-block decomposition
//                            (rows_pass: 4 row blocks x 2 column halves, persistent;
//                            K dividing 16, or 32, 64; SH2 <= 256), the backward
//                            optionally with the input gradients
//   gscan_bwd_kernel         the general backward (any K)
//   gscan_bwd_scan_kernel, gscan_fwd_tile_kernel, gscan_bwd_contract_kernel
//                            SH2 = 512 over 256-row tiles: scan pass, tile forward,
//                            contraction over row slabs
//   gscan_reduce_kernel      phase 2: fixed-order sum of the partials
//   gscan_adjoint_kernel     exact adjoints from stored projections
//   gscan_dinput_kernel, gscan_proj_kernel, gscan_proj2_kernel  rows x weights
//                            (rows_by_weights): input-gradient products and the
//                            projections written out for the shapes outside the
//                            fused kernels
//   gscan_gen_contract_kernel  those shapes' weight-gradient contractions
#include <cstdint>
#include <type_traits>

#include "gscan_internal.h"

namespace gscan {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f4 zero4()
{
    f4 z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

__device__ __forceinline__ u4 zero_u4()
{
    u4 z = {0u, 0u, 0u, 0u};
    return z;
}

// fp32 MFMA 16x16x4 (A: lane l -> row l%16, k l/16; B: k l/16, column l%16)
__device__ __forceinline__ f4 mfma_f32(float a, float b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// bf16 MFMA 16x16x32 (A: lane l -> row l%16, k 8(l/16)+e; B: k 8(l/16)+e, column l%16)
__device__ __forceinline__ f4 mfma_bf(u4 a, u4 b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// two floats -> packed bf16 pair (round to nearest even), first in the low half
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// x = hi + lo for eight values (packed eight bf16 per u4)
struct Split {
    u4 hi, lo;
};

// Low halves of a split pair: bf16(a - hi_a), bf16(b - hi_b) for the pair
// h = pack_bf16(a, b).  Each remainder is the bf16 dot product -1 * hi + 0 *
// (the other half) + x: the products are exact and x - hi is representable
// in fp32 (hi is x rounded to 8 significant bits), so the remainder is exact
// whatever the dot product's internal rounding, in one instruction instead
// of unpacking hi and subtracting.  The two selector constants are passed
// in scalar registers: as an inline constant, (-1, 0) is encoded as the
// fp32 -1.0 (0xbf800000), which the hardware reads as (0, -1).
__device__ __forceinline__ uint32_t pack_lo(uint32_t h, float a, float b)
{
    uint32_t m0 = 0x0000bf80u, m1 = 0xbf800000u;
    asm("" : "+s"(m0), "+s"(m1));
    const bf16x2 hv = __builtin_bit_cast(bf16x2, h);
    return pack_bf16(
        __builtin_amdgcn_fdot2_f32_bf16(hv, __builtin_bit_cast(bf16x2, m0), a, false),
        __builtin_amdgcn_fdot2_f32_bf16(hv, __builtin_bit_cast(bf16x2, m1), b, false));
}

__device__ __forceinline__ Split split8(const float (&v)[8])
{
    Split s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s.hi[i] = pack_bf16(v[2 * i], v[2 * i + 1]);
        s.lo[i] = pack_lo(s.hi[i], v[2 * i], v[2 * i + 1]);
    }
    return s;
}

// c += a * b with both operands split; LO_A = false when a is exact in bf16
template <bool LO_A>
__device__ __forceinline__ f4 mfma3(const Split &a, const Split &b, f4 c)
{
    c = mfma_bf(a.hi, b.lo, c);
    if (LO_A) c = mfma_bf(a.lo, b.hi, c);
    return mfma_bf(a.hi, b.hi, c);
}

// ---------------------------------------------------------------- input rows
// Projection ("P") layout of one 16-row block: lane l, unit q -> row l%16,
// columns 32q + 8(l/16) + 0..7.
template <typename T, int NQ> struct PBlk;

template <int NQ> struct PBlk<float, NQ> {
    static constexpr bool kLo = true;
    f4 v[NQ][2];
    __device__ __forceinline__ void load_unit(const float *__restrict__ row, int kg, int q)
    {
        v[q][0] = *reinterpret_cast<const f4 *>(row + 32 * q + 8 * kg);
        v[q][1] = *reinterpret_cast<const f4 *>(row + 32 * q + 8 * kg + 4);
    }
    // unit u of the row into register slot j (a ring of fewer slots than units)
    __device__ __forceinline__ void load_unit_at(const float *__restrict__ row, int kg, int u, int j)
    {
        v[j][0] = *reinterpret_cast<const f4 *>(row + 32 * u + 8 * kg);
        v[j][1] = *reinterpret_cast<const f4 *>(row + 32 * u + 8 * kg + 4);
    }
    __device__ __forceinline__ void load(const float *__restrict__ row, int kg)
    {
#pragma unroll
        for (int q = 0; q < NQ; ++q) load_unit(row, kg, q);
    }
    __device__ __forceinline__ Split op(int q) const
    {
        float x[8] = {v[q][0][0], v[q][0][1], v[q][0][2], v[q][0][3],
                      v[q][1][0], v[q][1][1], v[q][1][2], v[q][1][3]};
        return split8(x);
    }
};

template <int NQ> struct PBlk<uint16_t, NQ> {
    static constexpr bool kLo = false;  // bf16 storage is exact in hi
    u4 v[NQ];
    __device__ __forceinline__ void load_unit(const uint16_t *__restrict__ row, int kg, int q)
    {
        v[q] = *reinterpret_cast<const u4 *>(row + 32 * q + 8 * kg);
    }
    __device__ __forceinline__ void load_unit_at(const uint16_t *__restrict__ row, int kg, int u, int j)
    {
        v[j] = *reinterpret_cast<const u4 *>(row + 32 * u + 8 * kg);
    }
    __device__ __forceinline__ void load(const uint16_t *__restrict__ row, int kg)
    {
#pragma unroll
        for (int q = 0; q < NQ; ++q) load_unit(row, kg, q);
    }
    __device__ __forceinline__ Split op(int q) const
    {
        Split s;
        s.hi = v[q];
        s.lo = zero_u4();
        return s;
    }
};

// four consecutive columns of one row (transposed "T" layout loads), kept
// as stored until used so that a load never waits at its issue point
template <typename T> struct Col4;
template <> struct Col4<float> {
    using raw_t = f4;
    static __device__ __forceinline__ raw_t raw(const float *p) { return *reinterpret_cast<const f4 *>(p); }
    static __device__ __forceinline__ f4 widen(const raw_t &r) { return r; }
};
template <> struct Col4<uint16_t> {
    using raw_t = uint2;
    static __device__ __forceinline__ raw_t raw(const uint16_t *p) { return *reinterpret_cast<const uint2 *>(p); }
    static __device__ __forceinline__ f4 widen(const raw_t &u)
    {
        f4 r;
        r[0] = bf_lo(u.x);
        r[1] = bf_hi(u.x);
        r[2] = bf_lo(u.y);
        r[3] = bf_hi(u.y);
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

// Cross-row exchanges of a wavefront (rows of 16 lanes).  pair_rows gives
// every lane the values of the even and the odd row of its row pair (0-1 or
// 2-3); half_rows gives rows r and r + 2 the value of row r % 2 (.lo) and of
// row 2 + r % 2 (.hi).  Call them with every lane active (never under a
// lane-dependent condition): a lane reads the other row's register.
struct RowVals {
    float lo, hi;
};

__device__ __forceinline__ RowVals pair_rows(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

__device__ __forceinline__ RowVals half_rows(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

struct AffRows {
    Aff lo, hi;
};

__device__ __forceinline__ AffRows pair_aff(const Aff &a)
{
    const RowVals m = pair_rows(a.m), c = pair_rows(a.c), r = pair_rows(__int_as_float(a.r));
    return {{m.lo, c.lo, __float_as_int(r.lo)}, {m.hi, c.hi, __float_as_int(r.hi)}};
}

__device__ __forceinline__ AffRows half_aff(const Aff &a)
{
    const RowVals m = half_rows(a.m), c = half_rows(a.c), r = half_rows(__int_as_float(a.r));
    return {{m.lo, c.lo, __float_as_int(r.lo)}, {m.hi, c.hi, __float_as_int(r.hi)}};
}

// Prefix over the four lane groups (rows) of a wavefront, lower rows first:
// within row pairs, then the second pair after the first pair's total.
// excl: composition of the rows before; total: of all four rows.
__device__ __forceinline__ void scan_up(const Aff &mine, int lane, Aff &excl, Aff &total)
{
    const int kg = lane >> 4;
    const bool odd = kg & 1, second = kg >= 2;
    const AffRows p1 = pair_aff(mine);
    const Aff s1 = odd ? compose(mine, p1.lo) : mine;
    const AffRows t1 = pair_aff(s1);     // .hi: the pair's composition
    const AffRows h1 = half_aff(t1.hi);  // .lo: the first pair's, in rows 2-3
    const Aff s2 = second ? compose(s1, h1.lo) : s1;  // inclusive prefix
    const AffRows p2 = pair_aff(s2);
    const AffRows h2 = half_aff(p2.hi);
    excl = odd ? p2.lo : (second ? h2.lo : aff_id());
    total = second ? p2.hi : h2.hi;
}

// Suffix over the four rows, higher rows first (mirror of scan_up).
__device__ __forceinline__ void scan_down(const Aff &mine, int lane, Aff &excl, Aff &total)
{
    const int kg = lane >> 4;
    const bool odd = kg & 1, first = kg < 2;
    const AffRows p1 = pair_aff(mine);
    const Aff s1 = odd ? mine : compose(mine, p1.hi);
    const AffRows t1 = pair_aff(s1);     // .lo: the pair's composition
    const AffRows h1 = half_aff(t1.lo);  // .hi: the second pair's, in rows 0-1
    const Aff s2 = first ? compose(s1, h1.hi) : s1;  // inclusive suffix
    const AffRows p2 = pair_aff(s2);
    const AffRows h2 = half_aff(p2.lo);
    excl = odd ? (first ? h2.hi : aff_id()) : p2.hi;
    total = first ? p2.lo : h2.lo;
}

__device__ __forceinline__ float sigmoid(float a)
{
    return __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// The gate and its complement 1 - g = sigmoid(-a) from one exponential: with
// e = exp(-a), g = 1/(1+e) and 1 - g = e*g.  The product form serves a > 0,
// where 1 - g would cancel as the gate saturates towards 1 (the logistic
// derivative g(1-g) keeps its relative precision there); for a <= 0,
// g <= 1/2 and 1 - g is exact to rounding, and e*g would be inf*0 once e
// overflows.
struct Gate {
    float g, gc;
};

__device__ __forceinline__ Gate gate_of(float a)
{
    const float e = __expf(-a);
    const float g = __builtin_amdgcn_rcpf(1.0f + e);
    Gate r = {g, a > 0.f ? e * g : 1.0f - g};
    return r;
}

// ------------------------------------------------------------ row bookkeeping
// A lane's four rows in a block are base + 4*(l/16) + j, j = 0..3, with base
// uniform across the wavefront.  (sample, step) = divmod(row, K) is formed
// from divmod(base, K) (one uniform division) and the lane's fixed offsets
// divmod(4*(l/16) + j, K) (computed once), so no per-row division is needed.
struct LaneOff {
    int ob[4], ot[4];
};

__device__ __forceinline__ LaneOff lane_offsets(int kg, int K)
{
    LaneOff o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int v = 4 * kg + j;
        o.ob[j] = v / K;
        o.ot[j] = v - o.ob[j] * K;
    }
    return o;
}

struct RowPos {
    int bl, t;
};

// divmod of a wavefront-uniform value
__device__ __forceinline__ RowPos base_pos(int base, int K)
{
    const int b = __builtin_amdgcn_readfirstlane(base / K);
    RowPos p = {b, base - b * K};
    return p;
}

__device__ __forceinline__ RowPos row_pos(const RowPos &bp, const LaneOff &lo, int j, int K)
{
    RowPos p = {bp.bl + lo.ob[j], bp.t + lo.ot[j]};
    if (p.t >= K) {
        p.t -= K;
        ++p.bl;
    }
    return p;
}

__device__ __forceinline__ int wave_id()
{
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// context[b][s] = v into the forward's outputs (each (b, s) has one writer,
// so the add into the caller's row needs no atomic)
__device__ __forceinline__ void put_context(const CtxOut &o, int64_t b, int D, int s, float v)
{
    if (o.ctx) o.ctx[b * D + s] = v;
    if (o.enr) {
        float *e = o.enr + b * o.ld + s;
        *e = *e + v;
    }
}

// --------------------------------------------------------------- weight slice
// LDS image of [W_A | W_B | W_C][:, s0 .. s0+16) as bf16 hi/lo in MFMA
// B-operand order: entry ((q*3 + w)*2 + part)*64 + lane holds rows
// 32q + 8(lane/16) + 0..7 of weight w for state s0 + lane%16.
// The slice rows (16 contiguous floats each) are fetched with 16-byte loads,
// all issued up front; the rearrangement goes through a raw LDS tile of
// kRawRows rows, one weight (and row range) per round.
// largest multiple of 64 rows that divides SH2 and fits 16 KiB (256 rows)
constexpr int raw_rows_of(int nq)
{
    int best = 64;
    for (int r = 64; r <= 256; r += 64)
        if ((nq * 32) % r == 0) best = r;
    return best;
}

template <int NQ, int NT = kThreads>
struct WStage {
    static constexpr int SH2 = NQ * 32;
    static constexpr int kRawRows = raw_rows_of(NQ);
    static constexpr int kPieces = SH2 * 4;                  // 16-byte pieces per weight
    static constexpr int kPer = (kPieces + NT - 1) / NT;     // per thread per weight
    static constexpr int kRounds = SH2 / kRawRows;           // row ranges per weight
    static_assert(SH2 % kRawRows == 0 && kRawRows % 64 == 0, "row ranges of whole pieces");
    static_assert(kRounds == 1 || (kRawRows * 4) % NT == 0, "pieces of a round per thread");
    f4 v[3][kPer];

    __device__ __forceinline__ void load(const float *__restrict__ WA, const float *__restrict__ WB,
                                         const float *__restrict__ WC, int D, int s0)
    {
#pragma unroll
        for (int w = 0; w < 3; ++w) {
            const float *W = w == 0 ? WA : (w == 1 ? WB : WC);
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                // row idx/4, columns 4(idx%4)..; clamped rather than guarded so
                // that no path skips a load (waits for older loads stay exact)
                const int idx = kPieces % NT == 0 ? threadIdx.x + i * NT
                                                  : min(threadIdx.x + i * NT, kPieces - 1);
                v[w][i] = *reinterpret_cast<const f4 *>(W + (idx >> 2) * D + s0 + 4 * (idx & 3));
            }
        }
    }
    // raw: kRawRows * 16 floats of LDS, free during the call.  Ends with the
    // image written; the caller's barrier publishes it.
    __device__ __forceinline__ void store(u4 *Wl, float *raw) const
    {
        constexpr int kEntries = kRawRows / 32 * kWave;  // image entries per round
        constexpr int kPerRound = kRounds == 1 ? kPer : kRawRows * 4 / NT;
#pragma unroll
        for (int w = 0; w < 3; ++w)
#pragma unroll
            for (int rc = 0; rc < kRounds; ++rc) {
                if (w + rc > 0) __syncthreads();  // previous round's reads done
#pragma unroll
                for (int i = 0; i < kPerRound; ++i) {
                    const int idx = threadIdx.x + i * NT;
                    if (kRounds > 1 || kPieces % NT == 0 || idx < kPieces)
                        *reinterpret_cast<f4 *>(raw + 4 * idx) = v[w][rc * kPerRound + i];
                }
                __syncthreads();
#pragma unroll
                for (int j = 0; j < (kEntries + NT - 1) / NT; ++j) {
                    const int e = threadIdx.x + j * NT;
                    if (e < kEntries) {
                        const int ql = e >> 6, ln = e & 63;
                        float x[8];
#pragma unroll
                        for (int k = 0; k < 8; ++k)
                            x[k] = raw[(32 * ql + 8 * (ln >> 4) + k) * 16 + (ln & 15)];
                        const Split sp = split8(x);
                        const int q = rc * (kRawRows / 32) + ql;
                        Wl[((q * 3 + w) * 2 + 0) * kWave + ln] = sp.hi;
                        Wl[((q * 3 + w) * 2 + 1) * kWave + ln] = sp.lo;
                    }
                }
            }
    }
};

__device__ __forceinline__ Split wop(const u4 *Wl, int q, int w, int lane)
{
    Split s;
    s.hi = Wl[((q * 3 + w) * 2 + 0) * kWave + lane];
    s.lo = Wl[((q * 3 + w) * 2 + 1) * kWave + lane];
    return s;
}

// A|Bv projection of one 16-row block (results in MFMA output layout).  The
// block is taken by reference: a local copy of its registers cost one move
// per register and block.
template <typename TIn, int NQ>
__device__ __forceinline__ void project(const PBlk<TIn, NQ> &blk, const u4 *Wl, int lane,
                                        f4 &aA, f4 &aB)
{
    constexpr bool LO = PBlk<TIn, NQ>::kLo;
    aA = zero4();
    aB = zero4();
    // the weight operands of unit q + 1 are read while unit q is projected
    Split wan = wop(Wl, 0, 0, lane), wbn = wop(Wl, 0, 1, lane);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const Split wa = wan, wb = wbn;
        if (q + 1 < NQ) {
            wan = wop(Wl, q + 1, 0, lane);
            wbn = wop(Wl, q + 1, 1, lane);
        }
        const Split h = blk.op(q);
        aA = mfma3<LO>(h, wa, aA);
        aB = mfma3<LO>(h, wb, aB);
        // keep the weight-operand reads of later units from being hoisted
        // further (they would pin NQ x 16 registers next to the in-flight rows)
        __builtin_amdgcn_sched_barrier(0);
    }
}

// C projection partial over units q = wave + 4u for the group's 16 samples.
template <typename TIn, int NQ>
struct CvLoad {
    static constexpr int kU = (NQ + kWaves - 1) / kWaves;
    PBlk<TIn, 1> u[kU];
    __device__ __forceinline__ void load(const TIn *__restrict__ row, int wave, int kg)
    {
        // every unit loaded (clamped) so that no path skips a load
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            const int q = wave + kWaves * i;
            u[i].load(row + 32 * (q < NQ ? q : NQ - 1), kg);
        }
    }
    __device__ __forceinline__ f4 partial(const u4 *Wl, int wave, int lane) const
    {
        // unconditional products (a unit past SH2 repeats the last one and is
        // dropped by the select), so the loads have unconditional uses and
        // stay where they were issued
        constexpr bool LO = PBlk<TIn, 1>::kLo;
        f4 acc = zero4();
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            const int q = wave + kWaves * i;
            const f4 t = mfma3<LO>(u[i].op(0), wop(Wl, q < NQ ? q : NQ - 1, 2, lane), acc);
            acc = q < NQ ? t : acc;
        }
        return acc;
    }
};

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
// blocks of 16, carrying the state across blocks.  Two register buffers:
// the loads of block b+1 are issued just before block b is projected, so
// the memory system sees requests roughly in the order they are needed.
template <typename TIn, int NQ>
__device__ __forceinline__ void fwd_block(const PBlk<TIn, NQ> &blk, const u4 *Wl, int base,
                                          int lr_end, int K, int D, int s0, int64_t b0,
                                          float a_shift, const float (*cvp)[16][16], int lane,
                                          const LaneOff &lo, float &xc, const CtxOut &out)
{
    const int kg = lane >> 4, ln = lane & 15;
    const RowPos bp = base_pos(base, K);
    f4 aA[1], aB[1];
    project<TIn, NQ>(blk, Wl, lane, aA[0], aB[0]);
    Aff map[4];
    Aff F = aff_id();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = base + 4 * kg + j;
        Aff m;
        if (r >= lr_end) {
            m = aff_id();
        } else {
            m.m = sigmoid(aA[0][j] + a_shift);
            m.c = aB[0][j];
            m.r = row_pos(bp, lo, j, K).t == 0;
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
        const int r = base + 4 * kg + j;
        const RowPos rp = row_pos(bp, lo, j, K);
        if (r < lr_end && rp.t == K - 1) {
            const int bl = rp.bl;
            const float cv = cvp[0][bl][ln] + cvp[1][bl][ln] + cvp[2][bl][ln] + cvp[3][bl][ln];
            put_context(out, b0 + bl, D, s0 + ln, cv * x);
        }
    }
    xc = apply(total, xc);
}

template <typename TIn, int NQ>
__global__ void __launch_bounds__(kThreads, NQ <= 8 ? 2 : 1)
gscan_fwd_kernel(const TIn *__restrict__ hh, const TIn *__restrict__ hs2,
                 const float *__restrict__ WA, const float *__restrict__ WB,
                 const float *__restrict__ WC, int64_t B, int K, int D, int slices,
                 int64_t groups, float a_shift, CtxOut out)
{
    constexpr int SH2 = NQ * 32;
    __shared__ u4 Wl[NQ * 6 * kWave];
    __shared__ float cvp[kWaves][16][16];
    __shared__ f4 wraw[raw_rows_of(NQ) * 4];

    int64_t g;
    int slice;
    decode_block(slices, g, slice);
    if (g >= groups) return;
    const int s0 = slice * kSlice;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int kg = lane >> 4, ln = lane & 15;
    const int64_t b0 = g * kGroupSamples;
    const int nb = (int)(B - b0 < kGroupSamples ? B - b0 : kGroupSamples);
    const int lr_begin = 4 * wave * K;
    const int lr_end = (4 * wave + 4 < nb ? 4 * wave + 4 : nb) * K;
    const bool active = lr_begin < lr_end;
    const TIn *__restrict__ hg = hh + b0 * K * SH2;  // the group's first row
    const LaneOff lo = lane_offsets(kg, K);
    auto rowp = [&](int base) {
        const int r = base + ln;
        return hg + (uint32_t)((r < lr_end ? r : lr_end - 1) * SH2);
    };

    // loads in the order they are consumed: weights, h_s2, first h block
    WStage<NQ> wst;
    wst.load(WA, WB, WC, D, s0);
    CvLoad<TIn, NQ> cvl;
    cvl.load(hs2 + b0 * SH2 + (uint32_t)((ln < nb ? ln : nb - 1) * SH2), wave, kg);
    PBlk<TIn, NQ> b0buf, b1buf;
    b0buf.load(rowp(lr_begin), kg);  // clamped: a valid row even for an idle wavefront
    wst.store(Wl, reinterpret_cast<float *>(wraw));
    __syncthreads();
    {
        const f4 cp = cvl.partial(Wl, wave, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) cvp[wave][4 * kg + j][ln] = cp[j];
    }
    __syncthreads();
    if (!active) return;

    // the next block is always requested (clamped to the last row past the
    // end), so the wait for the current block leaves it in flight
    float xc = 0.f;
    for (int base = lr_begin; base < lr_end; base += 2 * kBlockRows) {
        const int base1 = base + kBlockRows;
        b1buf.load(rowp(base1), kg);
        fwd_block<TIn, NQ>(b0buf, Wl, base, lr_end, K, D, s0, b0, a_shift, cvp, lane, lo, xc, out);
        if (base1 >= lr_end) break;
        b0buf.load(rowp(base1 + kBlockRows), kg);
        fwd_block<TIn, NQ>(b1buf, Wl, base1, lr_end, K, D, s0, b0, a_shift, cvp, lane, lo, xc, out);
    }
}

template <typename TIn, int NQ>
__global__ void __launch_bounds__(kThreads, NQ <= 8 ? 2 : 1)
gscan_fwd_persist_kernel(const TIn *__restrict__ hh, const TIn *__restrict__ hs2,
                 const float *__restrict__ WA, const float *__restrict__ WB,
                 const float *__restrict__ WC, int64_t B, int K, int D, int slices,
                 int64_t groups, int64_t nrows, float a_shift, CtxOut out)
{
    constexpr int SH2 = NQ * 32;
    __shared__ u4 Wl[NQ * 6 * kWave];
    __shared__ float cvp[kWaves][16][16];
    __shared__ f4 wraw[raw_rows_of(NQ) * 4];

    // persistent over the groups g, g + nrows, ... of one state slice (more
    // groups than grid rows): the weights are staged once per workgroup
    int64_t g;
    int slice;
    decode_block(slices, g, slice);
    if (g >= groups) return;
    const int s0 = slice * kSlice;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int kg = lane >> 4, ln = lane & 15;
    const int lr_begin = 4 * wave * K;
    const LaneOff lo = lane_offsets(kg, K);
    auto samples_of = [&](int64_t gg) {
        return (int)(B - gg * kGroupSamples < kGroupSamples ? B - gg * kGroupSamples
                                                            : kGroupSamples);
    };
    auto end_of = [&](int nb) { return (4 * wave + 4 < nb ? 4 * wave + 4 : nb) * K; };
    // a row of group gg for this lane, clamped to the wavefront's last row
    // (a valid row even for an idle wavefront: its end is at least K)
    auto rowp = [&](int64_t gg, int lr_end, int base) {
        const int r = base + ln;
        return hh + gg * kGroupSamples * K * SH2 + (uint32_t)((r < lr_end ? r : lr_end - 1) * SH2);
    };
    auto cv_rows = [&](int64_t gg, int nb) {
        return hs2 + gg * kGroupSamples * SH2 + (uint32_t)((ln < nb ? ln : nb - 1) * SH2);
    };

    // loads in the order they are consumed: weights, h_s2, first h block
    int nb = samples_of(g);
    int lr_end = end_of(nb);
    WStage<NQ> wst;
    wst.load(WA, WB, WC, D, s0);
    CvLoad<TIn, NQ> cvl;
    cvl.load(cv_rows(g, nb), wave, kg);
    PBlk<TIn, NQ> b0buf, b1buf;
    b0buf.load(rowp(g, lr_end, lr_begin), kg);
    wst.store(Wl, reinterpret_cast<float *>(wraw));
    for (;;) {
        const int64_t b0 = g * kGroupSamples;
        __syncthreads();  // weights staged; the previous group's readers of cvp done
        {
            const f4 cp = cvl.partial(Wl, wave, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) cvp[wave][4 * kg + j][ln] = cp[j];
        }
        __syncthreads();
        if (lr_begin < lr_end) {
            // the next block is always requested (clamped to the last row past
            // the end), so the wait for the current block leaves it in flight
            float xc = 0.f;
            for (int base = lr_begin; base < lr_end; base += 2 * kBlockRows) {
                const int base1 = base + kBlockRows;
                b1buf.load(rowp(g, lr_end, base1), kg);
                fwd_block<TIn, NQ>(b0buf, Wl, base, lr_end, K, D, s0, b0, a_shift, cvp, lane, lo,
                                   xc, out);
                if (base1 >= lr_end) break;
                b0buf.load(rowp(g, lr_end, base1 + kBlockRows), kg);
                fwd_block<TIn, NQ>(b1buf, Wl, base1, lr_end, K, D, s0, b0, a_shift, cvp, lane, lo,
                                   xc, out);
            }
        }
        g += nrows;
        if (g >= groups) break;
        // the next group's C rows and first block go out before the barriers
        nb = samples_of(g);
        lr_end = end_of(nb);
        cvl.load(cv_rows(g, nb), wave, kg);
        b0buf.load(rowp(g, lr_end, lr_begin), kg);
    }
}

// =============================== forward, several state slices per workgroup
// With D > 16 the kernels above re-read and re-split every row once per
// 16-state slice.  Here a workgroup of 8 wavefronts takes two groups of 16
// samples (wavefronts 0-3 and 4-7, four samples each) and S slices: each
// 32-column unit of a row block is split once and multiplied with the A and
// B weights of all S slices, held in LDS as one bf16 hi/lo image (S * SH2 *
// 32 pairs, at most 128 KiB).  The C weights pass through the same LDS first,
// for the C values of both groups.  Each wavefront takes two 16-row blocks
// per pass, so that every weight operand read from LDS serves both.
constexpr int kWavesM = 8;
constexpr int kThreadsM = kWave * kWavesM;

// LDS image of NW weights over S slices: entry r = (s * NQ + q) * NW + w
// holds, for lane l, rows 32q + 8(l/16) + 0..7 of weight w at state
// s0 + 16s + l%16, split into bf16 high (u4 index 2r * 64 + l) and low
// (index (2r + 1) * 64 + l).  Read straight from the fp32 weights: each
// lane group of 16 reads 64 contiguous bytes of a row.
template <int NQ, int S, int NW>
__device__ __forceinline__ void stage_image(u4 *img, const float *__restrict__ W0,
                                            const float *__restrict__ W1, int D, int s0)
{
    constexpr int kEnt = S * NQ * NW * kWave;
    constexpr int kRounds = (kEnt + kThreadsM - 1) / kThreadsM;
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
        const int e = threadIdx.x + i * kThreadsM;
        if (kEnt % kThreadsM == 0 || e < kEnt) {
            const int lane = e & 63, r = e >> 6;
            const int w = NW == 1 ? 0 : r % NW;
            const int sq = r / NW, q = sq % NQ, s = sq / NQ;
            const float *__restrict__ W = w == 0 ? W0 : W1;
            const float *p = W + (32 * q + 8 * (lane >> 4)) * D + s0 + 16 * s + (lane & 15);
            float x[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = p[k * D];
            const Split sp = split8(x);
            img[(2 * r) * kWave + lane] = sp.hi;
            img[(2 * r + 1) * kWave + lane] = sp.lo;
        }
    }
}

__device__ __forceinline__ Split img_op(const u4 *img, int r, int lane)
{
    Split s;
    s.hi = img[(2 * r) * kWave + lane];
    s.lo = img[(2 * r + 1) * kWave + lane];
    return s;
}

template <typename TIn, int NQ, int S>
__global__ void __launch_bounds__(kThreadsM, 1)
gscan_fwd_ms_kernel(const TIn *__restrict__ hh, const TIn *__restrict__ hs2,
                    const float *__restrict__ WA, const float *__restrict__ WB,
                    const float *__restrict__ WC, int64_t B, int K, int D, int sgroups,
                    int64_t groups, float a_shift, CtxOut out)
{
    constexpr int SH2 = NQ * 32;
    constexpr bool LO = PBlk<TIn, NQ>::kLo;
    constexpr int kImg = S * NQ * 4 * kWave;  // u4 entries of the A|B image
    constexpr int kPart = 2 * 4 * S * 16 * 16 / 4;  // u4 entries of the C partials
    __shared__ u4 img[kImg > kPart ? kImg : kPart];
    __shared__ float cvs[2][S][16][16];  // C values of both groups

    // (pair of groups, set of S slices); the slice sets of one pair run on one XCD
    int64_t pr;
    int sg;
    decode_block(sgroups, pr, sg);
    if (pr >= (groups + 1) / 2) return;  // whole workgroup
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int team = wave >> 2, wt = wave & 3;
    const int kg = lane >> 4, ln = lane & 15;
    const int s0 = sg * S * kSlice;
    // the second group of a pair may lie past the batch: that team repeats
    // the last group's loads and takes part in the barriers, writing nothing
    const int64_t graw = 2 * pr + team;
    const bool gvalid = graw < groups;
    const int64_t g = gvalid ? graw : groups - 1;
    const int64_t b0 = g * kGroupSamples;
    const int nb = (int)(B - b0 < kGroupSamples ? B - b0 : kGroupSamples);
    const int lr_begin = 4 * wt * K;
    const int lr_end = (4 * wt + 4 < nb ? 4 * wt + 4 : nb) * K;
    const TIn *__restrict__ hg = hh + b0 * K * SH2;
    const LaneOff lo = lane_offsets(kg, K);
    auto rowp = [&](int base) {
        const int r = base + ln;
        return hg + (uint32_t)((r < lr_end ? r : lr_end - 1) * SH2);
    };

    // C values: h_s2 units q = wt + 4i of the group against the C image
    CvLoad<TIn, NQ> cvl;
    cvl.load(hs2 + b0 * SH2 + (uint32_t)((ln < nb ? ln : nb - 1) * SH2), wt, kg);
    // Two 16-row blocks (32 rows) per pass: each weight operand read from
    // LDS feeds the products of both blocks, halving the LDS traffic per
    // row.  The rows wait in a ring of R register slots per block: slot
    // (q % R) holds unit q, and as soon as a unit has been split its slot
    // takes the next unit that maps to it (unit q + R of this pair, or a unit
    // of the next pair), so R < NQ slots keep R units of lead on every load.
    // The first pair's first R units go out before the weight staging.
    // R divides NQ (a slot holds units q, q + R, ...): four where it can,
    // whole blocks for SH2 <= 192.
    constexpr int R = NQ % 4 == 0 && NQ >= 8 ? 4 : (NQ == 10 ? 5 : (NQ == 14 ? 7 : NQ));
    static_assert(NQ % R == 0, "ring slots");
    PBlk<TIn, R> r0, r1;
#pragma unroll
    for (int u = 0; u < R; ++u) {
        r0.load_unit_at(rowp(lr_begin), kg, u, u);
        r1.load_unit_at(rowp(lr_begin + kBlockRows), kg, u, u);
    }
    stage_image<NQ, S, 1>(img, WC, WC, D, s0);
    __syncthreads();
    f4 cp[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        f4 acc = zero4();
#pragma unroll
        for (int i = 0; i < CvLoad<TIn, NQ>::kU; ++i) {
            const int q = wt + kWaves * i;
            const f4 t = mfma3<LO>(cvl.u[i].op(0), img_op(img, s * NQ + (q < NQ ? q : NQ - 1), lane), acc);
            acc = q < NQ ? t : acc;
        }
        cp[s] = acc;
    }
    __syncthreads();  // C image read
    float(*const pt)[4][S][16][16] = reinterpret_cast<float(*)[4][S][16][16]>(img);
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) pt[team][wt][s][4 * kg + j][ln] = cp[s][j];
    __syncthreads();
    for (int e = threadIdx.x; e < 2 * S * 256; e += kThreadsM) {
        const int tm = e / (S * 256), s = (e / 256) % S, bl = (e >> 4) & 15, l = e & 15;
        cvs[tm][s][bl][l] = (pt[tm][0][s][bl][l] + pt[tm][1][s][bl][l]) +
                            (pt[tm][2][s][bl][l] + pt[tm][3][s][bl][l]);
    }
    __syncthreads();  // partials read before the A|B image overwrites them
    stage_image<NQ, S, 2>(img, WA, WB, D, s0);
    __syncthreads();
    if (!gvalid || lr_begin >= lr_end) return;

    float xc[S];
#pragma unroll
    for (int s = 0; s < S; ++s) xc[s] = 0.f;
    for (int base = lr_begin; base < lr_end; base += 2 * kBlockRows) {
        const TIn *__restrict__ row0 = rowp(base), *__restrict__ row1 = rowp(base + kBlockRows);
        // the next pair's rows (clamped past the end)
        const TIn *__restrict__ nrow0 = rowp(base + 2 * kBlockRows);
        const TIn *__restrict__ nrow1 = rowp(base + 3 * kBlockRows);
        // slot (u % R) is free once unit u is split: it takes unit u + R of
        // this pair, or unit u + R - NQ of the next
        auto refill = [&](int u) __attribute__((always_inline)) {
            const int n = u + R;
            if (n < NQ) {
                r0.load_unit_at(row0, kg, n, u % R);
                r1.load_unit_at(row1, kg, n, u % R);
            } else {
                r0.load_unit_at(nrow0, kg, n - NQ, u % R);
                r1.load_unit_at(nrow1, kg, n - NQ, u % R);
            }
        };
        f4 aA0[S], aB0[S], aA1[S], aB1[S];
#pragma unroll
        for (int s = 0; s < S; ++s) {
            aA0[s] = zero4();
            aB0[s] = zero4();
            aA1[s] = zero4();
            aB1[s] = zero4();
        }
        // unit q + 1 is split (and its slot refilled) in the same stretch as
        // unit q's products, so the split's vector work can issue while the
        // matrix cores run
        Split h0n = r0.op(0), h1n = r1.op(0);
        refill(0);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const Split h0 = h0n, h1 = h1n;
            if (q + 1 < NQ) {
                h0n = r0.op((q + 1) % R);
                h1n = r1.op((q + 1) % R);
                refill(q + 1);
            }
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const Split wa = img_op(img, (s * NQ + q) * 2, lane);
                const Split wb = img_op(img, (s * NQ + q) * 2 + 1, lane);
                aA0[s] = mfma3<LO>(h0, wa, aA0[s]);
                aA1[s] = mfma3<LO>(h1, wa, aA1[s]);
                aB0[s] = mfma3<LO>(h0, wb, aB0[s]);
                aB1[s] = mfma3<LO>(h1, wb, aB1[s]);
            }
            // keep later units' operand reads from being hoisted further
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const int bb = base + kBlockRows * hb;
            const RowPos bp = base_pos(bb, K);
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const f4 pa = hb ? aA1[s] : aA0[s], pbv = hb ? aB1[s] : aB0[s];
                Aff map[4];
                Aff F = aff_id();
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = bb + 4 * kg + j;
                    Aff m;
                    if (r >= lr_end) {
                        m = aff_id();
                    } else {
                        m.m = sigmoid(pa[j] + a_shift);
                        m.c = pbv[j];
                        m.r = row_pos(bp, lo, j, K).t == 0;
                    }
                    map[j] = m;
                    F = compose(m, F);
                }
                Aff excl, total;
                scan_up(F, lane, excl, total);
                float x = apply(excl, xc[s]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x = apply(map[j], x);
                    const int r = bb + 4 * kg + j;
                    const RowPos rp = row_pos(bp, lo, j, K);
                    if (r < lr_end && rp.t == K - 1)
                        put_context(out, b0 + rp.bl, D, s0 + 16 * s + ln, cvs[team][s][rp.bl][ln] * x);
                }
                xc[s] = apply(total, xc[s]);
            }
        }
    }
}

// ============================================================= backward kernel
constexpr int nsb_of(int nq) { return nq * 32 / 64; }
constexpr int sbw_of(int nq) { return (nsb_of(nq) + kWaves - 1) / kWaves; }

// Rows of a chunk in the transposed ("T") layout for one 64-column
// superblock ib: lane l holds columns 64*ib + 4*(l%16) + 0..3 of chunk row
// 16(2*kap + e/4) + 4(l/16) + e%4 in hv[e]; this row order is the
// contraction's MFMA k index 8(l/16) + e.
template <typename TIn, int NQ>
__device__ __forceinline__ void load_t_half(typename Col4<TIn>::raw_t (&hv)[8],
                                            const TIn *__restrict__ hg, int cb, int NR, int ib,
                                            int kap, int lane)
{
    constexpr int SH2 = NQ * 32;
    const int kg = lane >> 4, ln = lane & 15;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int r = cb + kBlockRows * (2 * kap + e / 4) + 4 * kg + (e & 3);
        const int rc = r < NR ? r : NR - 1;
        hv[e] = Col4<TIn>::raw(hg + (uint32_t)(rc * SH2 + 64 * ib + 4 * ln));
    }
}

// acc{A,B}[c] += sum over the 32 chunk rows of half kap of h[r, i] (x) d{A,B}[r, s]
// for i = 64*ib + 4*(4*(l/16) + jj) + c, s = l%16 (one superblock).
template <typename TIn>
__device__ __forceinline__ void contract_half(f4 (&accA)[4], f4 (&accB)[4],
                                              const typename Col4<TIn>::raw_t (&hv)[8],
                                              const Split &sA, const Split &sB)
{
    constexpr bool LO = PBlk<TIn, 1>::kLo;
    f4 w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = Col4<TIn>::widen(hv[e]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float col[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) col[e] = w[e][c];
        const Split sh = split8(col);
        accA[c] = mfma3<LO>(sh, sA, accA[c]);
        accB[c] = mfma3<LO>(sh, sB, accB[c]);
    }
}

// dL/dA, dL/dBv of chunk half kap as split B operands, rows outside [lo, hi) zeroed.
__device__ __forceinline__ void grad_operands(Split &sA, Split &sB, const f4 (*dab)[2][kWave],
                                              int kap, int cb, int lo, int hi, int lane)
{
    const int kg = lane >> 4;
    const f4 a0 = dab[2 * kap][0][lane], a1 = dab[2 * kap + 1][0][lane];
    const f4 b0 = dab[2 * kap][1][lane], b1 = dab[2 * kap + 1][1][lane];
    float da[8], db[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int r = cb + kBlockRows * (2 * kap + e / 4) + 4 * kg + (e & 3);
        const bool in = r >= lo && r < hi;
        da[e] = in ? (e < 4 ? a0[e] : a1[e - 4]) : 0.f;
        db[e] = in ? (e < 4 ? b0[e] : b1[e - 4]) : 0.f;
    }
    sA = split8(da);
    sB = split8(db);
}

// All superblocks of this wavefront; hv0 holds superblock `wave`'s rows when
// EARLY (requested together with the chunk's projection rows, so they are
// served from the same cache lines), otherwise rows are loaded here.
template <typename TIn, int NQ, bool EARLY>
__device__ __forceinline__ void contract_rows(f4 (&accA)[sbw_of(NQ)][4],
                                              f4 (&accB)[sbw_of(NQ)][4],
                                              const typename Col4<TIn>::raw_t (&hv0)[2][8],
                                              const TIn *__restrict__ hg, int cb, int NR, int lo,
                                              int hi, const f4 (*dab)[2][kWave], int wave,
                                              int lane)
{
    constexpr int NSB = nsb_of(NQ);
    constexpr int SBW = sbw_of(NQ);
    if (wave >= NSB) return;
#pragma unroll
    for (int kap = 0; kap < 2; ++kap) {
        Split sA, sB;
        grad_operands(sA, sB, dab, kap, cb, lo, hi, lane);
#pragma unroll
        for (int sbi = 0; sbi < SBW; ++sbi) {
            const int ib = wave + kWaves * sbi;
            if (ib >= NSB) break;
            if (EARLY && sbi == 0) {
                contract_half<TIn>(accA[0], accB[0], hv0[kap], sA, sB);
            } else {
                typename Col4<TIn>::raw_t hv[8];
                load_t_half<TIn, NQ>(hv, hg, cb, NR, ib, kap, lane);
                contract_half<TIn>(accA[sbi], accB[sbi], hv, sA, sB);
            }
        }
    }
}

// Persistent over groups.  Rows of a group are processed in 64-row chunks,
// wavefront w projecting block w of the chunk.  dL/dA and dL/dBv of the
// chunk go to LDS and every wavefront contracts all 64 rows against its own
// 64-column superblocks of SH2 (the "i split"), so each wavefront keeps only
// SH2/8 gradient accumulators per set.  The next chunk's rows (possibly the
// next group's) are requested right after the current chunk's projection.
//
// ALIGNED (K divides 16): every 16-row block holds whole samples, so blocks
// need no state from one another and the cross-wavefront scan is skipped.
// Otherwise the forward state and the reverse adjoint are carried across
// blocks through LDS, and a sample that continues past the chunk end is
// handled with an "open" accumulator: its rows' adjoints are computed with
// the future gates set to 1; when the next chunk's gates of that sample are
// known the open accumulator is scaled by their product (per state) before
// the new rows are added (Horner's scheme), and once the sample ends it is
// folded into the closed accumulator.
template <typename TIn, int NQ, bool ALIGNED>
__global__ void __launch_bounds__(kThreads, NQ <= 8 ? 2 : 1)
gscan_bwd_kernel(const TIn *__restrict__ hh, const TIn *__restrict__ hs2,
                 const float *__restrict__ WA, const float *__restrict__ WB,
                 const float *__restrict__ WC, int64_t B, int K, int D, int slices,
                 int64_t groups, int64_t nrows, float a_shift, const float *__restrict__ dctx,
                 float *__restrict__ part, float *__restrict__ ab_out,
                 float *__restrict__ cv_out)
{
    constexpr int SH2 = NQ * 32;
    constexpr int NSB = nsb_of(NQ);
    constexpr int SBW = sbw_of(NQ);
    constexpr bool EARLY = SBW == 1;  // T rows requested with the chunk's projection rows
    constexpr int NOPEN = ALIGNED ? 1 : SBW;  // open accumulators (unused when aligned)
    __shared__ u4 Wl[NQ * 6 * kWave];
    __shared__ float cvp[2][kWaves][16][16];  // C partials, by group parity
    __shared__ float dctl[2][16][16];         // d_context slice, by group parity
    __shared__ float dCl[2][16][16];          // dL/dC = d_context * x_K, by group parity
    __shared__ float fsum[ALIGNED ? 1 : 2][kWaves][3][16];
    __shared__ float rsum[ALIGNED ? 1 : 2][kWaves][3][16];
    __shared__ f4 dab[2][kWaves][2][kWave];
    __shared__ float gprev[2][16];

    int64_t rho;
    int slice;
    decode_block(slices, rho, slice);
    const int s0 = slice * kSlice;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = wave_id();
    const int kg = lane >> 4, ln = lane & 15;
    // (sample, step) of a row: shifts when K is a power of two dividing 16,
    // otherwise the division-free offsets
    const int kshift = __builtin_ctz((unsigned)K);
    LaneOff lof;
    if constexpr (!ALIGNED) lof = lane_offsets(kg, K);
    auto rowpos = [&](const RowPos &bp, int lr, int j) {
        if constexpr (ALIGNED) {
            RowPos p = {lr >> kshift, lr & (K - 1)};
            return p;
        } else {
            return row_pos(bp, lof, j, K);
        }
    };

    f4 accAc[SBW][4], accBc[SBW][4], accC[SBW][4];
    f4 accAo[NOPEN][4], accBo[NOPEN][4];
#pragma unroll
    for (int i = 0; i < SBW; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            accAc[i][c] = zero4();
            accBc[i][c] = zero4();
            accC[i][c] = zero4();
        }
#pragma unroll
    for (int i = 0; i < NOPEN; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            accAo[i][c] = zero4();
            accBo[i][c] = zero4();
        }

    // rows of chunk c of group g for this wavefront's projection
    auto prow = [&](int64_t gg, int cbase) {
        const int64_t bb = gg * kGroupSamples;
        const int nbb = (int)(B - bb < kGroupSamples ? B - bb : kGroupSamples);
        const int nr = nbb * K;
        const int r = cbase + kBlockRows * wave + ln;
        return hh + bb * K * SH2 + (uint32_t)((r < nr ? r : nr - 1) * SH2);
    };

    PBlk<TIn, NQ> pb;
    {
        // the adjoint buffer doubles as the raw tile of the weight staging
        WStage<NQ> wst;
        wst.load(WA, WB, WC, D, s0);
        static_assert(sizeof(dab) >= raw_rows_of(NQ) * 16 * sizeof(float), "raw tile");
        wst.store(Wl, reinterpret_cast<float *>(dab));
    }

    int chunk_id = 0;
    int gpar = 0;
    for (int64_t g = rho; g < groups; g += nrows, gpar ^= 1) {
        const int64_t b0 = g * kGroupSamples;
        const int nb = (int)(B - b0 < kGroupSamples ? B - b0 : kGroupSamples);
        const TIn *__restrict__ hg = hh + b0 * K * SH2;  // the group's first row
        const int NR = nb * K;
        const int nch = (NR + kChunkRows - 1) / kChunkRows;
        {
            CvLoad<TIn, NQ> cvl;
            cvl.load(hs2 + b0 * SH2 + (uint32_t)((ln < nb ? ln : nb - 1) * SH2), wave, kg);
            const int bl = tid >> 4, s = tid & 15;
            dctl[gpar][bl][s] = bl < nb ? dctx[(b0 + bl) * D + s0 + s] : 0.f;
            if (g == rho) __syncthreads();  // weights staged
            const f4 cp = cvl.partial(Wl, wave, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) cvp[gpar][wave][4 * kg + j][ln] = cp[j];
        }
        __syncthreads();
        if (cv_out) {  // C of the group's samples, for the input gradients
            const int bl = tid >> 4, s = tid & 15;
            if (bl < nb)
                cv_out[(b0 + bl) * D + s0 + s] = cvp[gpar][0][bl][s] + cvp[gpar][1][bl][s] +
                                                 cvp[gpar][2][bl][s] + cvp[gpar][3][bl][s];
        }
        // lambda_K = dL/dx_K = d_context * C for local sample bl, state l%16
        auto lam = [&](int bl) {
            return dctl[gpar][bl][ln] * (cvp[gpar][0][bl][ln] + cvp[gpar][1][bl][ln] +
                                         cvp[gpar][2][bl][ln] + cvp[gpar][3][bl][ln]);
        };

        float xc = 0.f;
        for (int c = 0; c < nch; ++c, ++chunk_id) {
            const int buf = chunk_id & 1;
            const int cb = c * kChunkRows;
            const int ce = cb + kChunkRows < NR ? cb + kChunkRows : NR;
            const int lr0 = cb + kBlockRows * wave;
            // the chunk's projection rows and, right behind them, its transposed rows
            f4 aA[1], aB[1];
            typename Col4<TIn>::raw_t hv0[2][8];
            pb.load(prow(g, cb), kg);
            if constexpr (EARLY) {
                if (wave < NSB) {
                    load_t_half<TIn, NQ>(hv0[0], hg, cb, NR, wave, 0, lane);
                    load_t_half<TIn, NQ>(hv0[1], hg, cb, NR, wave, 1, lane);
                }
            }
            project<TIn, NQ>(pb, Wl, lane, aA[0], aB[0]);
            if (ab_out) {
                // the projections A | Bv of this block's rows, for the input
                // gradients (samples may continue past the chunk, so the
                // exact adjoints come from a later per-sample pass).  Lane
                // indices from an opaque zero, computed here, not held.
                int z;
                asm volatile("s_mov_b32 %0, 0" : "=s"(z));
                const int zl = (threadIdx.x + z) & 63;
                const int zr = cb + kBlockRows * wave + 4 * (zl >> 4);
                float *o = ab_out + (b0 * K + zr) * (int64_t)(2 * D) + s0 + (zl & 15);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (zr + j < ce) {
                        o[j * 2 * D] = aA[0][j];
                        o[j * 2 * D + D] = aB[0][j];
                    }
            }

            // per-row maps (forward state and reverse adjoint)
            RowPos bp = {0, 0};
            if constexpr (!ALIGNED) bp = base_pos(lr0, K);
            Aff fm[4], rm[4];
            float gate[4], gcom[4];
            Aff F = aff_id();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = lr0 + 4 * kg + j;
                const RowPos rp = rowpos(bp, r, j);
                const int bl = rp.bl, t = rp.t;
                const Gate gg = gate_of(aA[0][j] + a_shift);
                const float gt = gg.g;
                gate[j] = gt;
                gcom[j] = gg.gc;
                if (r >= ce) {
                    fm[j] = aff_id();
                    rm[j] = aff_id();
                } else {
                    fm[j].m = gt;
                    fm[j].c = aB[0][j];
                    fm[j].r = t == 0;
                    rm[j].m = gt;
                    rm[j].c = (t == 0 && bl > 0) ? lam(bl - 1) : 0.f;
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

            float xin = 0.f, xnext = 0.f, gpre = 1.f, gall = 1.f, mu;
            if constexpr (ALIGNED) {
                // the block starts a sample and ends one: no carries needed
                const int last = (lr0 + kBlockRows < ce ? lr0 + kBlockRows : ce) - 1;
                mu = last >= lr0 ? lam(last >> kshift) : 0.f;
            } else {
                if (kg == 0) {
                    fsum[buf][wave][0][ln] = Ft.m;
                    fsum[buf][wave][1][ln] = Ft.c;
                    fsum[buf][wave][2][ln] = (float)Ft.r;
                    rsum[buf][wave][0][ln] = Rt.m;
                    rsum[buf][wave][1][ln] = Rt.c;
                    rsum[buf][wave][2][ln] = (float)Rt.r;
                }
                __syncthreads();
                xin = xc;
                xnext = xc;
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
                mu = lam((ce - 1) / K);
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
            }

            // the sample open at the chunk start (if any) and its last row
            const bool has_prev = !ALIGNED && (cb % K) != 0;
            const int prev_end = (cb / K + 1) * K - 1;

            // forward walk: state before each row, dL/dC at sample ends,
            // gate product of the open sample
            float x = apply(Fx, xin);
            float grun = Fx.m * gpre;
            float xbef[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = lr0 + 4 * kg + j;
                const RowPos rp = rowpos(bp, r, j);
                const int bl = rp.bl, t = rp.t;
                xbef[j] = t == 0 ? 0.f : x;
                x = apply(fm[j], x);
                grun *= fm[j].m;
                if (r < ce && t == K - 1) dCl[gpar][bl][ln] = dctl[gpar][bl][ln] * x;
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
                dA4[j] = v ? m_in * xbef[j] * (gt * gcom[j]) : 0.f;
                m_in = apply(rm[j], m_in);
            }
            dab[buf][wave][0][lane] = dA4;
            dab[buf][wave][1][lane] = dB4;
            __syncthreads();

            // weight-gradient contraction of the chunk
            if constexpr (ALIGNED) {
                contract_rows<TIn, NQ, EARLY>(accAc, accBc, hv0, hg, cb, NR, cb, ce, dab[buf], wave,
                                              lane);
            } else {
                const int bl_top = (ce - 1) / K;
                const bool top_open = (bl_top + 1) * K > ce;
                const int rN = top_open ? bl_top * K : ce;  // rows >= rN continue past the chunk
                if (!has_prev && !top_open) {
                    contract_rows<TIn, NQ, EARLY>(accAc, accBc, hv0, hg, cb, NR, cb, ce, dab[buf],
                                                  wave, lane);
                } else {
                    if (has_prev) {
                        const float gs = prev_end < ce ? gprev[buf][ln] : gall;
#pragma unroll
                        for (int i = 0; i < NOPEN; ++i)
#pragma unroll
                            for (int cc = 0; cc < 4; ++cc) {
                                accAo[i][cc] *= gs;
                                accBo[i][cc] *= gs;
                            }
                    }
                    if (rN > cb) {
                        contract_rows<TIn, NQ, EARLY>(accAo, accBo, hv0, hg, cb, NR, cb, rN, dab[buf],
                                                      wave, lane);
#pragma unroll
                        for (int i = 0; i < NOPEN; ++i)
#pragma unroll
                            for (int cc = 0; cc < 4; ++cc) {
                                accAc[i][cc] += accAo[i][cc];
                                accBc[i][cc] += accBo[i][cc];
                                accAo[i][cc] = zero4();
                                accBo[i][cc] = zero4();
                            }
                    }
                    if (rN < ce)
                        contract_rows<TIn, NQ, EARLY>(accAo, accBo, hv0, hg, cb, NR, rN, ce, dab[buf],
                                                      wave, lane);
                }
                xc = xnext;
            }
        }

        // dW_C rows of this group: h_s2^T @ dL/dC (dCl complete after the last
        // chunk's barrier), fp32 MFMA with k = 4 samples per step
#pragma unroll
        for (int sbi = 0; sbi < SBW; ++sbi) {
            const int ib = wave + kWaves * sbi;
            if (ib >= NSB) break;
            f4 hv[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int bl = 4 * a + kg;
                const int blc = bl < nb ? bl : nb - 1;
                hv[a] = Col4<TIn>::widen(
                    Col4<TIn>::raw(hs2 + b0 * SH2 + (uint32_t)(blc * SH2 + 64 * ib + 4 * ln)));
            }
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int bl = 4 * a + kg;
                const float dc = bl < nb ? dCl[gpar][bl][ln] : 0.f;
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) accC[sbi][cc] = mfma_f32(hv[a][cc], dc, accC[sbi][cc]);
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

struct BTask {
    int64_t g;  // group (no task when g >= groups)
    int c;      // chunk within the group
    int k;      // ordinal of the group in this workgroup (LDS parity)
    int n;      // ordinal of the chunk in this workgroup
};

// ================================= backward, K dividing 16, or 32, 64 ("rows")
// When K divides 16 every 16-row block holds whole samples, so the block's
// scans need nothing from other blocks: projection replay, forward and
// reverse scans, and the weight-gradient contraction over the block's own
// 16 rows.  With K = 32 or 64 a sample fills 2 or 4 blocks of one 64-row
// chunk, and one exchange of the blocks' state maps through LDS completes
// the scans.  The contraction needs h with rows along the MFMA k index,
// while the row loads put columns along k.  The split block (bf16 high and
// low planes) goes to a per-wavefront LDS tile right after the split, and
// ds_read_b64_tr_b16 reads it back transposed: four rows of one column per
// lane.  Four rows of high parts and the same four rows of low parts make
// one k = 32 operand [high | low]; its products with [dhigh | dhigh] and
// [dlow | 0] give the three terms of the split product in two MFMAs.  No
// transposed reloads and no second split.  One persistent workgroup per CU;
// the next chunk's rows are requested as soon as the current chunk has
// been split, the next group's h_s2 rows at the start of each step.

typedef short s4v __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// i%4 of the 8-byte chunks addressed by lanes 4j + i/4, j = 0..3.  With lane
// p of group g addressing row 4g + p/4, columns c + 4(p%4) .. +3 of a
// row-major bf16 tile, lane i gets column c + i of rows 4g .. 4g+3.
__device__ __forceinline__ uint2 read_tr(const uint16_t *p)
{
    const s4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s4v *)(p));
    return __builtin_bit_cast(uint2, v);
}

// B operands for four rows 4(l/16) + j of one state: [dhigh | dhigh] and
// [dlow | 0] (LO), or [dhigh | dlow] when the A operand is [high | high]
struct GradOp {
    u4 b1, b2;
};

template <bool LO>
__device__ __forceinline__ GradOp grad_op(const f4 &d)
{
    const uint32_t h01 = pack_bf16(d[0], d[1]), h23 = pack_bf16(d[2], d[3]);
    const uint32_t l01 = pack_lo(h01, d[0], d[1]);
    const uint32_t l23 = pack_lo(h23, d[2], d[3]);
    GradOp g;
    if constexpr (LO) {
        g.b1 = u4{h01, h23, h01, h23};
        g.b2 = u4{l01, l23, 0u, 0u};
    } else {
        g.b1 = u4{h01, h23, l01, l23};
        g.b2 = zero_u4();
    }
    return g;
}

template <bool LO>
__device__ __forceinline__ f4 contract_op(const u4 &a, const GradOp &g, f4 acc)
{
    acc = mfma_bf(a, g.b1, acc);
    if constexpr (LO) acc = mfma_bf(a, g.b2, acc);
    return acc;
}

// Workgroup of 8 wavefronts, two per SIMD: wavefronts w and w+4 share the
// 16-row block w%4 of each 64-row chunk, each owning half of the SH2
// columns (units h*NQ/2 .. (h+1)*NQ/2 - 1, h = w/4).  Each loads, splits and
// projects its half; the two partial projections are added through LDS
// (both wavefronts form the same sum, so both run identical scans); each
// contracts its own half.  Gradient accumulators are then SH2/2 x 16 x 2 per
// wavefront, which leaves room in 256 registers for the next chunk's rows.
constexpr int kWaves2 = 8;
constexpr int kThreads2 = kWave * kWaves2;

// Input gradients in the same pass (DIN, one 16-state slice: D = 16).  After
// the contraction each wavefront forms, for its block's 16 rows and its half
// of the columns, d_h_history = [dL/dA | dL/dBv] [W_A | W_B]^T, and at a
// group's end d_h_s2 = dL/dC W_C^T for its 32-column unit: per 16-column
// tile, the transposed product (W tile rows i, k = the 32 states of A and B)
// x ([dA | dB] with k = state, column = row), three bf16 MFMAs with both
// operands split.  The weight operand comes from the staged image by
// transposed reads (lane i, four states of row i per read); [dA | dB] is
// written split to the wavefront's transposition tile as [plane][state][row]
// and read back the same way.  A lane ends with four consecutive columns of
// one row: one 128-bit store.
//
// Transposed read of four consecutive states n0 .. n0+3 of the weight image
// rows i0 .. i0+15 (i0 % 16 == 0) of weight w, plane p: lane i of a 16-lane
// group gets W_w[i0 + i][n0 + j], j = 0..3.  Image entry (q, w, p, lane L)
// holds W_w[32q + 8(L/16) + e][L % 16], e = 0..7, so lane 4j + m of the group
// addresses the 8-byte half m % 2 of entry L = n0 + j + 16((i0 % 32) / 8 +
// m / 2): rows i0 + 4m .. +3 of state n0 + j.
__device__ __forceinline__ uint2 wimage_tr(const u4 *Wl, int q, int w, int p, int i0mod32, int n0,
                                           int pl)
{
    const int m = pl & 3, j = pl >> 2;
    const int L = n0 + j + 16 * ((i0mod32 >> 3) + (m >> 1));
    const char *b = reinterpret_cast<const char *>(Wl + ((q * 3 + w) * 2 + p) * kWave + L);
    return read_tr(reinterpret_cast<const uint16_t *>(b + 8 * (m & 1)));
}

// fp32 row pitch of the staging of two 16 x 16 output tiles (32 columns and
// 16 bytes of padding)
constexpr int kStgPitch = 36;

// 128-bit stores through a buffer resource of `bytes` bytes at `base`: the
// hardware drops a store at an offset past the end, so the stores for rows
// past the batch need no branch, and the compiler's waits on the memory
// counter (which stores share with the row loads) count them exactly.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(float *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void store_b128(__amdgpu_buffer_rsrc_t r, uint32_t off, const f4 &v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, (int)off, 0, 0);
}

// KT: the scan length when fixed at compile time (the index arithmetic and
// the branches on K then fold), 0 to take it from the argument.
// MODE: kRowsBwd (weight-gradient partials), kRowsBwdDin (and the input
// gradients) or kRowsFwd (the forward: projection, forward scan, context =
// C * x_K at each sample's last row; no tile, no reverse walk).
constexpr int kRowsBwd = 0, kRowsBwdDin = 1, kRowsFwd = 2;

template <typename TIn, int NQ, int KT, int MODE>
__device__ __forceinline__ void
rows_pass(const TIn *__restrict__ hh, const TIn *__restrict__ hs2, const float *__restrict__ WA,
          const float *__restrict__ WB, const float *__restrict__ WC, int64_t B, int Kin, int D,
          int slices, int64_t groups, int64_t nrows, float a_shift,
          const float *__restrict__ dctx, float *__restrict__ part, float *__restrict__ dab_out,
          float *__restrict__ dc_out, float *__restrict__ dh_out, float *__restrict__ dhs2_out,
          const CtxOut &out)
{
    constexpr bool DIN = MODE == kRowsBwdDin;
    constexpr bool FWD = MODE == kRowsFwd;
    const int K = KT ? KT : Kin;
    constexpr int SH2 = NQ * 32;
    constexpr int NH = NQ / 2;        // units per column half
    constexpr int HC = SH2 / 2;       // columns per half
    constexpr bool LO = PBlk<TIn, NQ>::kLo;
    __shared__ u4 Wl[NQ * 6 * kWave];
    __shared__ float cvp[kWaves2][16][16];  // C partials of the current group
    __shared__ float dctl[16][16];          // d_context slice of the current group
    __shared__ float dCl[16][16];           // dL/dC = d_context * x_K
    __shared__ f4 xch[kWaves2][2][kWave];   // partial projections (A, B)
    __shared__ float bmap[4][2][16];         // per-block state maps (K >= 32)
    // per-wavefront transposition tile [plane hi|lo][row][column of the half],
    // rows padded by 8 columns so the 16 rows of a transposed read spread
    // over the banks; doubles as the raw tile of the weight staging and, at
    // the end, as the cross-wavefront sums
    constexpr int kPitch = HC + 8;
    constexpr int kPlanes = LO ? 2 : 1;
    // per-wavefront tile in bf16 elements (DIN: at least the [2][32][16] tile
    // of the split [dA | dB] and the [16][36] fp32 staging of two output tiles)
    constexpr int kTileE = kPlanes * 16 * kPitch;
    constexpr int kDinE = 16 * kStgPitch * 2;
    constexpr int kTile = DIN && kTileE < kDinE ? kDinE : kTileE;
    constexpr int kStage = FWD ? 0 : kWaves2 * kTile * 2;
    constexpr int kRed = FWD ? 0 : 2 * 2 * SH2 * 16 * 4;
    constexpr int kRaw = raw_rows_of(NQ) * 16 * 4;
    constexpr int kMem = kStage > kRed ? (kStage > kRaw ? kStage : kRaw) : (kRed > kRaw ? kRed : kRaw);
    __shared__ u4 stage_mem[kMem / 16];
    // the current group's h_s2 unit `wave`, split: [wave][plane][sample][column]
    __shared__ u4 hst_mem[FWD ? 1 : kWaves2 * kPlanes * 16 * 32 * 2 / 16];

    int64_t rho;
    int slice;
    decode_block(slices, rho, slice);
    const int s0 = slice * kSlice;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = wave_id();
    const int kg = lane >> 4, ln = lane & 15;
    const int blk = wave & 3, half = wave >> 2;
    const int kshift = __builtin_ctz((unsigned)K);  // K: a power of two <= 16, or 32, 64
    uint16_t *const tile = reinterpret_cast<uint16_t *>(stage_mem) + wave * kTile;
    uint16_t *const hst = reinterpret_cast<uint16_t *>(hst_mem) + wave * kPlanes * 16 * 32;

    f4 accA[NQ], accB[NQ], accC[2];  // i-tiles of this half; dW_C unit `wave`
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        accA[i] = zero4();
        accB[i] = zero4();
    }
    accC[0] = zero4();
    accC[1] = zero4();
    // The plain backward contracts a chunk's rows during the next chunk's
    // split and projection (PIPE): the contraction's products then issue
    // beside the split's vector work instead of in a phase of their own.
    // The chunk's [dA | dB] operands wait in registers, its split rows in
    // the wavefront's transposition tile, and the 16-column i-tiles 2u and
    // 2u + 1 are contracted just before unit u of the next chunk overwrites
    // them (LDS operations of one wavefront execute in order).  Before the
    // first chunk both the operands and the tile are zero.
    constexpr bool PIPE = !FWD && !DIN;
    GradOp pgA, pgB;
    pgA.b1 = pgA.b2 = pgB.b1 = pgB.b2 = zero_u4();
    const uint16_t *const trp = tile + (4 * kg + (ln >> 2)) * kPitch + 4 * (ln & 3);
    // contraction of i-tile tl of the rows in the tile against (gA, gB)
    auto contract_tile = [&](int tl, const GradOp &gA, const GradOp &gB)
                             __attribute__((always_inline)) {
        const uint2 h = read_tr(trp + 16 * tl);
        u4 av;
        if constexpr (LO) {
            const uint2 l = read_tr(trp + 16 * kPitch + 16 * tl);
            av = u4{h.x, h.y, l.x, l.y};
        } else {
            av = u4{h.x, h.y, h.x, h.y};
        }
        accA[tl] = contract_op<LO>(av, gA, accA[tl]);
        accB[tl] = contract_op<LO>(av, gB, accB[tl]);
    };

    auto samples_of = [&](int64_t gg) {
        return (int)(B - gg * kGroupSamples < kGroupSamples ? B - gg * kGroupSamples
                                                            : kGroupSamples);
    };
    auto advance = [&](const BTask &t) {
        BTask n = t;
        n.n = t.n + 1;
        const int nch = (samples_of(t.g) * K + kChunkRows - 1) / kChunkRows;
        if (t.c + 1 < nch) {
            n.c = t.c + 1;
        } else {
            n.g = t.g + nrows;
            n.c = 0;
            n.k = t.k + 1;
        }
        return n;
    };
    // this wavefront's half of the projection rows of a chunk (block blk)
    auto chunk_row = [&](const BTask &t) {
        const int nr = samples_of(t.g) * K;
        const int r = t.c * kChunkRows + kBlockRows * blk + ln;
        return hh + t.g * kGroupSamples * K * SH2 + (uint32_t)((r < nr ? r : nr - 1) * SH2 + HC * half);
    };
    auto load_chunk = [&](const BTask &t, PBlk<TIn, NH> &pb) { pb.load(chunk_row(t), kg); };
    // a group's h_s2 unit `wave` (C projection, dW_C) and d_context slice.
    // Loads here and in load_chunk are unconditional (clamped addresses) so
    // that every path issues the same loads and the waits for older ones
    // can leave the younger ones in flight.
    PBlk<TIn, 1> gcv;
    float gdc = 0.f;
    // need = false (the next chunk continues the current group, so nothing
    // consumes these registers): every lane reads the group's first line
    // instead, the same instructions with almost no traffic
    auto load_group = [&](int64_t gg, bool need = true) {
        // uniform 64-bit bases, 32-bit lane offsets
        const int nbb = samples_of(gg);
        const int64_t bb = gg * kGroupSamples;
        const TIn *const hsg = hs2 + bb * SH2;
        const uint32_t ho = (uint32_t)((ln < nbb ? ln : nbb - 1) * SH2 + 32 * (wave % NQ));
        gcv.load(hsg + (need ? ho : 0u), kg);
        if constexpr (!FWD) {
            const float *const dcg = dctx + bb * D + s0;
            const int bl = (tid >> 4) & 15, s = tid & 15;
            const uint32_t dofs = (uint32_t)((bl < nbb ? bl : nbb - 1) * D + s);
            gdc = dcg[need ? dofs : 0u];  // masked at use
        }
    };
    // C partials and d_context of a group into LDS (weights staged; every
    // reader of the previous group's values is past a barrier)
    auto use_group = [&](int nbb) {
        // an opaque zero keeps these lane addresses from being hoisted out of
        // the loop (and spilled): they are cheaper to recompute
        int z;
        asm volatile("s_mov_b32 %0, 0" : "=s"(z));
        const int ltid = tid + z, llane = lane + z;
        // unconditional split and product (see CvLoad::partial); the split
        // unit waits in LDS for this group's dW_C
        const Split hsS = gcv.op(0);
        if constexpr (!FWD) {
            // both halves write the same values; samples past the batch get 0
            dctl[(ltid >> 4) & 15][ltid & 15] = ((ltid >> 4) & 15) < nbb ? gdc : 0.f;
            uint16_t *const hw = hst + (llane & 15) * 32 + 8 * (llane >> 4);
            *reinterpret_cast<u4 *>(hw) = hsS.hi;
            if constexpr (LO) *reinterpret_cast<u4 *>(hw + 16 * 32) = hsS.lo;
        }
        f4 cp = mfma3<LO>(hsS, wop(Wl, wave % NQ, 2, llane), zero4());
        if (wave >= NQ) cp = zero4();
#pragma unroll
        for (int j = 0; j < 4; ++j) cvp[wave][4 * (llane >> 4) + j][llane & 15] = cp[j];
    };

    // cur: this chunk, in pb; nxt: the next one, requested into pb once this
    // chunk has been split.  One buffer and one copy of the step in the loop:
    // alternating two buffers by unrolling made the compiler alternate the
    // MFMA accumulators between two register sets.
    auto step = [&](const BTask &cur, PBlk<TIn, NH> &pb,
                    const BTask &nxt) __attribute__((always_inline)) {
        const int nb = samples_of(cur.g);
        const int NR = nb * K;
        const int nch = (NR + kChunkRows - 1) / kChunkRows;
        const int c = cur.c;
        const bool more = nxt.g < groups;
        // the rows of the next chunk's group (consumed at this step's end
        // when the next chunk starts a group; requested every step, one line
        // otherwise, so that the waits for the older rows of this chunk stay
        // exact); the next chunk's rows go out right after this chunk's
        // projection, into the registers it frees
        load_group(more ? nxt.g : cur.g, more && nxt.c == 0);
        // the first unit's weight operands (the rest follow one unit ahead)
        Split wAn = wop(Wl, half * NH, 0, lane), wBn = wop(Wl, half * NH, 1, lane);
        __syncthreads();  // last step's exchange read; this group's C partials visible
        const int cb = c * kChunkRows;
        const int ce = cb + kChunkRows < NR ? cb + kChunkRows : NR;
        const int lr0 = cb + kBlockRows * blk;

        // split this half once: projection from registers, contraction
        // transposed from the wavefront's LDS tile.  Each unit's registers
        // take the next chunk's unit as soon as it has been split (this chunk
        // again after the last).
        // The weight operands of unit u + 1 are read while unit u is split
        // and projected, so no LDS read latency sits between two units.
        const TIn *__restrict__ nrow = chunk_row(more ? nxt : cur);
        f4 pA = zero4(), pB = zero4();
#pragma unroll
        for (int u = 0; u < NH; ++u) {
            const Split wA = wAn, wB = wBn;
            if (u + 1 < NH) {
                wAn = wop(Wl, half * NH + u + 1, 0, lane);
                wBn = wop(Wl, half * NH + u + 1, 1, lane);
            }
            if constexpr (PIPE) {
                contract_tile(2 * u, pgA, pgB);
                contract_tile(2 * u + 1, pgA, pgB);
            }
            const Split sp = pb.op(u);
            pb.load_unit(nrow, kg, u);
            if constexpr (!FWD) {
                *reinterpret_cast<u4 *>(tile + ln * kPitch + 32 * u + 8 * kg) = sp.hi;
                if constexpr (LO)
                    *reinterpret_cast<u4 *>(tile + (16 + ln) * kPitch + 32 * u + 8 * kg) = sp.lo;
            }
            pA = mfma3<LO>(sp, wA, pA);
            pB = mfma3<LO>(sp, wB, pB);
            // keep later units' operand reads from being hoisted further
            __builtin_amdgcn_sched_barrier(0);
        }
        xch[wave][0][lane] = pA;
        xch[wave][1][lane] = pB;
        __syncthreads();
        const f4 aA = pA + xch[wave ^ 4][0][lane];  // same sum in both halves
        const f4 aB = pB + xch[wave ^ 4][1][lane];

        // The block starts and ends samples (K divides 16), so the scans stay
        // inside the block: a lane's four rows hold one sample's rows when
        // K >= 4, whole samples when K < 4; a sample spans kgs = K/4 lane
        // groups.  Rows past the group's end are identity steps with zero
        // gradients.  Resets are selects, never multiplications, so a
        // non-finite value stays inside its sample.
        float gate[4], gcom[4], beta[4];
        int tj[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = lr0 + 4 * kg + j;
            tj[j] = r & (K - 1);
            const bool v = r < ce;
            const Gate gg = gate_of(aA[j] + a_shift);
            gate[j] = v ? gg.g : 1.f;
            gcom[j] = gg.gc;
            beta[j] = v ? aB[j] : 0.f;
        }
        // LDS values of the walks, read up front (clamped rows; used only
        // where the row is valid): d_context at each row's sample, and
        // lambda_K = dL/dx_K = d_context * C (C from the eight wavefronts'
        // partials) of the sample of the lane's last row and, when K < 4, of
        // the sample before each row (a sample starting inside the lane)
        auto lam_k = [&](int sj, float dcs) {
            float cs = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves2; ++w) cs += cvp[w][sj][ln];
            return dcs * cs;
        };
        float dcv[4] = {0.f, 0.f, 0.f, 0.f}, lprev[4] = {0.f, 0.f, 0.f, 0.f};
        float llast = 0.f;
        if constexpr (!FWD) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sj = (lr0 + 4 * kg + j) >> kshift;
                dcv[j] = dctl[sj < 15 ? sj : 15][ln];
            }
            const int s3 = (lr0 + 4 * kg + 3) >> kshift;
            llast = lam_k(s3 < 15 ? s3 : 15, dcv[3]);
            if (K < 4) {
#pragma unroll
                for (int j = 1; j < 4; ++j) {
                    const int sj = (lr0 + 4 * kg + j) >> kshift;
                    const int sp = sj - 1 < 0 ? 0 : (sj - 1 < 15 ? sj - 1 : 15);
                    lprev[j] = lam_k(sp, dctl[sp][ln]);
                }
            }
        }

        const int kgs = K >> 2;  // lane groups per sample (K >= 8: 2, or 4 and more)
        const bool odd = kg & 1;
        const float G = gate[0] * gate[1] * gate[2] * gate[3];
        float x_in = 0.f, gsuf = 1.f;  // state entering the lane; gates of later groups
        float mx = 1.f;                // gate product of the block's earlier groups
        float tM = 1.f, tC = 0.f;      // the block's map (K >= 32)
        if (kgs > 1) {
            // forward: affine map (M, C) of the lane's rows, composed over the
            // sample's lane groups; first within pairs of groups, then (K = 16)
            // the second pair after the first pair's total
            float M = G, C = beta[0];
            C = gate[1] * C + beta[1];
            C = gate[2] * C + beta[2];
            C = gate[3] * C + beta[3];
            const RowVals pm = pair_rows(M), pc = pair_rows(C);
            if (odd) {
                C = M * pc.lo + C;
                M = M * pm.lo;
            }
            // reverse: product of the gates of the sample's later groups
            const RowVals pg = pair_rows(G);
            gsuf = odd ? 1.f : pg.hi;
            if (kgs > 2) {
                // the first pair's total (held by its odd group) into rows 2-3
                const float pM = pair_rows(M).hi, pC = pair_rows(C).hi;
                const float fM = half_rows(pM).lo, fC = half_rows(pC).lo;
                const bool second = kg >= 2;
                if (second) {
                    C = M * fC + C;
                    M = M * fM;
                }
                const RowVals qm = pair_rows(M), qc = pair_rows(C);  // (all lanes take part)
                x_in = odd ? qc.lo : (second ? fC : 0.f);
                mx = odd ? qm.lo : (second ? fM : 1.f);
                const float hP = half_rows(pg.lo * pg.hi).hi;  // the second pair's gates
                if (!second) gsuf *= hP;
                if (K >= 32) {
                    // the last group's inclusive map is the block's
                    tM = half_rows(qm.hi).hi;
                    tC = half_rows(qc.hi).hi;
                }
            } else {
                x_in = odd ? pc.lo : 0.f;
            }
        }

        if (K >= 32) {
            // a sample spans 2 or 4 blocks of the chunk: the blocks' maps
            // through LDS give the state entering this block and the gate
            // product of the sample's later blocks (samples start at chunk
            // starts, so none reaches into another chunk)
            if (half == 0 && kg == 0) {
                bmap[blk][0][ln] = tM;
                bmap[blk][1][ln] = tC;
            }
            __syncthreads();
            const int sb = lr0 >> kshift;
            float X = 0.f, Ga = 1.f;
#pragma unroll
            for (int b2 = 0; b2 < 4; ++b2) {
                const bool same = ((cb + kBlockRows * b2) >> kshift) == sb;
                const float bm = bmap[b2][0][ln], bc = bmap[b2][1][ln];
                if (same && b2 < blk) X = bm * X + bc;
                if (same && b2 > blk) Ga *= bm;
            }
            x_in = mx * X + x_in;
            gsuf *= Ga;
        }

        // forward walk: state before each row, dL/dC at sample ends
        float x = x_in;
        float xbef[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = lr0 + 4 * kg + j;
            xbef[j] = tj[j] == 0 ? 0.f : x;
            x = tj[j] == 0 ? beta[j] : gate[j] * x + beta[j];
            if (half == 0 && r < ce && tj[j] == K - 1) {
                if constexpr (FWD) {
                    // context = C * x_K (C from the eight wavefronts' partials)
                    const int sj = r >> kshift;
                    float cs = 0.f;
#pragma unroll
                    for (int w = 0; w < kWaves2; ++w) cs += cvp[w][sj][ln];
                    put_context(out, cur.g * kGroupSamples + sj, D, s0 + ln, cs * x);
                } else {
                    dCl[r >> kshift][ln] = dcv[j] * x;
                }
            }
        }
        if constexpr (FWD) {
            if (c == nch - 1) {
                __syncthreads();  // every reader of this group's C partials is done
                if (more) use_group(samples_of(nxt.g));
            }
            return;
        }
        // reverse walk: adjoint of each row's output state, entering the
        // lane's last row as lambda_K of its sample times the later gates
        float m_in = llast * gsuf;
        f4 dA4, dB4;
#pragma unroll
        for (int j = 3; j >= 0; --j) {
            const int r = lr0 + 4 * kg + j;
            const bool v = r < ce;
            const float gt = gate[j];
            dB4[j] = v ? m_in : 0.f;
            dA4[j] = v ? m_in * xbef[j] * (gt * gcom[j]) : 0.f;
            // a sample starts at row j (K < 4): the row before ends the previous one
            if (j > 0) m_in = tj[j] == 0 ? lprev[j] : gt * m_in;
        }

        if (!DIN && dab_out && half == 0) {
            // dL/dA | dL/dB of this block's rows, for the input gradients
            float *o = dab_out + (cur.g * kGroupSamples * K + lr0 + 4 * kg) * (int64_t)(2 * D) + s0 + ln;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (lr0 + 4 * kg + j < ce) {
                    o[j * 2 * D] = dA4[j];
                    o[j * 2 * D + D] = dB4[j];
                }
        }
        // weight-gradient contraction of this half over the block's 16 rows
        const GradOp gA = grad_op<LO>(dA4), gB = grad_op<LO>(dB4);
        if constexpr (PIPE) {
            pgA = gA;  // contracted during the next chunk's split
            pgB = gB;
        } else {
#pragma unroll
            for (int tl = 0; tl < NQ; ++tl) {
                contract_tile(tl, gA, gB);
                if (tl % 2 == 1) __builtin_amdgcn_sched_barrier(0);  // bounded read-ahead
            }
        }

        if constexpr (DIN) {
            // [dA | dB] split into the tile as [plane][state][row] (32-byte
            // state rows; the contraction's reads of the tile come first in
            // this wavefront's LDS order), then read back transposed: lane l
            // gets row l % 16 of states 8(l/16) .. +7 (dA for l < 32, dB after)
            const uint32_t a01 = pack_bf16(dA4[0], dA4[1]), a23 = pack_bf16(dA4[2], dA4[3]);
            const uint32_t b01 = pack_bf16(dB4[0], dB4[1]), b23 = pack_bf16(dB4[2], dB4[3]);
            *reinterpret_cast<uint2 *>(tile + ln * 16 + 4 * kg) = uint2{a01, a23};
            *reinterpret_cast<uint2 *>(tile + (16 + ln) * 16 + 4 * kg) = uint2{b01, b23};
            *reinterpret_cast<uint2 *>(tile + 512 + ln * 16 + 4 * kg) =
                uint2{pack_lo(a01, dA4[0], dA4[1]), pack_lo(a23, dA4[2], dA4[3])};
            *reinterpret_cast<uint2 *>(tile + 512 + (16 + ln) * 16 + 4 * kg) =
                uint2{pack_lo(b01, dB4[0], dB4[1]), pack_lo(b23, dB4[2], dB4[3])};
            const uint16_t *const dp = tile + (8 * kg + (ln >> 2)) * 16 + 4 * (ln & 3);
            const uint2 h0 = read_tr(dp), h1 = read_tr(dp + 64);
            const uint2 l0 = read_tr(dp + 512), l1 = read_tr(dp + 576);
            const u4 dH = {h0.x, h0.y, h1.x, h1.y}, dL = {l0.x, l0.y, l1.x, l1.y};
            const int wsel = kg >> 1, n0 = 8 * (kg & 1);
            // the group's rows; rows past the batch fall past the resource
            const __amdgpu_buffer_rsrc_t orsc =
                out_rsrc(dh_out + cur.g * kGroupSamples * K * (int64_t)SH2, (uint32_t)(NR * SH2 * 4));
            // Two tiles (32 columns: one 128-byte line of each of the 16 rows)
            // at a time pass through the tile as [row][column] fp32, so that
            // each store writes whole lines: lane l takes row l/8 (+ 8),
            // bytes 16(l % 8) .. +15 of the line.  Half-line stores left
            // part of the lines to be filled by reads from memory.
            float *const stg = reinterpret_cast<float *>(tile);
            const uint32_t ooff = ((uint32_t)(lr0 + (lane >> 3)) * SH2 + HC * half + 4 * (lane & 7)) * 4;
#pragma unroll
            for (int t = 0; t < NQ; ++t) {
                const int q = half * NH + t / 2;
                const uint2 wh0 = wimage_tr(Wl, q, wsel, 0, 16 * (t & 1), n0, ln);
                const uint2 wh1 = wimage_tr(Wl, q, wsel, 0, 16 * (t & 1), n0 + 4, ln);
                const uint2 wl0 = wimage_tr(Wl, q, wsel, 1, 16 * (t & 1), n0, ln);
                const uint2 wl1 = wimage_tr(Wl, q, wsel, 1, 16 * (t & 1), n0 + 4, ln);
                const u4 wH = {wh0.x, wh0.y, wh1.x, wh1.y}, wL = {wl0.x, wl0.y, wl1.x, wl1.y};
                f4 o = mfma_bf(wH, dL, zero4());
                o = mfma_bf(wL, dH, o);
                o = mfma_bf(wH, dH, o);
                *reinterpret_cast<f4 *>(stg + ln * kStgPitch + 16 * (t & 1) + 4 * kg) = o;
                if (t % 2 == 1) {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const f4 v = *reinterpret_cast<const f4 *>(
                            stg + ((lane >> 3) + 8 * h2) * kStgPitch + 4 * (lane & 7));
                        store_b128(orsc, ooff + (8 * h2 * SH2 + 32 * (t / 2)) * 4, v);
                    }
                    __builtin_amdgcn_sched_barrier(0);  // bounded read-ahead
                }
            }
        }

        if (c == nch - 1) {
            __syncthreads();  // dL/dC of the whole group written
            if (!DIN && dc_out && tid < 256) {
                const int bl = tid >> 4, s = tid & 15;
                if (bl < nb) dc_out[(cur.g * kGroupSamples + bl) * D + s0 + s] = dCl[bl][s];
            }
            // dW_C of unit `wave` over the group's samples (k = sample), the
            // split unit read back transposed
            f4 dc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int bl = 4 * kg + e;
                dc[e] = bl < nb ? dCl[bl][ln] : 0.f;
            }
            const GradOp gC = grad_op<LO>(dc);
            const uint16_t *const hsp = hst + (4 * kg + (ln >> 2)) * 32 + 4 * (ln & 3);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint2 h = read_tr(hsp + 16 * t);
                u4 av;
                if constexpr (LO) {
                    const uint2 l = read_tr(hsp + 16 * 32 + 16 * t);
                    av = u4{h.x, h.y, l.x, l.y};
                } else {
                    av = u4{h.x, h.y, h.x, h.y};
                }
                accC[t] = contract_op<LO>(av, gC, accC[t]);
            }
            if constexpr (DIN) {
                // d_h_s2 of unit `wave`: W_C tile (k = states 0..15, zero
                // above) x dL/dC (k = state, column = sample)
                if (wave < NQ) {
                    const bool kv = kg < 2;
                    const float *const dcr = &dCl[ln][8 * (kg & 1)];
                    float dv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) dv[e] = kv ? dcr[e] : 0.f;
                    const Split ds = split8(dv);
                    const __amdgpu_buffer_rsrc_t orsc =
                        out_rsrc(dhs2_out + cur.g * kGroupSamples * (int64_t)SH2, (uint32_t)(nb * SH2 * 4));
                    // whole-line stores through the staging, as for d_h_history
                    float *const stg = reinterpret_cast<float *>(tile);
                    const uint32_t ooff = ((uint32_t)(lane >> 3) * SH2 + 32 * wave + 4 * (lane & 7)) * 4;
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const uint2 wh0 = wimage_tr(Wl, wave, 2, 0, 16 * t, 8 * (kg & 1), ln);
                        const uint2 wh1 = wimage_tr(Wl, wave, 2, 0, 16 * t, 8 * (kg & 1) + 4, ln);
                        const uint2 wl0 = wimage_tr(Wl, wave, 2, 1, 16 * t, 8 * (kg & 1), ln);
                        const uint2 wl1 = wimage_tr(Wl, wave, 2, 1, 16 * t, 8 * (kg & 1) + 4, ln);
                        const u4 wH = kv ? u4{wh0.x, wh0.y, wh1.x, wh1.y} : zero_u4();
                        const u4 wL = kv ? u4{wl0.x, wl0.y, wl1.x, wl1.y} : zero_u4();
                        f4 o = mfma_bf(wH, ds.lo, zero4());
                        o = mfma_bf(wL, ds.hi, o);
                        o = mfma_bf(wH, ds.hi, o);
                        *reinterpret_cast<f4 *>(stg + ln * kStgPitch + 16 * t + 4 * kg) = o;
                    }
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const f4 v = *reinterpret_cast<const f4 *>(
                            stg + ((lane >> 3) + 8 * h2) * kStgPitch + 4 * (lane & 7));
                        store_b128(orsc, ooff + 8 * h2 * SH2 * 4, v);
                    }
                }
            }
            // the next group's C partials and d_context: every reader of this
            // group's values (in the walks) is past the barrier above; dCl is
            // rewritten only after the next step's first barrier
            if (more) use_group(samples_of(nxt.g));
        }
    };

    PBlk<TIn, NH> pA;
    BTask cur = {rho, 0, 0, 0};
    {
        WStage<NQ, kThreads2> wst;
        wst.load(WA, WB, WC, D, s0);
        const BTask t0 = {cur.g < groups ? cur.g : groups - 1, 0, 0, 0};
        load_group(t0.g);
        // the first chunk's rows go out in two halves, before and after the
        // weight staging (measured faster than all of them before or after)
        constexpr int kPre = NH / 2 > 0 ? NH / 2 : NH;
#pragma unroll
        for (int u = 0; u < kPre; ++u) pA.load_unit(chunk_row(t0), kg, u);
        __builtin_amdgcn_sched_barrier(0);
        wst.store(Wl, reinterpret_cast<float *>(stage_mem));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = kPre; u < NH; ++u) pA.load_unit(chunk_row(t0), kg, u);
    }
    __syncthreads();  // weights staged
    if constexpr (PIPE) {
        // the tile held the raw weights: zero it for the first chunk's
        // (empty) pending contraction
        for (int e = lane; e < kTile / 8; e += kWave)
            reinterpret_cast<u4 *>(tile)[e] = zero_u4();
    }
    if (cur.g < groups) use_group(samples_of(cur.g));
    while (cur.g < groups) {
        const BTask nxt = advance(cur);
        step(cur, pA, nxt);
        cur = nxt;
    }
    if constexpr (FWD) return;
    if constexpr (PIPE) {
#pragma unroll
        for (int tl = 0; tl < NQ; ++tl) contract_tile(tl, pgA, pgB);
    }

    // sums over the four blocks of each half: (b0 + b2) + (b1 + b3), in LDS
    // (over the transposition tiles, once every wavefront is done with its
    // own).  Layout [r][A|B][i/4][s][i%4]: a lane's four consecutive rows i
    // of one state are one 16-byte entry and a wavefront's entries one
    // contiguous KiB, so the writes and reads are 128-bit and free of bank
    // conflicts.  The workgroup partial keeps that layout ("quad" layout:
    // [which][i/4][s][i%4] over the full D); phase 2 maps it back to [i][s].
    __syncthreads();
    f4 (*const redq)[2][SH2 / 4][16] = reinterpret_cast<f4 (*)[2][SH2 / 4][16]>(stage_mem);
    auto put = [&](int r, bool add) {
#pragma unroll
        for (int tl = 0; tl < NQ; ++tl) {
            const int iq = (HC * half + 16 * tl) / 4 + kg;
            f4 &ra = redq[r][0][iq][ln];
            f4 &rb = redq[r][1][iq][ln];
            ra = add ? ra + accA[tl] : accA[tl];
            rb = add ? rb + accB[tl] : accB[tl];
        }
    };
    if (blk < 2) put(blk, false);
    __syncthreads();
    if (blk >= 2) put(blk - 2, true);
    __syncthreads();
    // this workgroup's partial: part[rho][which][i/4][s][i%4], written with
    // non-temporal stores (read once, by phase 2, from beyond the L2s: the
    // end of the kernel then has no partials to write back from L2)
    float *P = part + rho * 3 * (int64_t)SH2 * D;
    constexpr int kVec = 2 * SH2 * 16 / 4;  // f4 entries of [A|B][i/4][s]
    for (int v = tid; v < kVec; v += kThreads2) {
        const int which = v / (SH2 * 4);
        const int rem = v - which * SH2 * 4;
        const int iq = rem >> 4, s = rem & 15;
        const f4 r0 = redq[0][which][iq][s];
        const f4 r1 = redq[1][which][iq][s];
        __builtin_nontemporal_store(
            r0 + r1, reinterpret_cast<f4 *>(P + which * (int64_t)SH2 * D + ((int64_t)iq * D + s0 + s) * 4));
    }
    if (wave < NQ) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int iq = (32 * wave + 16 * t) / 4 + kg;
            __builtin_nontemporal_store(
                accC[t], reinterpret_cast<f4 *>(P + 2 * (int64_t)SH2 * D + ((int64_t)iq * D + s0 + ln) * 4));
        }
    }
}

template <typename TIn, int NQ, int KT, bool DIN>
__global__ void __launch_bounds__(kThreads2, 1)
gscan_bwd_rows_kernel(const TIn *__restrict__ hh, const TIn *__restrict__ hs2,
                      const float *__restrict__ WA, const float *__restrict__ WB,
                      const float *__restrict__ WC, int64_t B, int Kin, int D, int slices,
                      int64_t groups, int64_t nrows, float a_shift,
                      const float *__restrict__ dctx, float *__restrict__ part,
                      float *__restrict__ dab_out, float *__restrict__ dc_out,
                      float *__restrict__ dh_out, float *__restrict__ dhs2_out)
{
    rows_pass<TIn, NQ, KT, DIN ? kRowsBwdDin : kRowsBwd>(
        hh, hs2, WA, WB, WC, B, Kin, D, slices, groups, nrows, a_shift, dctx, part, dab_out,
        dc_out, dh_out, dhs2_out, CtxOut{});
}

// The forward with the per-block backward's decomposition: one persistent
// workgroup per CU, the weights staged once, 64-row chunks requested one
// chunk ahead, each 16-row block projected by two wavefronts (halves of the
// columns), then the forward scan and the context at each sample's end.
template <typename TIn, int NQ, int KT>
__global__ void __launch_bounds__(kThreads2, 1)
gscan_fwd_rows_kernel(const TIn *__restrict__ hh, const TIn *__restrict__ hs2,
                      const float *__restrict__ WA, const float *__restrict__ WB,
                      const float *__restrict__ WC, int64_t B, int Kin, int D, int slices,
                      int64_t groups, int64_t nrows, float a_shift, CtxOut out)
{
    rows_pass<TIn, NQ, KT, kRowsFwd>(hh, hs2, WA, WB, WC, B, Kin, D, slices, groups, nrows,
                                     a_shift, nullptr, nullptr, nullptr, nullptr, nullptr,
                                     nullptr, out);
}

// ======================== split backward: projection + scans, then contraction
// For wide rows (SH2 = 512, where the per-block kernel's LDS budget ends) and
// long scans the backward is split in two passes:
//   gscan_bwd_scan_kernel      projection replay, forward and reverse scans:
//                              dL/dA | dL/dBv per row ([B*K][2D] fp32) and
//                              dL/dC per sample ([B][D]) into the workspace
//   gscan_bwd_contract_kernel  the weight-gradient contractions as MFMA
//                              tiles over row slabs: h_history^T @ [dA | dB]
//                              and h_s2^T @ dC, one partial per slab
// followed by the fixed-order reduction of the partials.
//
// Scan pass.  A tile is 256 rows holding whole samples (K divides 256 and
// is a multiple of 32), so every wavefront's 32 rows (two MFMA row blocks)
// belong to one sample.  A workgroup of 8 wavefronts owns 32 states (two
// 16-state slices), keeps their A|B weights as one split image in LDS and
// walks tiles persistently; the state groups of a tile run on one XCD at
// the same time, so the tile's rows come from HBM once and from L2 for the
// other groups.  Per tile: the C values of its samples (fp32 dot products
// against W_C columns held in registers), the A|B projection of each row
// block unit by unit (row data four units ahead, running on into the next
// tile), the gates and their complements, the lane-level scans, one
// exchange of per-wavefront maps through LDS, then the walks that give
// x_t, lambda_{t+1} and the adjoints of every row.
constexpr int kPsWaves = 8;
constexpr int kPsThreads = kWave * kPsWaves;
constexpr int kPsRows = 256;       // rows per tile
constexpr int kPsStates = 32;      // states per workgroup
constexpr int kPsDepth = 4;        // units of row data in flight

// The row pointers pass through the tile loop's registers, where the
// compiler no longer sees that they address global memory; the loads name
// the address space so that they are global (not flat) loads, whose waits
// do not also wait for LDS traffic.
typedef const __attribute__((address_space(1))) f4 gf4;
typedef const __attribute__((address_space(1))) u4 gu4;

template <typename TIn, int NQ> struct PsRing;

template <int NQ> struct PsRing<float, NQ> {
    f4 v[kPsDepth][2][2];  // [slot][row block][half]
    __device__ __forceinline__ void load(const float *const *row, int kg, int q, int slot)
    {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            v[slot][rb][0] = *(gf4 *)(row[rb] + 32 * q + 8 * kg);
            v[slot][rb][1] = *(gf4 *)(row[rb] + 32 * q + 8 * kg + 4);
        }
    }
    __device__ __forceinline__ Split op(int slot, int rb) const
    {
        float x[8] = {v[slot][rb][0][0], v[slot][rb][0][1], v[slot][rb][0][2], v[slot][rb][0][3],
                      v[slot][rb][1][0], v[slot][rb][1][1], v[slot][rb][1][2], v[slot][rb][1][3]};
        return split8(x);
    }
};

template <int NQ> struct PsRing<uint16_t, NQ> {
    u4 v[kPsDepth][2];
    __device__ __forceinline__ void load(const uint16_t *const *row, int kg, int q, int slot)
    {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
            v[slot][rb] = *(gu4 *)(row[rb] + 32 * q + 8 * kg);
    }
    __device__ __forceinline__ Split op(int slot, int rb) const
    {
        Split s;
        s.hi = v[slot][rb];
        s.lo = zero_u4();
        return s;
    }
};

// workgroup -> (state group, first tile): the nsg state groups of a tile sit
// on one XCD (blockIdx % 8) next to each other
__device__ __forceinline__ void ps_decode(int nsg, int &sg, int64_t &tile0, int64_t &tstride)
{
    const int id = blockIdx.x;
    const int xcd = id % kXcds, r = id / kXcds;
    sg = r % nsg;
    tile0 = (int64_t)(r / nsg) * kXcds + xcd;
    tstride = gridDim.x / nsg;
}

// FWD: the forward over the same tiles (projection and forward scan only):
// context = C * x_K at each sample's last row into `out`; no adjoints.
template <typename TIn, int NQ, int KT, bool FWD>
__device__ __forceinline__ void scan_tiles(const TIn *__restrict__ hh, const TIn *__restrict__ hs2,
                                           const float *__restrict__ WA,
                                           const float *__restrict__ WB,
                                           const float *__restrict__ WC, int64_t ntiles, int D,
                                           float a_shift, const float *__restrict__ dctx,
                                           float *__restrict__ dab, float *__restrict__ dcv,
                                           const CtxOut &out)
{
    constexpr int SH2 = NQ * 32;
    constexpr int S = 2;
    constexpr bool LO = PBlk<TIn, NQ>::kLo;
    constexpr int NS = kPsRows / KT;   // samples per tile
    constexpr int WPS = KT / 32;       // wavefronts per sample
    constexpr int KP = SH2 / 16;       // W_C rows per thread part (C values)
    static_assert(KT % 32 == 0 && kPsRows % KT == 0, "whole samples per tile and wavefront");
    static_assert(NQ >= kPsDepth, "ring deeper than a row");
    __shared__ u4 img[S * NQ * 4 * kWave];
    __shared__ float credp[16][NS][kPsStates];     // C partials by k part
    __shared__ float cl[2][NS][kPsStates];         // C, by tile parity
    __shared__ float dcl[2][NS][kPsStates];        // d_context, by tile parity
    __shared__ float fmap[2][kPsWaves][S][2][16];  // wavefront maps (M, C), by tile parity
    __shared__ float gprod[2][kPsWaves][S][16];    // wavefront gate products, by tile parity

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = wave_id();
    const int kg = lane >> 4, ln = lane & 15;
    const int nsg = D / kPsStates;
    int sg;
    int64_t tile, tstride;
    ps_decode(nsg, sg, tile, tstride);
    const int s0 = sg * kPsStates;

    // this wavefront's rows of a tile: 32 * wave + 16 * rb + (lane % 16)
    auto rows_of = [&](int64_t t, const TIn **row) {
        const int64_t tt = t < ntiles ? t : ntiles - 1;  // past the end: a valid tile, unused
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
            row[rb] = hh + (tt * kPsRows + 32 * wave + 16 * rb + ln) * (int64_t)SH2;
    };
    PsRing<TIn, NQ> ring;
    const TIn *rcur[2];
    rows_of(tile, rcur);
#pragma unroll
    for (int q = 0; q < kPsDepth; ++q) ring.load(rcur, kg, q, q);

    // thread (cp, cs) forms the part of C over W_C rows cp*KP .. +KP-1 for
    // state s0 + cs (the W_C values come from L2 each tile)
    const int cs = tid % kPsStates, cp = tid / kPsStates;
    const float *const wcp = WC + (int64_t)(cp * KP) * D + s0 + cs;
    stage_image<NQ, S, 2>(img, WA, WB, D, s0);
    __syncthreads();

    for (int par = 0; tile < ntiles; tile += tstride, par ^= 1) {
        const int64_t bt = tile * NS;  // first sample of the tile
        // ---- C partials of the tile's samples (plain fp32 dot products)
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const TIn *hp = hs2 + (bt + j) * SH2 + cp * KP;
            float acc = 0.f;
#pragma unroll
            for (int k = 0; k < KP; ++k) {
                float hv;
                if constexpr (LO) hv = hp[k];
                else hv = __uint_as_float((uint32_t)hp[k] << 16);
                acc = fmaf(hv, wcp[(int64_t)k * D], acc);
            }
            credp[cp][j][cs] = acc;
        }

        // ---- A|Bv projection of both row blocks, both slices
        const TIn *rnxt[2];
        rows_of(tile + tstride, rnxt);
        f4 aA[S][2], aB[S][2];
#pragma unroll
        for (int sl = 0; sl < S; ++sl)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                aA[sl][rb] = zero4();
                aB[sl][rb] = zero4();
            }
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int slot = q % kPsDepth;
            const Split h0 = ring.op(slot, 0), h1 = ring.op(slot, 1);
            // the slot takes unit q + depth (of this tile, or of the next)
            if (q + kPsDepth < NQ) ring.load(rcur, kg, q + kPsDepth, slot);
            else ring.load(rnxt, kg, q + kPsDepth - NQ, slot);
#pragma unroll
            for (int sl = 0; sl < S; ++sl) {
                const Split wa = img_op(img, (sl * NQ + q) * 2, lane);
                const Split wb = img_op(img, (sl * NQ + q) * 2 + 1, lane);
                aA[sl][0] = mfma3<LO>(h0, wa, aA[sl][0]);
                aA[sl][1] = mfma3<LO>(h1, wa, aA[sl][1]);
                aB[sl][0] = mfma3<LO>(h0, wb, aB[sl][0]);
                aB[sl][1] = mfma3<LO>(h1, wb, aB[sl][1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        rcur[0] = rnxt[0];
        rcur[1] = rnxt[1];

        // ---- gates and the lane-level scans.  Row 4*kg + j of block rb.
        float gt[S][2][4], gc[S][2][4];
        Aff excl[S][2], tot[S][2];
        float gsuf[S][2], gall[S][2];
#pragma unroll
        for (int sl = 0; sl < S; ++sl)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                Aff F = aff_id();
                float G = 1.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const Gate g = gate_of(aA[sl][rb][j] + a_shift);
                    gt[sl][rb][j] = g.g;
                    gc[sl][rb][j] = g.gc;
                    Aff m = {g.g, aB[sl][rb][j], 0};
                    F = compose(m, F);
                    G *= g.g;
                }
                scan_up(F, lane, excl[sl][rb], tot[sl][rb]);
                // gate products of the later lane groups of the block, and of all four
                const RowVals pg = pair_rows(G);
                const bool odd = kg & 1;
                const float pp = pg.lo * pg.hi;
                const RowVals hp = half_rows(pp);
                gsuf[sl][rb] = (odd ? 1.f : pg.hi) * (kg < 2 ? hp.hi : 1.f);
                gall[sl][rb] = hp.lo * hp.hi;
            }
        // the wavefront's own map and gate product
        if (kg == 0) {
#pragma unroll
            for (int sl = 0; sl < S; ++sl) {
                const Aff w = compose(tot[sl][1], tot[sl][0]);
                fmap[par][wave][sl][0][ln] = w.m;
                fmap[par][wave][sl][1][ln] = w.c;
                if (!FWD) gprod[par][wave][sl][ln] = gall[sl][0] * gall[sl][1];
            }
        }
        __syncthreads();
        // ---- C and d_context of the tile's samples
        if (tid < NS * kPsStates) {
            const int j = tid / kPsStates, s = tid % kPsStates;
            float c = 0.f;
#pragma unroll
            for (int p = 0; p < 16; ++p) c += credp[p][j][s];
            cl[par][j][s] = c;
            if (!FWD) dcl[par][j][s] = dctx[(bt + j) * D + s0 + s];
        }
        __syncthreads();

        if constexpr (FWD) {
            // the forward walk of the sample's last wavefront, last lane
            // group: x_K, and context = C * x_K
            const int sj = wave / WPS, w0 = sj * WPS;
            if (wave == w0 + WPS - 1 && kg == 3) {
#pragma unroll
                for (int sl = 0; sl < S; ++sl) {
                    const int st = 16 * sl + ln;
                    float xin = 0.f;
                    for (int w2 = w0; w2 < wave; ++w2)
                        xin = fmap[par][w2][sl][0][ln] * xin + fmap[par][w2][sl][1][ln];
                    const float x = apply(tot[sl][1], apply(tot[sl][0], xin));
                    put_context(out, bt + sj, D, s0 + st, cl[par][sj][st] * x);
                }
            }
            continue;
        }

        // ---- cross-wavefront folds, walks, adjoints
        const int sj = wave / WPS;            // sample of this wavefront in the tile
        const int w0 = sj * WPS;              // its first wavefront
        const int64_t row0 = tile * kPsRows + 32 * wave;
#pragma unroll
        for (int sl = 0; sl < S; ++sl) {
            const int st = 16 * sl + ln;      // state within the group
            // state entering the wavefront: earlier wavefronts of the sample
            float xin = 0.f;
            for (int w2 = w0; w2 < wave; ++w2)
                xin = fmap[par][w2][sl][0][ln] * xin + fmap[par][w2][sl][1][ln];
            // adjoint entering the wavefront's last row: lambda_K times the
            // gates of the sample's later wavefronts
            float lin = dcl[par][sj][st] * cl[par][sj][st];
            for (int w2 = wave + 1; w2 < w0 + WPS; ++w2) lin *= gprod[par][w2][sl][ln];
            float xbef[2][4];
            float x = apply(excl[sl][0], xin);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                if (rb == 1) x = apply(excl[sl][1], apply(tot[sl][0], xin));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    xbef[rb][j] = x;
                    x = gt[sl][rb][j] * x + aB[sl][rb][j];
                }
            }
            // the sample's last row (block 1, lane group 3, j = 3): dL/dC
            if (wave == w0 + WPS - 1 && kg == 3)
                dcv[(bt + sj) * D + s0 + st] = dcl[par][sj][st] * x;
#pragma unroll
            for (int rb = 1; rb >= 0; --rb) {
                float mu = lin * gsuf[sl][rb] * (rb == 0 ? gall[sl][1] : 1.f);
                float *o = dab + (row0 + 16 * rb + 4 * kg) * (int64_t)(2 * D) + s0 + st;
#pragma unroll
                for (int j = 3; j >= 0; --j) {
                    o[j * 2 * D + D] = mu;                                              // dL/dBv
                    o[j * 2 * D] = mu * xbef[rb][j] * (gt[sl][rb][j] * gc[sl][rb][j]);  // dL/dA
                    mu = gt[sl][rb][j] * mu;
                }
            }
        }
    }
}

template <typename TIn, int NQ, int KT>
__global__ void __launch_bounds__(kPsThreads, 1)
gscan_bwd_scan_kernel(const TIn *__restrict__ hh, const TIn *__restrict__ hs2,
                      const float *__restrict__ WA, const float *__restrict__ WB,
                      const float *__restrict__ WC, int64_t ntiles, int D, float a_shift,
                      const float *__restrict__ dctx, float *__restrict__ dab,
                      float *__restrict__ dcv)
{
    scan_tiles<TIn, NQ, KT, false>(hh, hs2, WA, WB, WC, ntiles, D, a_shift, dctx, dab, dcv,
                                   CtxOut{});
}

// The forward over 256-row tiles of whole samples, 32 states per workgroup:
// the scan pass's projection and forward scan, ending in the context.
template <typename TIn, int NQ, int KT>
__global__ void __launch_bounds__(kPsThreads, 1)
gscan_fwd_tile_kernel(const TIn *__restrict__ hh, const TIn *__restrict__ hs2,
                      const float *__restrict__ WA, const float *__restrict__ WB,
                      const float *__restrict__ WC, int64_t ntiles, int D, float a_shift,
                      CtxOut out)
{
    scan_tiles<TIn, NQ, KT, true>(hh, hs2, WA, WB, WC, ntiles, D, a_shift, nullptr, nullptr,
                                  nullptr, out);
}

// ---- contraction: part[slab][which0 + o / D][i][o % D] = sum over the
// slab's rows r of X[r][i] * Y[r][o], for i in [m0, m0 + MT), o in
// [n0, n0 + NT).  32 rows per step: both tiles are split into bf16 high /
// low planes in LDS (row-major, rows padded by 16 columns) and read back
// transposed with ds_read_b64_tr_b16, so lane l gets column l % 16 of rows
// 4(l/16) .. +3 and 16 + 4(l/16) .. +3: the MFMA k index 8(l/16) + e for
// both operands.  The eight wavefronts form a WM x WN grid over the tile.
// Two register sets hold the rows of the next two steps, so a step's loads
// have two steps of compute to arrive; double-buffered LDS, one barrier per
// step.
constexpr int kCtThreads = 512;
constexpr int kCtRows = 32;

// WHICH0: the partial the first output column goes to (0: dW_A, then dW_B;
// 2: dW_C), fixed at compile time so that the two launches are told apart
// in profiles.
template <typename TX, int MT, int NT, int WN, bool OVL>
__device__ __forceinline__ void
contract_slab(const TX *__restrict__ X, int ldx, const float *__restrict__ Y, int ldy,
              int64_t rows, int64_t rows_per_slab, int D, int SH2, float *__restrict__ part,
              int which0, int64_t slab, int mt, int nt)
{
    constexpr bool LO = !std::is_same<TX, uint16_t>::value;
    constexpr int kPl = LO ? 2 : 1;               // planes of X
    // LDS row pitches (bf16): a transposed read takes 32 bytes of each of
    // four rows per 16 lanes, so rows start 32 bytes apart on the banks
    constexpr int PX = MT + 16, PY = NT + 16;
    constexpr int WM = 8 / WN;                    // wavefront grid WM x WN
    constexpr int MTW = MT / 16 / WM;             // m tiles per wavefront
    constexpr int NTW = NT / 16 / WN;             // n tiles per wavefront
    constexpr int XV = kCtRows * MT / (LO ? 4 : 8) / kCtThreads;  // X pieces per thread
    constexpr int YV = kCtRows * NT / 4 / kCtThreads;             // Y pieces per thread
    static_assert(XV >= 1 && YV >= 1 && MTW >= 1 && NTW >= 1, "tile split");
    __shared__ uint16_t xs[2][kPl][kCtRows][PX];
    __shared__ uint16_t ys[2][2][kCtRows][PY];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = wave_id();
    const int kg = lane >> 4, ln = lane & 15;
    const int wm = wave % WM, wn = wave / WM;
    const int m0 = mt * MT, n0 = nt * NT;
    const int64_t r_begin = slab * rows_per_slab;
    const int64_t r_end = r_begin + rows_per_slab < rows ? r_begin + rows_per_slab : rows;

    typedef typename std::conditional<LO, f4, u4>::type xraw_t;
    xraw_t xvs[2][XV];
    f4 yvs[2][YV];
    constexpr int XCOLS = LO ? MT / 4 : MT / 8;   // pieces per X row
    // a step's rows through buffer resources that end where the slab's last
    // row ends: a uniform base, 32-bit lane offsets (the same every step),
    // and rows past the end read as zeros with no branch.  (A tile that runs
    // past the row's columns reads the next row's first columns, never past
    // the slab.)
    auto load = [&](int set, int64_t rb) {
        const int64_t left = r_end - rb;
        const uint32_t nv = (uint32_t)(left < kCtRows ? (left > 0 ? left : 0) : kCtRows);
        const int xn = nv ? (int)((nv * ldx - m0) * sizeof(TX)) : 0;
        const int yn = nv ? (int)((nv * ldy - n0) * 4) : 0;
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<TX *>(X + rb * ldx + m0), (short)0, xn, 0x00020000);
        const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(Y + rb * ldy + n0), (short)0, yn, 0x00020000);
#pragma unroll
        for (int u = 0; u < XV; ++u) {
            const int e = tid + kCtThreads * u;
            const int r = e / XCOLS, c = e % XCOLS;
            const uint32_t off = (uint32_t)(r * ldx + (LO ? 4 : 8) * c) * (uint32_t)sizeof(TX);
            xvs[set][u] = __builtin_bit_cast(xraw_t, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < YV; ++u) {
            const int e = tid + kCtThreads * u;
            const int r = e / (NT / 4), c = e % (NT / 4);
            const uint32_t off = (uint32_t)(r * ldy + 4 * c) * 4u;
            yvs[set][u] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(ry, (int)off, 0, 0));
        }
    };
    auto store = [&](int set, int buf) {
#pragma unroll
        for (int u = 0; u < XV; ++u) {
            const int e = tid + kCtThreads * u;
            const int r = e / XCOLS, c = e % XCOLS;
            if constexpr (LO) {
                const f4 x = xvs[set][u];
                const uint32_t h01 = pack_bf16(x[0], x[1]), h23 = pack_bf16(x[2], x[3]);
                const uint32_t l01 = pack_lo(h01, x[0], x[1]);
                const uint32_t l23 = pack_lo(h23, x[2], x[3]);
                *reinterpret_cast<uint2 *>(&xs[buf][0][r][4 * c]) = uint2{h01, h23};
                *reinterpret_cast<uint2 *>(&xs[buf][kPl - 1][r][4 * c]) = uint2{l01, l23};
            } else {
                *reinterpret_cast<u4 *>(&xs[buf][0][r][8 * c]) = xvs[set][u];
            }
        }
#pragma unroll
        for (int u = 0; u < YV; ++u) {
            const int e = tid + kCtThreads * u;
            const int r = e / (NT / 4), c = e % (NT / 4);
            const f4 y = yvs[set][u];
            const uint32_t h01 = pack_bf16(y[0], y[1]), h23 = pack_bf16(y[2], y[3]);
            const uint32_t l01 = pack_lo(h01, y[0], y[1]);
            const uint32_t l23 = pack_lo(h23, y[2], y[3]);
            *reinterpret_cast<uint2 *>(&ys[buf][0][r][4 * c]) = uint2{h01, h23};
            *reinterpret_cast<uint2 *>(&ys[buf][1][r][4 * c]) = uint2{l01, l23};
        }
    };
    // transposed operand: column c + ln of rows 4kg..+3 and 16 + 4kg..+3
    auto operand = [&](const uint16_t *tile, int pitch, int c) {
        const uint16_t *p = tile + (4 * kg + (ln >> 2)) * pitch + c + 4 * (ln & 3);
        const uint2 a = read_tr(p), b = read_tr(p + 16 * pitch);
        return u4{a.x, a.y, b.x, b.y};
    };

    f4 acc[MTW][NTW];
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[i][j] = zero4();

    auto contract = [&](int buf) {
        Split bo[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int c = 16 * (NTW * wn + j);
            bo[j].hi = operand(&ys[buf][0][0][0], PY, c);
            bo[j].lo = operand(&ys[buf][1][0][0], PY, c);
        }
#pragma unroll
        for (int i = 0; i < MTW; ++i) {
            const int c = 16 * (MTW * wm + i);
            Split ao;
            ao.hi = operand(&xs[buf][0][0][0], PX, c);
            ao.lo = LO ? operand(&xs[buf][kPl - 1][0][0], PX, c) : zero_u4();
#pragma unroll
            for (int j = 0; j < NTW; ++j) acc[i][j] = mfma3<LO>(ao, bo[j], acc[i][j]);
        }
    };
    // OVL: step k contracts LDS buffer k % 2 and, in the same stretch,
    // splits the rows of step k + 1 (register set (k + 1) % 2) into the
    // other buffer, so that the split's vector work issues beside the
    // products; the set then takes the rows of step k + 3.  The barrier at
    // the end of step k publishes buffer (k + 1) % 2 and closes the reads of
    // buffer k % 2, which step k + 1 refills.  Its extra barrier before the
    // first step costs more than the overlap gains on short slabs, where
    // step k instead splits its own rows (set k % 2) into buffer k % 2, the
    // barrier publishes them (and closes the reads of step k - 1), the set
    // takes the rows of step k + 2, and the buffer is contracted.  Rows past
    // the slab load as zeros.
    if (!OVL && r_begin < r_end) {
        load(0, r_begin);
        load(1, r_begin + kCtRows);
        for (int64_t rb = r_begin; rb < r_end; rb += 2 * kCtRows) {
            store(0, 0);
            __syncthreads();
            load(0, rb + 2 * kCtRows);
            contract(0);
            if (rb + kCtRows >= r_end) break;
            store(1, 1);
            __syncthreads();
            load(1, rb + 3 * kCtRows);
            contract(1);
        }
    }
    if (OVL && r_begin < r_end) {
        load(0, r_begin);
        load(1, r_begin + kCtRows);
        store(0, 0);
        load(0, r_begin + 2 * kCtRows);
        __syncthreads();
        for (int64_t rb = r_begin; rb < r_end; rb += 2 * kCtRows) {
            store(1, 1);
            load(1, rb + 3 * kCtRows);
            contract(0);
            __syncthreads();
            if (rb + kCtRows >= r_end) break;
            store(0, 0);
            load(0, rb + 4 * kCtRows);
            contract(1);
            __syncthreads();
        }
    }
    // partial of this slab: lane l holds i = m-tile row 4(l/16) + e, o = l % 16.
    // A tile that runs past SH2 or past the ldy columns of Y (shapes outside
    // the fused kernels) read neighbouring rows' values or zeros there; those
    // land only in the entries it does not store.
    float *P = part + slab * 3 * (int64_t)SH2 * D;
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int o = n0 + 16 * (NTW * wn + j) + ln;
            if (o >= ldy) continue;
            const int which = which0 + o / D, s = o % D;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ii = m0 + 16 * (MTW * wm + i) + 4 * kg + e;
                if (ii < SH2) P[((int64_t)which * SH2 + ii) * D + s] = acc[i][j][e];
            }
        }
}

template <typename TX, int MT, int NT, int WN, int WHICH0>
__global__ void __launch_bounds__(kCtThreads, 1)
gscan_bwd_contract_kernel(const TX *__restrict__ X, int ldx, const float *__restrict__ Y, int ldy,
                          int64_t rows, int64_t rows_per_slab, int D, int SH2,
                          float *__restrict__ part)
{
    contract_slab<TX, MT, NT, WN, true>(X, ldx, Y, ldy, rows, rows_per_slab, D, SH2, part, WHICH0,
                                        blockIdx.x, blockIdx.y, blockIdx.z);
}

// Both contractions of the materialised-projection path in one launch, on
// the same tile shape: workgroup (slab, m tile, n tile), slab slowest, takes
// that tile of h_history^T [dA | dB] (job 0, partials 0 and 1) and then,
// where job 1 has the same tile (its outputs are the first D of job 0's
// 2D), that tile of h_s2^T dC (partial 2) over the slab's samples: one
// workgroup per CU and no second round for the small job.
struct CtJob {
    const void *X;
    int ldx;
    const float *Y;
    int ldy;
    int64_t rows, rps;
    int which0, gm, gn;
};

template <typename TX, int MT, int NT>
__global__ void __launch_bounds__(kCtThreads, 1)
gscan_gen_contract_kernel(CtJob j0, CtJob j1, int D, int SH2, float *__restrict__ part)
{
    const int per = j0.gm * j0.gn;
    const int64_t slab = blockIdx.x / per;
    const int r = (int)(blockIdx.x - slab * per);
    const int mt = r / j0.gn, nt = r % j0.gn;
    contract_slab<TX, MT, NT, 4, false>(static_cast<const TX *>(j0.X), j0.ldx, j0.Y, j0.ldy, j0.rows,
                                 j0.rps, D, SH2, part, j0.which0, slab, mt, nt);
    if (nt < j1.gn) {  // the same for every thread of the workgroup
        __syncthreads();  // the tiles' LDS buffers are read to the end first
        contract_slab<TX, MT, NT, 4, false>(static_cast<const TX *>(j1.X), j1.ldx, j1.Y, j1.ldy,
                                     j1.rows, j1.rps, D, SH2, part, j1.which0, slab, mt, nt);
    }
}

// ================================================= phase 2: partial reduction
// Workgroup = 32 consecutive gradient entries; thread (seg, quad) sums rows
// r = seg, seg+16, ... of four consecutive entries, eight rows in flight at
// a time; the 16 row segments are then added in segment order.  Fixed order,
// so bitwise reproducible.
constexpr int kRedCols = 32;
// 128 threads (16 row segments): a workgroup this small finds room on a CU
// while the phase-1 workgroups there are still draining
constexpr int kRedThreads = 128;
constexpr int kRedSegs = kRedThreads / (kRedCols / 4);

__global__ void __launch_bounds__(kRedThreads)
gscan_reduce_kernel(const float *__restrict__ part, int64_t nrows, int64_t wsz, int D, int qlay,
                    float *__restrict__ dWA, float *__restrict__ dWB, float *__restrict__ dWC)
{
    __shared__ double red[kRedSegs][kRedCols];
    const int t = threadIdx.x;
    const int quad = t % (kRedCols / 4), seg = t / (kRedCols / 4);
    const int64_t per = 3 * wsz;
    const int64_t o = (int64_t)blockIdx.x * kRedCols + 4 * quad;
    double s[4] = {0.0, 0.0, 0.0, 0.0};
    const float *p = part + o;
    int64_t r = seg;
    for (; r + 7 * kRedSegs < nrows; r += 8 * kRedSegs) {
        f4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f4 *>(p + (r + u * kRedSegs) * per);
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) s[i] += (double)v[u][i];
    }
    for (; r < nrows; r += kRedSegs) {
        const f4 v = *reinterpret_cast<const f4 *>(p + r * per);
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] += (double)v[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) red[seg][4 * quad + i] = s[i];
    __syncthreads();
    if (t < kRedCols) {
        double v = 0.0;
#pragma unroll
        for (int sg = 0; sg < kRedSegs; ++sg) v += red[sg][t];
        const int64_t oo = (int64_t)blockIdx.x * kRedCols + t;
        const int64_t which = oo / wsz, e = oo - which * wsz;
        float *out = which == 0 ? dWA : (which == 1 ? dWB : dWC);
        // quad layout [i/4][s][i%4] -> [i][s]
        const int64_t q = e >> 2;
        const int64_t eo = qlay ? ((q / D) * 4 + (e & 3)) * D + q % D : e;
        out[eo] = (float)v;
    }
}

// Exact adjoints per (sample, state) from stored projections, in place:
// ab [B*K][2D] holds A | Bv on entry and dL/dA | dL/dB on exit; cv [B][D]
// holds C on entry and dL/dC on exit.  The forward pass keeps x_t in the Bv
// slot (Bv_t is not needed once x_{t+1} is known); the reverse pass reads A_t
// and x_t and overwrites both slots.  Used where samples cross the backward
// kernel's chunks (its per-row adjoints there are provisional).
__global__ void __launch_bounds__(kThreads)
gscan_adjoint_kernel(float *__restrict__ ab, float *__restrict__ cv,
                     const float *__restrict__ dctx, int64_t B, int64_t K, int D, float a_shift)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= B * D) return;
    const int64_t b = i / D;
    const int s = (int)(i - b * D);
    float *base = ab + b * K * 2 * D + s;
    // Steps in chunks of kC: a chunk's loads all go out before its stores
    // (which overwrite slots the chunk has already read), so the loads of
    // a chunk are in flight together instead of one step at a time.
    constexpr int kC = 8;
    float x = 0.f;
    for (int64_t t0 = 0; t0 < K; t0 += kC) {
        const int n = K - t0 < kC ? (int)(K - t0) : kC;
        float av[kC], bv[kC];
#pragma unroll
        for (int u = 0; u < kC; ++u) {
            if (u < n) {
                const float *row = base + (t0 + u) * 2 * D;
                av[u] = row[0];
                bv[u] = row[D];
            }
        }
#pragma unroll
        for (int u = 0; u < kC; ++u) {
            if (u < n) {
                const float g = sigmoid(av[u] + a_shift);
                base[(t0 + u) * 2 * D + D] = x;  // x_t
                x = g * x + bv[u];
            }
        }
    }
    const float d = dctx[i];
    float lam = d * cv[i];
    cv[i] = d * x;  // dL/dC = d_context * x_K
    for (int64_t t1 = K; t1 > 0; t1 -= kC) {
        const int n = t1 < kC ? (int)t1 : kC;
        const int64_t t0 = t1 - n;
        float av[kC], xv[kC];
#pragma unroll
        for (int u = 0; u < kC; ++u) {
            if (u < n) {
                const float *row = base + (t0 + u) * 2 * D;
                av[u] = row[0];
                xv[u] = row[D];
            }
        }
#pragma unroll
        for (int u = kC - 1; u >= 0; --u) {
            if (u < n) {
                float *row = base + (t0 + u) * 2 * D;
                const Gate gg = gate_of(av[u] + a_shift);
                row[D] = lam;                           // dL/dBv_t
                row[0] = lam * xv[u] * (gg.g * gg.gc);  // dL/dA_t
                lam = gg.g * lam;
            }
        }
    }
}

// ===================================================== input gradients
// out[r][i] = sum_k in[r][k] * Wk(k, i) over k < KD, where Wk(k, i) is
// W1[i][k] for k < D1 and W2[i][k - D1] otherwise: d_h_history from
// [dL/dA | dL/dB] rows (W1 = W_A, W2 = W_B, KD = 2D) and d_h_s2 from dL/dC rows
// (W1 = W_C, KD = D).  Computed transposed on the matrix cores, outᵀ tile =
// Wkᵀ tile x inᵀ tile, so a lane ends with four consecutive columns of one
// row (one 128-bit store).  Both operands fp32, split hi/lo (3 bf16 MFMA per
// product).  A workgroup stages the split weights of CT column tiles for all
// k (zero past KD) in LDS, then walks 64-row tiles (16 rows per wavefront).
//
// The same loop serves the projections of Forward Step 1 where they are
// written out (shapes outside the fused kernels): WT = kWProj reads the
// weights the other way round, Wk(k, o) = W1[k][o] for o < D1 and
// W2[k][o - D1] otherwise ([A | Bv] = h_history [W_A | W_B], C = h_s2 W_C),
// and the rows may be bf16 (exact in the high half: 2 MFMA per product).
constexpr int kDinRows = 64;
constexpr int64_t kDinMaxWorkgroups = 512;  // persistent workgroups over all column slices
constexpr int kWDin = 0, kWProj = 1;

template <typename TIn, int CT, int WT>
__device__ __forceinline__ void
rows_by_weights(const TIn *__restrict__ in, const float *__restrict__ W1,
                const float *__restrict__ W2, int D1, int KD, int NOUT, int64_t nrows,
                float *__restrict__ out, int64_t bid, int64_t nblk)
{
    constexpr bool LO = !std::is_same<TIn, uint16_t>::value;
    extern __shared__ u4 img[];  // [kc][ct][hi, lo][lane]
    __shared__ float stg[kWaves][16][kStgPitch];  // per-wavefront output staging
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kg = lane >> 4, ln = lane & 15;
    const int nkc = (KD + 31) / 32;
    // 1-D persistent grid of (row tile, column slice) pairs, XCD-aware: the
    // slices of one row tile run on one XCD at about the same time, so the
    // tile comes from HBM once and from that XCD's L2 for the other slices.
    // bid: this workgroup's index among the nblk of its launch (or of its
    // part of a launch, which starts at a multiple of the XCD count).
    const int nsl = NOUT / (16 * CT);
    const int64_t rest = bid / kXcds;
    const int slice = (int)(rest % nsl);
    const int64_t t0 = (rest / nsl) * kXcds + bid % kXcds;
    const int64_t tstride = nblk / nsl;
    const int c0 = slice * CT * 16;
    for (int e0 = tid; e0 < nkc * CT * kWave; e0 += kThreads) {
        const int l = e0 & (kWave - 1), ct = (e0 / kWave) % CT, kc = e0 / kWave / CT;
        const int i = c0 + 16 * ct + (l & 15);
        const int k = 32 * kc + 8 * (l >> 4);  // eight k on one side of D1 (D1 % 16 == 0)
        float v[8];
        if (k < KD) {
            if constexpr (WT == kWDin) {
                const float *src = k < D1 ? W1 + (int64_t)i * D1 + k
                                          : W2 + (int64_t)i * (KD - D1) + (k - D1);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = src[e];
            } else {
                // eight k of one output column; KD % 16 == 0 keeps them < KD
                const float *src = i < D1 ? W1 + (int64_t)k * D1 + i
                                          : W2 + (int64_t)k * (NOUT - D1) + (i - D1);
                const int pitch = i < D1 ? D1 : NOUT - D1;
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = src[(int64_t)e * pitch];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.f;
        }
        const Split sp = split8(v);
        img[((kc * CT + ct) * 2 + 0) * kWave + l] = sp.hi;
        img[((kc * CT + ct) * 2 + 1) * kWave + l] = sp.lo;
    }
    __syncthreads();
    const int64_t tiles = (nrows + kDinRows - 1) / kDinRows;
    // the row's k chunks in groups of kG, the next group's loads issued
    // before the current group's products
    constexpr int kG = 4;
    typedef typename std::conditional<LO, f4, u4>::type raw_t;
    constexpr int kPieces = LO ? 2 : 1;  // 16-byte pieces per chunk and lane
    const int ngr = (nkc + kG - 1) / kG;
    // the lane's row in tile t (clamped to the last row)
    auto row_of = [&](int64_t t) {
        const int64_t r = t * kDinRows + 16 * wave + ln;
        return in + (r < nrows ? r : nrows - 1) * (int64_t)KD;
    };
    auto load_group = [&](raw_t (&v)[kG][kPieces], const TIn *rowp, int g) {
#pragma unroll
        for (int u = 0; u < kG; ++u) {
            const int k = 32 * (g * kG + u) + 8 * kg;
            const TIn *src = rowp + (k < KD ? k : 0);
#pragma unroll
            for (int h = 0; h < kPieces; ++h)
                v[u][h] = *reinterpret_cast<const raw_t *>(src + h * (16 / sizeof(TIn)));
        }
    };
    raw_t cur[kG][kPieces], nxt[kG][kPieces];
    if (t0 < tiles) load_group(cur, row_of(t0), 0);
    for (int64_t t = t0; t < tiles; t += tstride) {
        const int64_t r = t * kDinRows + 16 * wave + ln;
        const TIn *rowp = row_of(t);
        f4 acc[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[ct] = zero4();
        for (int g = 0; g < ngr; ++g) {
            // the next group of this tile, or the first of the next tile
            if (g + 1 < ngr) load_group(nxt, rowp, g + 1);
            else if (t + tstride < tiles) load_group(nxt, row_of(t + tstride), 0);
#pragma unroll
            for (int u = 0; u < kG; ++u) {
                const int kc = g * kG + u;
                if (kc >= nkc) break;
                const bool kin = 32 * kc + 8 * kg < KD;
                Split hs;
                if constexpr (LO) {
                    const f4 a = cur[u][0], b = cur[u][kPieces - 1];
                    float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = kin ? x[e] : 0.f;
                    hs = split8(x);
                } else {
                    hs.hi = kin ? cur[u][0] : zero_u4();
                    hs.lo = zero_u4();
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    Split w;
                    w.hi = img[((kc * CT + ct) * 2 + 0) * kWave + lane];
                    w.lo = img[((kc * CT + ct) * 2 + 1) * kWave + lane];
                    if constexpr (LO) {
                        acc[ct] = mfma3<true>(w, hs, acc[ct]);
                    } else {
                        acc[ct] = mfma_bf(w.lo, hs.hi, acc[ct]);
                        acc[ct] = mfma_bf(w.hi, hs.hi, acc[ct]);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < kG; ++u)
#pragma unroll
                for (int h = 0; h < kPieces; ++h) cur[u][h] = nxt[u][h];
        }
        if constexpr (CT == 1) {
            if (r < nrows) *reinterpret_cast<f4 *>(out + r * NOUT + c0 + 4 * kg) = acc[0];
        } else {
            // two column tiles (one 128-byte line of each row) at a time
            // through LDS, so that every store writes whole lines: lane l
            // takes row l/8 (+ 8), bytes 16(l % 8) .. +15 of the line
            float *const sg = &stg[wave][0][0];
            const int64_t r0 = t * kDinRows + 16 * wave + (lane >> 3);
#pragma unroll
            for (int cp = 0; cp < CT / 2; ++cp) {
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    *reinterpret_cast<f4 *>(sg + ln * kStgPitch + 16 * u + 4 * kg) = acc[2 * cp + u];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const f4 v = *reinterpret_cast<const f4 *>(
                        sg + ((lane >> 3) + 8 * h2) * kStgPitch + 4 * (lane & 7));
                    const int64_t rr = r0 + 8 * h2;
                    if (rr < nrows)
                        *reinterpret_cast<f4 *>(out + rr * NOUT + c0 + 32 * cp + 4 * (lane & 7)) = v;
                }
            }
        }
    }
}

// WHICH only names the launch in profiles: 0 for d_h_history, 1 for d_h_s2
template <int CT, int WHICH>
__global__ void __launch_bounds__(kThreads)
gscan_dinput_kernel(const float *__restrict__ in, const float *__restrict__ W1,
                    const float *__restrict__ W2, int D1, int KD, int SH2, int64_t nrows,
                    float *__restrict__ out)
{
    rows_by_weights<float, CT, kWDin>(in, W1, W2, D1, KD, SH2, nrows, out, blockIdx.x, gridDim.x);
}

// WHICH: 0 for [A | Bv] from h_history, 1 for C from h_s2 (profile names)
template <typename TIn, int CT, int WHICH>
__global__ void __launch_bounds__(kThreads)
gscan_proj_kernel(const TIn *__restrict__ in, const float *__restrict__ W1,
                  const float *__restrict__ W2, int D1, int KD, int NOUT, int64_t nrows,
                  float *__restrict__ out)
{
    rows_by_weights<TIn, CT, kWProj>(in, W1, W2, D1, KD, NOUT, nrows, out, blockIdx.x,
                                     gridDim.x);
}

// Both projections of Forward Step 1 in one launch: workgroups [0, nwg0)
// form [A | Bv] (job 0, CT0 output tiles per slice), the rest C (job 1,
// CT1), so that the small C projection runs beside the large one instead
// of after it.
struct ProjJob {
    const void *in;
    const float *W1, *W2;
    int D1, KD, NOUT;
    int64_t nrows;
    float *out;
};

template <typename TIn, int CT0, int CT1>
__global__ void __launch_bounds__(kThreads)
gscan_proj2_kernel(ProjJob j0, ProjJob j1, int64_t nwg0)
{
    const int64_t b = blockIdx.x;
    if (b < nwg0)
        rows_by_weights<TIn, CT0, kWProj>(static_cast<const TIn *>(j0.in), j0.W1, j0.W2, j0.D1,
                                          j0.KD, j0.NOUT, j0.nrows, j0.out, b, nwg0);
    else
        rows_by_weights<TIn, CT1, kWProj>(static_cast<const TIn *>(j1.in), j1.W1, j1.W2, j1.D1,
                                          j1.KD, j1.NOUT, j1.nrows, j1.out, b - nwg0,
                                          (int64_t)gridDim.x - nwg0);
}

// ----------------------------------------------------------------- dispatch
template <typename TIn, int NQ>
hipError_t fwd_launch(const Plan &p, const void *hh, const void *hs2, const float *WA,
                      const float *WB, const float *WC, float a_shift, const CtxOut &ctx,
                      hipStream_t st)
{
    if constexpr (NQ <= 8) {
        if (p.fwd_perblock) {
            auto go = [&](auto kern) {
                hipLaunchKernelGGL(kern, dim3((unsigned)p.bwd_grid), dim3(kThreads2), 0, st,
                                   static_cast<const TIn *>(hh), static_cast<const TIn *>(hs2), WA,
                                   WB, WC, p.B, (int)p.K, (int)p.D, p.slices, p.groups,
                                   p.bwd_rows, a_shift, ctx);
                return hipGetLastError();
            };
            if (p.K == 8) return go(gscan_fwd_rows_kernel<TIn, NQ, 8>);
            return go(gscan_fwd_rows_kernel<TIn, NQ, 0>);
        }
    }
    if (p.fwd_tile) {
        const int64_t ntiles = p.B * p.K / kPsRows;
        auto go = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3((unsigned)p.ps_grid), dim3(kPsThreads), 0, st,
                               static_cast<const TIn *>(hh), static_cast<const TIn *>(hs2), WA,
                               WB, WC, ntiles, (int)p.D, a_shift, ctx);
            return hipGetLastError();
        };
        if constexpr (NQ == 8 || NQ == 16) {
            if (p.K == 64) return go(gscan_fwd_tile_kernel<TIn, NQ, 64>);
            if (p.K == 256) return go(gscan_fwd_tile_kernel<TIn, NQ, 256>);
        }
        return hipErrorInvalidValue;
    }
    if (p.fwd_ms == 4) {
        if constexpr (4 * NQ <= 32) {
            hipLaunchKernelGGL((gscan_fwd_ms_kernel<TIn, NQ, 4>), dim3((unsigned)p.fwd_grid),
                               dim3(kThreadsM), 0, st, static_cast<const TIn *>(hh),
                               static_cast<const TIn *>(hs2), WA, WB, WC, p.B, (int)p.K,
                               (int)p.D, p.slices / 4, p.groups, a_shift, ctx);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    if (p.fwd_ms == 2) {
        hipLaunchKernelGGL((gscan_fwd_ms_kernel<TIn, NQ, 2>), dim3((unsigned)p.fwd_grid),
                           dim3(kThreadsM), 0, st, static_cast<const TIn *>(hh),
                           static_cast<const TIn *>(hs2), WA, WB, WC, p.B, (int)p.K, (int)p.D,
                           p.slices / 2, p.groups, a_shift, ctx);
        return hipGetLastError();
    }
    if (p.fwd_prow < p.fwd_rows)
        hipLaunchKernelGGL((gscan_fwd_persist_kernel<TIn, NQ>), dim3((unsigned)p.fwd_grid),
                           dim3(kThreads), 0, st, static_cast<const TIn *>(hh),
                           static_cast<const TIn *>(hs2), WA, WB, WC, p.B, (int)p.K, (int)p.D,
                           p.slices, p.groups, p.fwd_prow, a_shift, ctx);
    else
        hipLaunchKernelGGL((gscan_fwd_kernel<TIn, NQ>), dim3((unsigned)p.fwd_grid), dim3(kThreads),
                           0, st, static_cast<const TIn *>(hh), static_cast<const TIn *>(hs2), WA,
                           WB, WC, p.B, (int)p.K, (int)p.D, p.slices, p.groups, a_shift, ctx);
    return hipGetLastError();
}

// the split backward: scan pass, then the two contractions into slab partials
template <typename TIn, int NQ>
hipError_t split_launch(const Plan &p, const void *hh, const void *hs2, const float *WA,
                        const float *WB, const float *WC, float a_shift, const float *dctx,
                        float *part, float *dab, float *dc, hipStream_t st)
{
    char *ws = reinterpret_cast<char *>(part);
    float *ab = dab ? dab : reinterpret_cast<float *>(ws + p.split_dab);
    float *cv = dc ? dc : reinterpret_cast<float *>(ws + p.split_dc);
    const int64_t ntiles = p.B * p.K / kPsRows;
    auto scan = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)p.ps_grid), dim3(kPsThreads), 0, st,
                           static_cast<const TIn *>(hh), static_cast<const TIn *>(hs2), WA, WB, WC,
                           ntiles, (int)p.D, a_shift, dctx, ab, cv);
        return hipGetLastError();
    };
    hipError_t e;
    if constexpr (NQ == 8 || NQ == 16) {
        if (p.K == 64) e = scan(gscan_bwd_scan_kernel<TIn, NQ, 64>);
        else if (p.K == 256) e = scan(gscan_bwd_scan_kernel<TIn, NQ, 256>);
        else return hipErrorInvalidValue;
    } else {
        return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const int64_t rows = p.B * p.K;
    // slabs of whole 32-row steps
    const int64_t rps = ((rows + p.split_slabs - 1) / p.split_slabs + kCtRows - 1) / kCtRows * kCtRows;
    const int64_t rpsc = (p.B + p.split_slabs - 1) / p.split_slabs;
    const int sh2 = (int)p.SH2, d = (int)p.D;
    // h_history^T @ [dA | dB]: 2D outputs in tiles of 128
    hipLaunchKernelGGL((gscan_bwd_contract_kernel<TIn, 256, 128, 4, 0>),
                       dim3((unsigned)p.split_slabs, (unsigned)(p.SH2 / 256), (unsigned)(2 * p.D / 128)),
                       dim3(kCtThreads), 0, st, static_cast<const TIn *>(hh), sh2,
                       (const float *)ab, 2 * d, rows, rps, d, sh2, part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // h_s2^T @ dC: D outputs in tiles of 128, or 64
    if (p.D % 128 == 0)
        hipLaunchKernelGGL((gscan_bwd_contract_kernel<TIn, 256, 128, 4, 2>),
                           dim3((unsigned)p.split_slabs, (unsigned)(p.SH2 / 256), (unsigned)(p.D / 128)),
                           dim3(kCtThreads), 0, st, static_cast<const TIn *>(hs2), sh2,
                           (const float *)cv, d, p.B, rpsc, d, sh2, part);
    else
        hipLaunchKernelGGL((gscan_bwd_contract_kernel<TIn, 256, 64, 4, 2>),
                           dim3((unsigned)p.split_slabs, (unsigned)(p.SH2 / 256), (unsigned)(p.D / 64)),
                           dim3(kCtThreads), 0, st, static_cast<const TIn *>(hs2), sh2,
                           (const float *)cv, d, p.B, rpsc, d, sh2, part);
    return hipGetLastError();
}

template <typename TIn, int NQ>
hipError_t bwd_launch(const Plan &p, const void *hh, const void *hs2, const float *WA,
                      const float *WB, const float *WC, float a_shift, const float *dctx,
                      float *part, float *dab, float *dc, float *dh, float *dhs2, hipStream_t st)
{
    if (dh && !p.fused_dinput()) return hipErrorInvalidValue;
    if (p.bwd_split) return split_launch<TIn, NQ>(p, hh, hs2, WA, WB, WC, a_shift, dctx, part, dab, dc, st);
    const bool aligned = 16 % p.K == 0;
    if constexpr (NQ <= 8) {
        if (p.bwd_rows_kernel) {
            auto go = [&](auto kern) {
                hipLaunchKernelGGL(kern, dim3((unsigned)p.bwd_grid), dim3(kThreads2), 0, st,
                                   static_cast<const TIn *>(hh), static_cast<const TIn *>(hs2), WA,
                                   WB, WC, p.B, (int)p.K, (int)p.D, p.slices, p.groups,
                                   p.bwd_rows, a_shift, dctx, part, dab, dc, dh, dhs2);
                return hipGetLastError();
            };
            // the input gradients in the same pass (one state slice)
            if (dh) {
                if (p.K == 8) return go(gscan_bwd_rows_kernel<TIn, NQ, 8, true>);
                return go(gscan_bwd_rows_kernel<TIn, NQ, 0, true>);
            }
            // K = 8 (the spec's history length) and K = 64 run with K folded in
            if (p.K == 8) return go(gscan_bwd_rows_kernel<TIn, NQ, 8, false>);
            if (p.K == 64) return go(gscan_bwd_rows_kernel<TIn, NQ, 64, false>);
            return go(gscan_bwd_rows_kernel<TIn, NQ, 0, false>);
        }
    }
    // K dividing 16 with NQ <= 8 always takes the per-block kernel above
    if constexpr (NQ > 8) {
        if (aligned) {
            hipLaunchKernelGGL((gscan_bwd_kernel<TIn, NQ, true>), dim3((unsigned)p.bwd_grid),
                               dim3(kThreads), 0, st, static_cast<const TIn *>(hh),
                               static_cast<const TIn *>(hs2), WA, WB, WC, p.B, (int)p.K, (int)p.D,
                               p.slices, p.groups, p.bwd_rows, a_shift, dctx, part, dab, dc);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gscan_bwd_kernel<TIn, NQ, false>), dim3((unsigned)p.bwd_grid),
                       dim3(kThreads), 0, st, static_cast<const TIn *>(hh),
                       static_cast<const TIn *>(hs2), WA, WB, WC, p.B, (int)p.K, (int)p.D,
                       p.slices, p.groups, p.bwd_rows, a_shift, dctx, part, dab, dc);
    return hipGetLastError();
}

template <typename TIn>
hipError_t fwd_by_nq(const Plan &p, const void *hh, const void *hs2, const float *WA,
                     const float *WB, const float *WC, float a, const CtxOut &ctx, hipStream_t st)
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
                     float *dab, float *dc, float *dh, float *dhs2, hipStream_t st)
{
    switch (p.nq) {
    case 2: return bwd_launch<TIn, 2>(p, hh, hs2, WA, WB, WC, a, dctx, part, dab, dc, dh, dhs2, st);
    case 4: return bwd_launch<TIn, 4>(p, hh, hs2, WA, WB, WC, a, dctx, part, dab, dc, dh, dhs2, st);
    case 6: return bwd_launch<TIn, 6>(p, hh, hs2, WA, WB, WC, a, dctx, part, dab, dc, dh, dhs2, st);
    case 8: return bwd_launch<TIn, 8>(p, hh, hs2, WA, WB, WC, a, dctx, part, dab, dc, dh, dhs2, st);
    case 10: return bwd_launch<TIn, 10>(p, hh, hs2, WA, WB, WC, a, dctx, part, dab, dc, dh, dhs2, st);
    case 12: return bwd_launch<TIn, 12>(p, hh, hs2, WA, WB, WC, a, dctx, part, dab, dc, dh, dhs2, st);
    case 14: return bwd_launch<TIn, 14>(p, hh, hs2, WA, WB, WC, a, dctx, part, dab, dc, dh, dhs2, st);
    case 16: return bwd_launch<TIn, 16>(p, hh, hs2, WA, WB, WC, a, dctx, part, dab, dc, dh, dhs2, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool make_plan(int64_t B, int64_t K, int64_t SH2, int64_t D, int dtype, Plan *p)
{
    if (B < 1 || K < 1 || SH2 < 16 || SH2 > kMaxSH2Generic || SH2 % 16 != 0 || D < kSlice ||
        D > kMaxD || D % kSlice != 0 || (dtype != 0 && dtype != 1))
        return false;
    // 32-bit element offsets inside a 16-sample group (16 * K * SH2 < 2^31)
    if (K > (int64_t(1) << 18) || B > (int64_t(1) << 40) || B * K > (int64_t(1) << 46))
        return false;
    Plan q;
    q.B = B;
    q.K = K;
    q.SH2 = SH2;
    q.D = D;
    q.dtype = dtype;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    if (SH2 % 64 != 0 || SH2 > kMaxSH2) {
        // materialised projections: partial slabs enough for about 1024
        // contraction workgroups (64 x 64 output tiles), at least 16 rows each
        q.generic = true;
        q.slices = (int)(D / kSlice);
        // contraction tiles: 128 or 256 columns of h, 64 or 128 outputs,
        // whichever wastes less of the last tile; slabs for about 256
        // workgroups of the [dA | dB] contraction, at least 32 rows each
        auto pick = [](int64_t n, int64_t a, int64_t b) { return (n + a - 1) / a * a < (n + b - 1) / b * b ? a : b; };
        q.gen_mt = (int)pick(SH2, 128, 256);
        q.gen_nt_ab = (int)pick(2 * D, 64, 128);
        const int64_t tiles = (SH2 + q.gen_mt - 1) / q.gen_mt * ((2 * D + q.gen_nt_ab - 1) / q.gen_nt_ab);
        const int64_t rows = B * K;
        int64_t slabs = 256 / tiles;
        const int64_t most = (rows + 31) / 32;
        if (slabs > most) slabs = most;
        if (slabs < 1) slabs = 1;
        q.gen_slabs = slabs;
        q.bwd_rows = slabs;
        const int64_t wsz = SH2 * D;
        q.red_grid = 3 * wsz / kRedCols;
        const size_t part = (size_t)(slabs * 3 * wsz * 4);
        const size_t abb = (size_t)rows * (size_t)(2 * D) * sizeof(float);
        q.split_dab = up(part);
        q.split_dc = up(q.split_dab + abb);
        q.ws_bytes = q.split_dc + (size_t)(B * D) * sizeof(float);
        q.fwd_cv = up(abb);
        q.fwd_scratch = q.fwd_cv + (size_t)(B * D) * sizeof(float);
        *p = q;
        return true;
    }
    q.nq = (int)(SH2 / 32);
    q.slices = (int)(D / kSlice);
    q.groups = (B + kGroupSamples - 1) / kGroupSamples;
    q.fwd_rows = (q.groups + kXcds - 1) / kXcds * kXcds;
    // forward: two workgroups per CU, persistent beyond 512 group slots;
    // for D > 16, S = 4 or 2 slices per workgroup of two groups when the A|B
    // image fits (S * SH2 <= 1024) and either the scans are long enough to
    // amortise staging it (K >= 16) or there are few groups
    q.fwd_prow = q.fwd_rows < kFwdMaxRows ? q.fwd_rows : kFwdMaxRows;
    q.fwd_grid = q.fwd_prow * q.slices;
    q.fwd_ms = 0;
    if (q.slices >= 2 && (K >= 16 || q.groups <= kFwdMaxRows)) {
        for (int sv = 4; sv >= 2; sv /= 2)
            if (q.fwd_ms == 0 && q.slices % sv == 0 && sv * q.nq <= 32) q.fwd_ms = sv;
    }
    if (q.fwd_ms) {
        const int64_t pairs = (q.groups + 1) / 2;
        q.fwd_grid = (pairs + kXcds - 1) / kXcds * kXcds * (q.slices / q.fwd_ms);
    }
    // backward: the rows kernel (K divides 16 or is 32 or 64, SH2 <= 256) runs one persistent
    // workgroup per CU; the general kernel about two per CU when the weight
    // slice leaves room for two in LDS, one otherwise (256 CUs)
    q.bwd_rows_kernel = (16 % K == 0 || K == 32 || K == 64) && q.nq <= 8;
    const int64_t target = (q.bwd_rows_kernel || q.nq > 8) ? 256 : 512;
    int64_t cap = target / q.slices / kXcds * kXcds;
    if (cap < kXcds) cap = kXcds;
    q.bwd_rows = q.fwd_rows < cap ? q.fwd_rows : cap;
    q.bwd_grid = q.bwd_rows * q.slices;
    // the forward with the same decomposition where one slice holds every
    // state and each workgroup walks many groups (the one-group-per-workgroup
    // kernels start faster on a few groups per CU)
    q.fwd_perblock = q.bwd_rows_kernel && q.slices == 1 && q.groups > kFwdMaxRows;
    const int64_t wsz = SH2 * D;
    q.red_grid = 3 * wsz / kRedCols;
    q.ws_bytes = (size_t)(q.bwd_rows * 3 * wsz * 4);
    // split backward for the widest rows (SH2 = 512, beyond the per-block
    // kernel's LDS budget) when whole samples fill 256-row tiles (K = 64 or
    // 256 compiled) and the states come in groups of 64
    const int64_t ns = K > 0 && kPsRows % K == 0 ? kPsRows / K : 0;
    const bool tiles = (K == 64 || K == 256) && ns > 0 && B % ns == 0 && D % kPsStates == 0;
    if (tiles) {
        // persistent grid over the 256-row tiles, D / 32 state groups per tile
        const int64_t ntiles = B * K / kPsRows;
        const int64_t nsg = D / kPsStates;
        const int64_t cap = 256 / (8 * nsg) * (8 * nsg);
        const int64_t want = (ntiles + 7) / 8 * 8 * nsg;
        q.ps_grid = want < cap ? want : cap;
    }
    // the forward over those tiles where its A|B image is the multi-slice
    // kernel's (SH2 = 512)
    q.fwd_tile = tiles && SH2 == 512;
    if (tiles && SH2 == 512 && D % 64 == 0) {
        q.bwd_split = true;
        q.bwd_rows_kernel = false;
        const int64_t tiles_per_slab = (SH2 / 256) * (2 * D / 128);
        int64_t slabs = 256 / tiles_per_slab;
        if (slabs < 1) slabs = 1;
        q.split_slabs = slabs;
        const size_t part = (size_t)(slabs * 3 * wsz * 4);
        q.split_dab = up(part);
        q.split_dc = up(q.split_dab + (size_t)(B * K) * (size_t)(2 * D) * sizeof(float));
        q.ws_bytes = q.split_dc + (size_t)(B * D) * sizeof(float);
        q.bwd_rows = slabs;  // the reduction sums one partial per slab
    }
    if (q.fwd_grid > 0x7fffffff || q.bwd_grid > 0x7fffffff) return false;
    *p = q;
    return true;
}

hipError_t launch_forward(const Plan &p, const void *hh, const void *hs2, const float *WA,
                          const float *WB, const float *WC, float a_shift, const CtxOut &ctx,
                          void *scratch, hipStream_t st)
{
    if (p.generic) {
        if (!scratch) return hipErrorInvalidValue;
        char *sc = static_cast<char *>(scratch);
        return launch_gen_forward(p, hh, hs2, WA, WB, WC, a_shift, ctx,
                                  reinterpret_cast<float *>(sc),
                                  reinterpret_cast<float *>(sc + p.fwd_cv), st);
    }
    if (p.dtype == 1) return fwd_by_nq<uint16_t>(p, hh, hs2, WA, WB, WC, a_shift, ctx, st);
    return fwd_by_nq<float>(p, hh, hs2, WA, WB, WC, a_shift, ctx, st);
}

hipError_t launch_backward_partials(const Plan &p, const void *hh, const void *hs2,
                                    const float *WA, const float *WB, const float *WC,
                                    float a_shift, const float *dctx, float *part, float *dab,
                                    float *dc, float *dh, float *dhs2, hipStream_t st)
{
    if (p.generic) {
        if (dh) return hipErrorInvalidValue;
        char *ws = reinterpret_cast<char *>(part);
        float *ab = dab ? dab : reinterpret_cast<float *>(ws + p.split_dab);
        float *cv = dc ? dc : reinterpret_cast<float *>(ws + p.split_dc);
        return launch_gen_partials(p, hh, hs2, WA, WB, WC, a_shift, dctx, part, ab, cv, st);
    }
    return p.dtype == 1
               ? bwd_by_nq<uint16_t>(p, hh, hs2, WA, WB, WC, a_shift, dctx, part, dab, dc, dh, dhs2, st)
               : bwd_by_nq<float>(p, hh, hs2, WA, WB, WC, a_shift, dctx, part, dab, dc, dh, dhs2, st);
}

hipError_t launch_adjoint(const Plan &p, float *ab, float *cv, const float *dctx, float a_shift,
                          hipStream_t st)
{
    const int64_t n = p.B * p.D;
    hipLaunchKernelGGL(gscan_adjoint_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, st, ab, cv, dctx, p.B, p.K, (int)p.D, a_shift);
    return hipGetLastError();
}

// Launch shape of rows_by_weights: the widest column slice (CT tiles of 16)
// whose weight image fits (max_pairs (k chunk, tile) pairs of 2 KiB),
// narrowed while there are too few (row tile, slice) pairs to fill the chip.
// The projections take images up to 128 KiB (one workgroup per CU, but each
// long row split and read once instead of once per slice); the input
// gradients, whose rows are short and whose time is their output stream,
// keep two workgroups per CU (64 KiB).
struct RbwShape {
    int ct;
    size_t shmem;
    dim3 grid;
};

RbwShape rbw_shape(int64_t KD, int64_t NOUT, int64_t nrows, int max_pairs)
{
    const int nkc = (int)((KD + 31) / 32);
    const int tiles16 = (int)(NOUT / 16);
    const int64_t row_tiles = (nrows + kDinRows - 1) / kDinRows;
    int ct = 16;
    while (ct > 1 && (ct * nkc > max_pairs || tiles16 % ct != 0 ||
                      row_tiles * (tiles16 / ct) < kDinMaxWorkgroups))
        ct /= 2;
    RbwShape r;
    r.ct = ct;
    r.shmem = (size_t)nkc * ct * 2 * kWave * sizeof(u4);
    // persistent row-tile slots per slice, a multiple of the XCD count:
    // as many workgroups as fit on the chip at once (two per CU; one with an
    // image above 64 KiB), so that each stages its weight image once for
    // several row tiles
    const int nsl = tiles16 / ct;
    const int64_t wgs = r.shmem > 64 * 1024 ? kDinMaxWorkgroups / 2 : kDinMaxWorkgroups;
    int64_t slots = wgs / nsl / kXcds * kXcds;
    if (slots < kXcds) slots = kXcds;
    const int64_t need = (row_tiles + kXcds - 1) / kXcds * kXcds;
    if (slots > need) slots = need;
    r.grid = dim3((unsigned)(slots * nsl));
    return r;
}

template <int WHICH>
hipError_t launch_dinput_which(const float *in, const float *W1, const float *W2, int64_t D1,
                               int64_t KD, int64_t SH2, int64_t nrows, float *out, hipStream_t st)
{
    if (nrows <= 0) return hipSuccess;
    const RbwShape sh = rbw_shape(KD, SH2, nrows, 32);
    const dim3 grid = sh.grid;
    const size_t shmem = sh.shmem;
    const int d1 = (int)D1, kd = (int)KD, sh2 = (int)SH2;
    switch (sh.ct) {
    case 16: hipLaunchKernelGGL((gscan_dinput_kernel<16, WHICH>), grid, dim3(kThreads), shmem, st, in, W1, W2, d1, kd, sh2, nrows, out); break;
    case 8: hipLaunchKernelGGL((gscan_dinput_kernel<8, WHICH>), grid, dim3(kThreads), shmem, st, in, W1, W2, d1, kd, sh2, nrows, out); break;
    case 4: hipLaunchKernelGGL((gscan_dinput_kernel<4, WHICH>), grid, dim3(kThreads), shmem, st, in, W1, W2, d1, kd, sh2, nrows, out); break;
    case 2: hipLaunchKernelGGL((gscan_dinput_kernel<2, WHICH>), grid, dim3(kThreads), shmem, st, in, W1, W2, d1, kd, sh2, nrows, out); break;
    default: hipLaunchKernelGGL((gscan_dinput_kernel<1, WHICH>), grid, dim3(kThreads), shmem, st, in, W1, W2, d1, kd, sh2, nrows, out); break;
    }
    return hipGetLastError();
}

template <typename TIn, int WHICH>
hipError_t launch_proj_which(const TIn *in, const float *W1, const float *W2, int64_t D1,
                             int64_t KD, int64_t NOUT, int64_t nrows, float *out, hipStream_t st)
{
    if (nrows <= 0) return hipSuccess;
    const RbwShape sh = rbw_shape(KD, NOUT, nrows, 64);
    const dim3 grid = sh.grid;
    const size_t shmem = sh.shmem;
    const int d1 = (int)D1, kd = (int)KD, no = (int)NOUT;
    switch (sh.ct) {
    case 16: hipLaunchKernelGGL((gscan_proj_kernel<TIn, 16, WHICH>), grid, dim3(kThreads), shmem, st, in, W1, W2, d1, kd, no, nrows, out); break;
    case 8: hipLaunchKernelGGL((gscan_proj_kernel<TIn, 8, WHICH>), grid, dim3(kThreads), shmem, st, in, W1, W2, d1, kd, no, nrows, out); break;
    case 4: hipLaunchKernelGGL((gscan_proj_kernel<TIn, 4, WHICH>), grid, dim3(kThreads), shmem, st, in, W1, W2, d1, kd, no, nrows, out); break;
    case 2: hipLaunchKernelGGL((gscan_proj_kernel<TIn, 2, WHICH>), grid, dim3(kThreads), shmem, st, in, W1, W2, d1, kd, no, nrows, out); break;
    default: hipLaunchKernelGGL((gscan_proj_kernel<TIn, 1, WHICH>), grid, dim3(kThreads), shmem, st, in, W1, W2, d1, kd, no, nrows, out); break;
    }
    return hipGetLastError();
}

namespace {
template <typename TIn, int CT0>
hipError_t proj2_ct1(const ProjJob &j0, const ProjJob &j1, const RbwShape &s0,
                     const RbwShape &s1, hipStream_t st)
{
    const size_t shmem = s0.shmem > s1.shmem ? s0.shmem : s1.shmem;
    const dim3 grid(s0.grid.x + s1.grid.x);
    const int64_t nwg0 = s0.grid.x;
    if (s1.ct == CT0)
        hipLaunchKernelGGL((gscan_proj2_kernel<TIn, CT0, CT0>), grid, dim3(kThreads), shmem, st,
                           j0, j1, nwg0);
    else if constexpr (CT0 >= 2)
        hipLaunchKernelGGL((gscan_proj2_kernel<TIn, CT0, CT0 / 2>), grid, dim3(kThreads), shmem,
                           st, j0, j1, nwg0);
    return hipGetLastError();
}

template <typename TIn>
hipError_t proj2(const ProjJob &j0, const ProjJob &j1, const RbwShape &s0, const RbwShape &s1,
                 hipStream_t st)
{
    switch (s0.ct) {
    case 16: return proj2_ct1<TIn, 16>(j0, j1, s0, s1, st);
    case 8: return proj2_ct1<TIn, 8>(j0, j1, s0, s1, st);
    case 4: return proj2_ct1<TIn, 4>(j0, j1, s0, s1, st);
    case 2: return proj2_ct1<TIn, 2>(j0, j1, s0, s1, st);
    default: return proj2_ct1<TIn, 1>(j0, j1, s0, s1, st);
    }
}
}  // namespace

hipError_t launch_proj_ab_c(int dtype, const void *hh, const void *hs2, const float *WA,
                            const float *WB, const float *WC, int64_t rows, int64_t B,
                            int64_t SH2, int64_t D, float *ab, float *cv, hipStream_t st)
{
    const RbwShape s0 = rbw_shape(SH2, 2 * D, rows, 64), s1 = rbw_shape(SH2, D, B, 64);
    if (s1.ct != s0.ct && 2 * s1.ct != s0.ct) {
        // slice widths the combined kernel is not compiled for: two launches
        hipError_t e = launch_proj(dtype, hh, WA, WB, D, SH2, 2 * D, rows, ab, st);
        if (e == hipSuccess) e = launch_proj(dtype, hs2, WC, nullptr, D, SH2, D, B, cv, st);
        return e;
    }
    const ProjJob j0 = {hh, WA, WB, (int)D, (int)SH2, (int)(2 * D), rows, ab};
    const ProjJob j1 = {hs2, WC, nullptr, (int)D, (int)SH2, (int)D, B, cv};
    return dtype == 1 ? proj2<uint16_t>(j0, j1, s0, s1, st) : proj2<float>(j0, j1, s0, s1, st);
}

hipError_t launch_proj(int dtype, const void *in, const float *W1, const float *W2, int64_t D1,
                       int64_t KD, int64_t NOUT, int64_t nrows, float *out, hipStream_t st)
{
    const bool ab = W2 != nullptr;
    if (dtype == 1)
        return ab ? launch_proj_which<uint16_t, 0>(static_cast<const uint16_t *>(in), W1, W2, D1, KD, NOUT, nrows, out, st)
                  : launch_proj_which<uint16_t, 1>(static_cast<const uint16_t *>(in), W1, W2, D1, KD, NOUT, nrows, out, st);
    return ab ? launch_proj_which<float, 0>(static_cast<const float *>(in), W1, W2, D1, KD, NOUT, nrows, out, st)
              : launch_proj_which<float, 1>(static_cast<const float *>(in), W1, W2, D1, KD, NOUT, nrows, out, st);
}

hipError_t launch_gen_contract(const Plan &p, const void *hh, const void *hs2, const float *ab,
                               const float *cv, float *part, hipStream_t st)
{
    const int64_t rows = p.B * p.K;
    // slabs of whole 32-row steps over the rows; the samples split evenly
    const int64_t rps = ((rows + p.gen_slabs - 1) / p.gen_slabs + kCtRows - 1) / kCtRows * kCtRows;
    const int64_t rpsc = (p.B + p.gen_slabs - 1) / p.gen_slabs;
    const int d2 = (int)(2 * p.D), d = (int)p.D;
    const int MT = p.gen_mt, NT = p.gen_nt_ab;  // one tile shape for both jobs
    const int gm = (int)((p.SH2 + MT - 1) / MT);
    const CtJob j0 = {hh, (int)p.SH2, ab, d2, rows, rps, 0, gm, (d2 + NT - 1) / NT};
    const CtJob j1 = {hs2, (int)p.SH2, cv, d, p.B, rpsc, 2, gm, (d + NT - 1) / NT};
    const dim3 grid((unsigned)(p.gen_slabs * j0.gm * j0.gn));
    const int sh2 = (int)p.SH2;
#define GSCAN_GEN_CT(TX, MTV, NTV)                                                              \
    hipLaunchKernelGGL((gscan_gen_contract_kernel<TX, MTV, NTV>), grid, dim3(kCtThreads), 0, st, \
                       j0, j1, d, sh2, part)
    if (p.dtype == 1) {
        if (MT == 256 && NT == 128) GSCAN_GEN_CT(uint16_t, 256, 128);
        else if (MT == 256) GSCAN_GEN_CT(uint16_t, 256, 64);
        else if (NT == 128) GSCAN_GEN_CT(uint16_t, 128, 128);
        else GSCAN_GEN_CT(uint16_t, 128, 64);
    } else {
        if (MT == 256 && NT == 128) GSCAN_GEN_CT(float, 256, 128);
        else if (MT == 256) GSCAN_GEN_CT(float, 256, 64);
        else if (NT == 128) GSCAN_GEN_CT(float, 128, 128);
        else GSCAN_GEN_CT(float, 128, 64);
    }
#undef GSCAN_GEN_CT
    return hipGetLastError();
}

hipError_t launch_dinput(const float *in, const float *W1, const float *W2, int64_t D1, int64_t KD,
                         int64_t SH2, int64_t nrows, float *out, hipStream_t st)
{
    return W2 ? launch_dinput_which<0>(in, W1, W2, D1, KD, SH2, nrows, out, st)
              : launch_dinput_which<1>(in, W1, W2, D1, KD, SH2, nrows, out, st);
}

hipError_t launch_backward_reduce(const Plan &p, const float *part, float *dWA, float *dWB,
                                  float *dWC, hipStream_t st)
{
    // the per-block kernel writes its partials in the quad layout; the
    // general kernel and the split contraction in [which][i][s]
    hipLaunchKernelGGL(gscan_reduce_kernel, dim3((unsigned)p.red_grid), dim3(kRedThreads), 0, st,
                       part, p.bwd_rows, p.SH2 * p.D, (int)p.D, p.bwd_rows_kernel ? 1 : 0, dWA,
                       dWB, dWC);
    return hipGetLastError();
}

}  // namespace gscan
