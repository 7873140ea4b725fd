// CIFG matrix-memory update, independent mode, for gfx950 (MI355X).
//
// BURT-IMMA CUDA Kernel API Reference, section 2.3 batched_cifg_update with
// shared_memory_mode = false: every sample b applies section 2.2
// cifg_update, steps 1-4, to its own memory matrix:
//   concat = [h_b ; x_b],  f = sigmoid(W_f concat + b_f)      (d_model gates)
//   C_b[i][j] <- f[i] C_b[i][j] + (1 - f[i]) h_b[i] h_b[j]
// The page's kernel takes one block per row of C.  Here the update is a
// pure stream of C (read once, written once) with a small dot product per
// row in front of it, so one workgroup takes a tile of 4 rows of 4 samples
// (small enough that several workgroups per CU, at different phases, keep
// reads and writes of C in flight together: 8 samples per tile took 15%
// longer).  It requests the gate inputs of the tile (the 4 vectors
// [h_b ; x_b] and the 4 rows of W_f, 1024 columns per round, L2-resident)
// and then the tile's
// first 512 columns of C, stages the gate inputs in LDS, forms the 16 gates
// (sixteen lanes per gate, each a strided part of the dot product, added in
// a fixed tree) while C is in flight, and then updates and stores the tile,
// 512 columns at a time, with 16-byte accesses.
// Arithmetic is fp32 throughout; 1 - f is formed as exp(-a) * f for a > 0
// (no cancellation when the gate saturates).
#include <cstdint>

#include "gscan_internal.h"

namespace gscan {
namespace {

constexpr int kCifgThreads = 256;
constexpr int kCifgRows = 4;        // rows of C per tile
constexpr int kCifgSamples = 4;     // samples per tile
constexpr int kCifgPairs = kCifgRows * kCifgSamples;
constexpr int kCifgLanesPerGate = kCifgThreads / kCifgPairs;  // 16
constexpr int kCifgCols = 512;      // columns per pass
constexpr int kCifgPer = kCifgPairs * (kCifgCols / 4) / kCifgThreads;  // 16-byte pieces per thread and pass
constexpr int kCifgK = 1024;        // gate-input columns staged per round
constexpr int kCifgPitch = kCifgK + 4;  // LDS row pitch (floats): rows start on different banks
constexpr int kCifgStageRows = kCifgSamples + kCifgRows;  // concat rows, then W_f rows
constexpr int kCifgStage = kCifgStageRows * kCifgK / 4 / kCifgThreads;  // pieces per thread and round

typedef float f4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kCifgThreads)
gscan_cifg_kernel(float *__restrict__ C, const float *__restrict__ H, const float *__restrict__ X,
                  const float *__restrict__ W, const float *__restrict__ bias, int64_t B, int d,
                  int din)
{
    // gate inputs of one round: [h_b ; x_b] of the tile's samples, then the
    // tile's 4 rows of W_f, each kCifgK columns wide
    __shared__ float stg[kCifgStageRows][kCifgPitch];
    __shared__ float fl[kCifgPairs], fcl[kCifgPairs], hil[kCifgPairs];
    const int tid = threadIdx.x;
    const int64_t b0 = (int64_t)blockIdx.x * kCifgSamples;
    const int i0 = blockIdx.y * kCifgRows;
    const int q4 = d / 4;  // 16-byte pieces per row of C
    const int L = d + din;

    // pair p: sample p / 4, row p % 4 of the tile (clamped to a valid one)
    auto pair_ok = [&](int p) {
        return b0 + p / kCifgRows < B && i0 + p % kCifgRows < d;
    };
    // staged piece v of a round starting at column k0: stage row v / 256,
    // columns 4 * (v % 256); rows past the batch or the matrix repeat a valid one
    auto stage_src = [&](int v, int k0) {
        const int r = v / (kCifgK / 4), k = k0 + 4 * (v % (kCifgK / 4));
        if (k >= L) return (const f4 *)nullptr;
        if (r < kCifgSamples) {
            const int64_t b = b0 + r < B ? b0 + r : B - 1;
            return reinterpret_cast<const f4 *>(k < d ? H + b * d + k : X + b * din + (k - d));
        }
        const int i = i0 + (r - kCifgSamples) < d ? i0 + (r - kCifgSamples) : d - 1;
        return reinterpret_cast<const f4 *>(W + (int64_t)i * L + k);
    };
    auto load_stage = [&](f4 (&sv)[kCifgStage], int k0) {
#pragma unroll
        for (int j = 0; j < kCifgStage; ++j) {
            const f4 *src = stage_src(tid + kCifgThreads * j, k0);
            sv[j] = src ? *src : f4{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto store_stage = [&](const f4 (&sv)[kCifgStage]) {
#pragma unroll
        for (int j = 0; j < kCifgStage; ++j) {
            const int v = tid + kCifgThreads * j;
            *reinterpret_cast<f4 *>(&stg[v / (kCifgK / 4)][4 * (v % (kCifgK / 4))]) = sv[j];
        }
    };
    // Piece u of a pass belongs to sample u / 2 of the tile (a uniform base
    // pointer: its four rows are contiguous in C) and to row 2 (u % 2) + t7
    // of it, t7 = tid / 128, column 4 (tid % 128) of the pass: two lane
    // offsets serve every piece.
    const int t7 = tid >> 7, cl = tid & 127;
    auto sample_base = [&](int u) { return C + (b0 + (u >> 1)) * (int64_t)d * d; };
    auto piece_ok = [&](int u, int c4) {
        return b0 + (u >> 1) < B && i0 + 2 * (u & 1) + t7 < d && c4 < q4;
    };
    auto piece_off = [&](int u, int c4) { return (i0 + 2 * (u & 1) + t7) * d + 4 * c4; };
    auto load_c = [&](f4 (&cv)[kCifgPer], int c0) {
        const int c4 = c0 / 4 + cl;
#pragma unroll
        for (int u = 0; u < kCifgPer; ++u)
            cv[u] = piece_ok(u, c4)
                        ? *reinterpret_cast<const f4 *>(sample_base(u) + piece_off(u, c4))
                        : f4{0.f, 0.f, 0.f, 0.f};
    };

    // the first round of gate inputs (served by L2) is requested first, then
    // the first pass of C (from HBM): waiting for the former leaves the
    // latter in flight
    f4 sv[kCifgStage];
    load_stage(sv, 0);
    f4 cv[kCifgPer];
    load_c(cv, 0);

    // gates: lanes 16p .. 16p+15 form the dot product of W_f row i with
    // [h_b ; x_b], lane q taking the pieces q, q + 16, ... of each round;
    // the sixteen partial sums are added in a fixed tree
    const int gp = tid / kCifgLanesPerGate, gq = tid % kCifgLanesPerGate;
    const int gs = gp / kCifgRows, gr = kCifgSamples + gp % kCifgRows;
    float acc = 0.f;
    for (int k0 = 0; k0 < L; k0 += kCifgK) {
        if (k0 > 0) {
            __syncthreads();  // the previous round's reads are done
            load_stage(sv, k0);
        }
        store_stage(sv);
        __syncthreads();
        const int n4 = (L - k0 < kCifgK ? L - k0 : kCifgK) / 4;
        for (int k4 = gq; k4 < n4; k4 += kCifgLanesPerGate) {
            const f4 c = *reinterpret_cast<const f4 *>(&stg[gs][4 * k4]);
            const f4 w = *reinterpret_cast<const f4 *>(&stg[gr][4 * k4]);
            acc = fmaf(w[0], c[0], acc);
            acc = fmaf(w[1], c[1], acc);
            acc = fmaf(w[2], c[2], acc);
            acc = fmaf(w[3], c[3], acc);
        }
    }
#pragma unroll
    for (int o = kCifgLanesPerGate / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kCifgLanesPerGate);
    if (gq == 0) {
        const bool ok = pair_ok(gp);
        const int64_t b = ok ? b0 + gp / kCifgRows : 0;
        const int i = ok ? i0 + gp % kCifgRows : 0;
        const float a = acc + bias[i];
        const float e = __expf(-a);
        const float f = __builtin_amdgcn_rcpf(1.0f + e);
        fl[gp] = f;
        fcl[gp] = a > 0.f ? e * f : 1.0f - f;
        hil[gp] = H[b * d + i];
    }
    __syncthreads();

    for (int c0 = 0; c0 < d; c0 += kCifgCols) {
        if (c0 > 0) load_c(cv, c0);
        const int c4 = c0 / 4 + cl;
#pragma unroll
        for (int u = 0; u < kCifgPer; ++u) {
            if (piece_ok(u, c4)) {
                const int p = 2 * u + t7;  // = 4 (u / 2) + row
                const f4 hj = *reinterpret_cast<const f4 *>(H + (b0 + (u >> 1)) * d + 4 * c4);
                const float f = fl[p], fc = fcl[p], hi = hil[p];
                f4 o;
#pragma unroll
                for (int k = 0; k < 4; ++k) o[k] = fmaf(f, cv[u][k], fc * (hi * hj[k]));
                *reinterpret_cast<f4 *>(sample_base(u) + piece_off(u, c4)) = o;
            }
        }
    }
}

}  // namespace

hipError_t launch_cifg(float *C, const float *H, const float *X, const float *W_f,
                       const float *b_f, int64_t B, int64_t d, int64_t din, hipStream_t st)
{
    const dim3 grid((unsigned)((B + kCifgSamples - 1) / kCifgSamples),
                    (unsigned)((d + kCifgRows - 1) / kCifgRows));
    hipLaunchKernelGGL(gscan_cifg_kernel, grid, dim3(kCifgThreads), 0, st, C, H, X, W_f, b_f, B,
                       (int)d, (int)din);
    return hipGetLastError();
}

}  // namespace gscan
