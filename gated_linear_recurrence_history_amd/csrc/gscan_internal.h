// Internal interface between the C ABI (gscan_api.hip) and the kernels
// (gscan_kernels.hip).  The launch plan is pure host arithmetic.
#pragma once

#include <cstddef>
#include <cstdint>
#include <hip/hip_runtime.h>

namespace gscan {

// Work decomposition shared by every kernel.
constexpr int kWave = 64;          // lanes per wavefront
constexpr int kWaves = 4;          // wavefronts per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr int kGroupSamples = 16;  // samples per workgroup work item
constexpr int kSlice = 16;         // states per workgroup (one MFMA N tile)
constexpr int kBlockRows = 16;     // h_history rows per wavefront block (MFMA M tile)
constexpr int kChunkRows = kBlockRows * kWaves;  // rows per backward chunk
constexpr int kXcds = 8;           // MI355X accelerator complex dies
constexpr int kMaxSH2 = 512;       // the fused kernels (SH2 % 64 == 0)
constexpr int kMaxSH2Generic = 1024;  // the materialised-projection path (SH2 % 16 == 0)
constexpr int64_t kFwdMaxRows = 512;
constexpr int kMaxD = 256;

struct Plan {
    int64_t B = 0, K = 0, SH2 = 0, D = 0;
    int dtype = 0;          // 0 f32, 1 bf16
    int nq = 0;             // SH2 / 32
    int slices = 0;         // D / 16
    int64_t groups = 0;     // ceil(B / 16)
    int64_t fwd_rows = 0;   // group slots, one per group (multiple of 8)
    int64_t fwd_prow = 0;   // persistent rows of the forward grid (<= kFwdMaxRows)
    int64_t bwd_rows = 0;   // persistent workgroup rows of the backward grid (multiple of 8)
    int64_t fwd_grid = 0;
    int fwd_ms = 0;         // slices per workgroup of the multi-slice forward (0: one)
    int64_t bwd_grid = 0;
    int64_t red_grid = 0;
    bool bwd_rows_kernel = false;  // backward via the K-divides-16 kernel
    // split backward (scan pass, then contraction over row slabs): the
    // workspace holds the slab partials, dL/dA | dL/dB per row at split_dab
    // and dL/dC per sample at split_dc (byte offsets)
    bool bwd_split = false;
    bool fwd_tile = false;  // forward over the split backward's tiles (gscan_fwd_tile_kernel)
    bool fwd_perblock = false;  // forward with the per-block decomposition (gscan_fwd_rows_kernel)
    // shapes outside the fused kernels (SH2 not a multiple of 64, or above
    // 512): materialised projections, per-(sample, state) scans and plain
    // contractions into gen_slabs partials.  The workspace holds the
    // partials, A | Bv per row at split_dab and C per sample at split_dc;
    // the forward needs fwd_scratch bytes (A | Bv, then C at fwd_cv).
    bool generic = false;
    int64_t gen_slabs = 0;
    int gen_mt = 0, gen_nt_ab = 0;  // contraction tile (h columns, outputs), both contractions
    size_t fwd_scratch = 0, fwd_cv = 0;
    int64_t split_slabs = 0;
    int64_t ps_grid = 0;
    size_t split_dab = 0, split_dc = 0;
    size_t ws_bytes = 0;    // the backward's workspace (partials, and the split pass's adjoints)
    // phase 1 leaves the final dL/dA | dL/dB and dL/dC (not projections)
    bool adjoints_final() const { return bwd_rows_kernel || bwd_split || generic; }
    // phase 1 writes the input gradients itself (the per-block kernel with
    // one 16-state slice holds every state of a row)
    bool fused_dinput() const { return bwd_rows_kernel && slices == 1; }
};

// Where the forward writes context[b][s]: the context output (null: not
// written) and/or an add into row b of a caller buffer (null: none), whose
// pointer already includes the column offset, with row pitch `ld` floats.
struct CtxOut {
    float *ctx = nullptr;
    float *enr = nullptr;
    int64_t ld = 0;
};

// Fills `p` for a validated shape.  Returns false if the shape is unsupported.
bool make_plan(int64_t B, int64_t K, int64_t SH2, int64_t D, int dtype, Plan *p);

// scratch: p.fwd_scratch bytes of device memory (null when that is 0)
hipError_t launch_forward(const Plan &p, const void *h_history, const void *h_s2,
                          const float *W_A, const float *W_B, const float *W_C,
                          float a_shift, const CtxOut &out, void *scratch, hipStream_t stream);

// The materialised-projection path (p.generic): forward into `out` with
// A | Bv in ab [B*K][2D] and C in cv [B][D] as scratch; phase 1 of the
// backward into `part` with the adjoints left final in ab and cv.
hipError_t launch_gen_forward(const Plan &p, const void *hh, const void *hs2, const float *WA,
                              const float *WB, const float *WC, float a_shift, const CtxOut &ctx,
                              float *ab, float *cv, hipStream_t st);
hipError_t launch_gen_partials(const Plan &p, const void *hh, const void *hs2, const float *WA,
                               const float *WB, const float *WC, float a_shift,
                               const float *dctx, float *part, float *ab, float *cv,
                               hipStream_t st);

// out[nrows][NOUT] = in[nrows][KD] x [W1 | W2] (W1 [KD][D1], W2 [KD][NOUT-D1],
// or W2 null when NOUT == D1); `in` fp32 (dtype 0) or bf16 (dtype 1).
hipError_t launch_proj(int dtype, const void *in, const float *W1, const float *W2, int64_t D1,
                       int64_t KD, int64_t NOUT, int64_t nrows, float *out, hipStream_t stream);

// Both: ab [rows][2D] = h_history [W_A | W_B] and cv [B][D] = h_s2 W_C, in
// one launch where the slice widths allow.
hipError_t launch_proj_ab_c(int dtype, const void *hh, const void *hs2, const float *WA,
                            const float *WB, const float *WC, int64_t rows, int64_t B,
                            int64_t SH2, int64_t D, float *ab, float *cv, hipStream_t stream);

// The weight-gradient contractions of the materialised-projection path into
// p.gen_slabs partials: h_history^T [dA | dB] (ab [B*K][2D]) and h_s2^T dC
// (cv [B][D]).
hipError_t launch_gen_contract(const Plan &p, const void *hh, const void *hs2, const float *ab,
                               const float *cv, float *part, hipStream_t stream);

// Phase 1: per-workgroup weight-gradient partials into `partials`.  When
// `dab` / `dc` are not null they receive, for the input gradients, either
// the final dL/dA | dL/dB per row ([B*K][2D]) and dL/dC per sample ([B][D])
// (p.adjoints_final()), or the projections A | Bv and C in the same places,
// which launch_adjoint then turns into those adjoints.  When `dh` / `dhs2`
// are not null (only where p.fused_dinput(); dab and dc then null) phase 1
// writes d_h_history [B*K][SH2] and d_h_s2 [B][SH2] itself.
hipError_t launch_backward_partials(const Plan &p, const void *h_history, const void *h_s2,
                                    const float *W_A, const float *W_B, const float *W_C,
                                    float a_shift, const float *d_context, float *partials,
                                    float *dab, float *dc, float *dh, float *dhs2,
                                    hipStream_t stream);

// In place: A | Bv -> dL/dA | dL/dB per row, C -> dL/dC per sample.
hipError_t launch_adjoint(const Plan &p, float *ab, float *cv, const float *d_context,
                          float a_shift, hipStream_t stream);

// out[nrows][SH2] = in[nrows][KD] x [W1 | W2]^T (W1 [SH2][D1], W2 [SH2][KD-D1]).
hipError_t launch_dinput(const float *in, const float *W1, const float *W2, int64_t D1,
                         int64_t KD, int64_t SH2, int64_t nrows, float *out,
                         hipStream_t stream);

// Bias-gradient reduction: out[j] = sum_r grad[r][j] (two phases, fp64
// partials in `workspace` of colsum_workspace_bytes()).
size_t colsum_workspace_bytes(int64_t rows, int64_t cols);
hipError_t launch_colsum(const float *grad, int64_t rows, int64_t cols, float *out,
                         void *workspace, hipStream_t stream);

// CIFG matrix-memory update, independent mode, in place on C [B][d][d].
hipError_t launch_cifg(float *C, const float *H, const float *X, const float *W_f,
                       const float *b_f, int64_t B, int64_t d, int64_t din, hipStream_t stream);

// Phase 2: fixed-order sum of the partials into dW_A, dW_B, dW_C.
hipError_t launch_backward_reduce(const Plan &p, const float *partials, float *dW_A,
                                  float *dW_B, float *dW_C, hipStream_t stream);

}  // namespace gscan
