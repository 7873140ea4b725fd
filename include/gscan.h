/*
 * gscan -- gated temporal scan (Mamba2-style), forward and backward, for
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operation (foxhunt design spec "Custom Kernel Optimization - cuBLAS
 * Projections + Batch-Parallel Scans", Design 1 "Mamba2 Scan"):
 *
 *   Forward Step 1:  A = h_history @ W_A (+ a_shift),  Bv = h_history @ W_B,
 *                    C = h_s2 @ W_C
 *   Forward Step 2:  per (sample b, state s), x = 0, then for t = 0..K-1
 *                      x = sigmoid(A[b*K+t, s]) * x + Bv[b*K+t, s]
 *                    context[b, s] = C[b, s] * x
 *   Backward Steps 1-3: replay of the forward, reverse scan, and the weight
 *                    gradients of L = sum(d_context * context):
 *                      dW_A = h_history^T @ dL/dA,  dW_B = h_history^T @ dL/dBv,
 *                      dW_C = h_s2^T @ dL/dC   (dL/dC = d_context * x_K)
 *
 * Layouts (all dense, row-major, no padding):
 *   h_history [B*K][SH2]   row b*K + t holds sample b at step t (t = 0 oldest,
 *                          scanned first)
 *   h_s2      [B][SH2]
 *   W_A, W_B, W_C, dW_A, dW_B, dW_C   [SH2][D]   float32
 *   context, d_context                [B][D]     float32
 * h_history and h_s2 are float32 (GSCAN_F32) or bfloat16 (GSCAN_BF16, raw
 * 16-bit storage).  Everything else is float32; all accumulation is float32.
 *
 * Supported shapes: B >= 1, 1 <= K <= 262144, 16 <= SH2 <= 1024 with
 * SH2 % 16 == 0, 16 <= D <= 256 with D % 16 == 0, B*K*SH2 < 2^62; other
 * shapes return GSCAN_ERR_UNSUPPORTED_SHAPE.  Two paths serve them:
 *   - SH2 % 64 == 0 and SH2 <= 512: fused kernels that project and scan in
 *     one pass, keeping their weight slice (split into bf16 hi/lo halves) in
 *     the 160 KiB of LDS for the whole launch, 192 * SH2 bytes per 16
 *     states, with two wavefronts sharing a row block by halves of 32-column
 *     MFMA units;
 *   - every other supported SH2: the projections of Forward Step 1 are
 *     written out to device memory (B*K*2D + B*D floats), then scanned, and
 *     the weight gradients contracted from them, by separate kernels (the
 *     same split products, the same tolerances, about twice the fused
 *     kernels' time per byte).  Its forward takes that memory from the
 *     caller's workspace or, without one, from the stream-ordered allocator
 *     (hipMallocAsync, released with hipFreeAsync on the same stream); its
 *     backward keeps it in the workspace (the size queries include it).
 *
 * Pointers: every array pointer is DEVICE memory owned by the caller,
 * 16-byte aligned.  Inputs are read only and must not overlap outputs.  The
 * library keeps no allocation between calls, apart from the static scratch
 * array of gscan_backward_noalloc (below).
 *
 * Semantics: each call validates its arguments, enqueues its kernels on
 * `stream` and returns without synchronising; outputs are valid once the
 * stream reaches that point.  Outputs are overwritten, never accumulated
 * into.  Results are bitwise reproducible for identical inputs and shapes
 * (no floating-point atomics).  Calls are reentrant (gscan_backward_noalloc:
 * see its note on overlapping calls).
 *
 * Errors: a non-zero return is one of the GSCAN_ERR_* codes below.  All
 * argument checks run before anything is enqueued: on a validation error
 * nothing is launched and no output is touched.  gscan_last_error() gives a
 * human-readable detail for the calling thread's most recent failure.  NaN
 * or Inf in the inputs is not an error; it propagates per IEEE-754.
 */
#ifndef GSCAN_H
#define GSCAN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GSCAN_F32 = 0,  /* h_history / h_s2 stored as float32 */
    GSCAN_BF16 = 1  /* h_history / h_s2 stored as bfloat16 */
} gscan_dtype_t;

enum {
    GSCAN_OK = 0,
    GSCAN_ERR_INVALID_ARGUMENT = 1,  /* null pointer, non-positive size, bad dtype */
    GSCAN_ERR_UNSUPPORTED_SHAPE = 2, /* shape outside the supported set above */
    GSCAN_ERR_MISALIGNED = 3,        /* a pointer is not 16-byte aligned */
    GSCAN_ERR_WORKSPACE_TOO_SMALL = 4,
    GSCAN_ERR_HIP = 5                /* a HIP runtime call or launch failed */
};

/*
 * Forward pass (Forward Steps 1-2): writes context_out[B][D].
 * Equivalent to gscan_forward_ex(..., GSCAN_F32, 0.0f, NULL, 0, stream).
 */
int gscan_forward(const void *h_history, const void *h_s2,
                  const float *W_A, const float *W_B, const float *W_C,
                  int64_t B, int64_t K, int64_t SH2, int64_t D,
                  float *context_out, hipStream_t stream);

/*
 * Forward with the context folded into a caller buffer (the step after the
 * scan in the design spec: Forward Step 2 ends by accumulating the context
 * into h_enriched, and Step 3 applies it element-wise).  Reading taken:
 * h_enriched is a caller-owned fp32 row-major [B][ld_enriched] buffer (for
 * example the enriched hidden state, of width SH2) and the context is added
 * element-wise into the D columns starting at col_offset of each row:
 *   h_enriched[b][col_offset + s] += context[b][s]
 * Other columns are not touched.  Each element has exactly one writer, so no
 * atomics are needed.  context_out may be NULL (then only h_enriched is
 * updated) or a [B][D] buffer that must not overlap h_enriched.  h_enriched:
 * device memory, 4-byte aligned; requires D <= ld_enriched and
 * 0 <= col_offset <= ld_enriched - D (INVALID_ARGUMENT otherwise).  The add
 * is a read-modify-write of h_enriched in stream order: a concurrent writer
 * of the same rows on another stream races.  Other arguments (workspace
 * included) and errors as for gscan_forward_ex.
 */
int gscan_forward_enrich(const void *h_history, const void *h_s2,
                         const float *W_A, const float *W_B, const float *W_C,
                         int64_t B, int64_t K, int64_t SH2, int64_t D,
                         float *context_out, float *h_enriched, int64_t ld_enriched,
                         int64_t col_offset, gscan_dtype_t in_dtype, float a_shift,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward pass (Backward Steps 1-3): writes dW_A, dW_B, dW_C [SH2][D] for
 * the upstream gradient d_context[B][D].  Recomputes the forward from the
 * inputs; needs no saved activations.  Allocates its workspace stream-ordered
 * (hipMallocAsync / hipFreeAsync on `stream`).
 * Equivalent to gscan_backward_ex(..., GSCAN_F32, 0.0f, NULL, 0, stream).
 */
int gscan_backward(const void *h_history, const void *h_s2,
                   const float *W_A, const float *W_B, const float *W_C,
                   int64_t B, int64_t K, int64_t SH2, int64_t D,
                   const float *d_context, float *dW_A, float *dW_B, float *dW_C,
                   hipStream_t stream);

/*
 * Forward with input dtype, gate bias and an optional caller workspace.
 * a_shift is a constant added to every A value before the sigmoid (it
 * receives no gradient).  workspace: device memory of at least
 * gscan_forward_workspace_bytes() bytes, 256-byte aligned, or NULL to let the
 * call allocate stream-ordered.  Only the shapes outside the fused kernels
 * use it (for the projections of Forward Step 1); for the others the size
 * query returns 0 and workspace / workspace_bytes are ignored.  Contents on
 * entry are ignored.
 */
int gscan_forward_ex(const void *h_history, const void *h_s2,
                     const float *W_A, const float *W_B, const float *W_C,
                     int64_t B, int64_t K, int64_t SH2, int64_t D,
                     float *context_out, gscan_dtype_t in_dtype, float a_shift,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes gscan_forward_ex and gscan_forward_enrich need for this
 * shape: 0 where none is needed, and 0 for an unsupported shape (the calls
 * themselves report that). */
size_t gscan_forward_workspace_bytes(int64_t B, int64_t K, int64_t SH2, int64_t D,
                                     gscan_dtype_t in_dtype);

/*
 * Backward with input dtype, gate bias and an optional caller workspace.
 * workspace: device memory of at least gscan_backward_workspace_bytes()
 * bytes, 256-byte aligned, or NULL to let the call allocate stream-ordered.
 * The workspace holds per-workgroup weight-gradient partials of the
 * two-phase reduction; its contents on entry are ignored.
 */
int gscan_backward_ex(const void *h_history, const void *h_s2,
                      const float *W_A, const float *W_B, const float *W_C,
                      int64_t B, int64_t K, int64_t SH2, int64_t D,
                      const float *d_context, float *dW_A, float *dW_B, float *dW_C,
                      gscan_dtype_t in_dtype, float a_shift,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The two phases of gscan_backward_ex, callable separately (for example to
 * time them, or to run the reduction later on the same stream):
 *
 * Phase 1 writes one weight-gradient partial per backward workgroup into
 * `workspace` (required here, at least gscan_backward_workspace_bytes(),
 * 256-byte aligned).  Phase 2 sums those partials in a fixed order -- so the
 * result is bitwise reproducible -- and overwrites dW_A, dW_B, dW_C.  Phase 2
 * must see the same shape and dtype as the phase 1 that filled the workspace.
 * This is the two-phase batch-parallel reduction of the design spec (section
 * "IQN Bias Grad Reduce": block partials, then a reduction of the partials)
 * applied to the weight gradients.
 */
int gscan_backward_partials(const void *h_history, const void *h_s2,
                            const float *W_A, const float *W_B, const float *W_C,
                            int64_t B, int64_t K, int64_t SH2, int64_t D,
                            const float *d_context, gscan_dtype_t in_dtype, float a_shift,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

int gscan_backward_reduce(const void *workspace, size_t workspace_bytes,
                          int64_t B, int64_t K, int64_t SH2, int64_t D,
                          gscan_dtype_t in_dtype, float *dW_A, float *dW_B, float *dW_C,
                          hipStream_t stream);

/*
 * Backward with input gradients: everything gscan_backward_ex computes, and
 * the gradients of L with respect to the inputs, by the chain rule through
 * the three projections of Forward Step 1:
 *   d_h_history[b*K+t][i] = sum_s dL/dA_vals[b*K+t][s] W_A[i][s]
 *                                + dL/dB_vals[b*K+t][s] W_B[i][s]
 *   d_h_s2[b][i]          = sum_s dL/dC_vals[b][s] W_C[i][s]
 * (the design spec's backward stops at the weight gradients; these are what
 * a layer below the scan needs).  d_h_history [B*K][SH2] and d_h_s2 [B][SH2]
 * are fp32 row-major for either input dtype, caller-owned, 16-byte aligned,
 * overwritten.  workspace: at least gscan_backward_full_workspace_bytes(),
 * 256-byte aligned, or NULL to allocate stream-ordered; it holds the
 * weight-gradient partials and, for shapes whose backward does not form the
 * input gradients in the same pass (the size query accounts for this),
 * dL/dA | dL/dB per row and dL/dC per sample; contents on entry are
 * ignored.  Errors as for gscan_backward_ex.
 */
int gscan_backward_full_ex(const void *h_history, const void *h_s2,
                           const float *W_A, const float *W_B, const float *W_C,
                           int64_t B, int64_t K, int64_t SH2, int64_t D,
                           const float *d_context, float *dW_A, float *dW_B, float *dW_C,
                           float *d_h_history, float *d_h_s2,
                           gscan_dtype_t in_dtype, float a_shift,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes gscan_backward_full_ex needs for this shape (0 if unsupported). */
size_t gscan_backward_full_workspace_bytes(int64_t B, int64_t K, int64_t SH2, int64_t D,
                                           gscan_dtype_t in_dtype);

/*
 * Batch-parallel bias-gradient reduction (design spec section "IQN Bias Grad
 * Reduce"; the KAN and Q-denoise bias gradients share the pattern):
 *   out[j] = sum over r < rows of grad[r][j],  j < cols
 * grad: fp32 row-major [rows][cols] device memory (4-byte aligned; may be
 * NULL when rows == 0), out: fp32 [cols], overwritten (zeros when rows == 0).
 * Two phases with fp64 partials summed in a fixed order, so the result is
 * bitwise reproducible.  workspace: at least
 * gscan_bias_grad_reduce_workspace_bytes(rows, cols), 256-byte aligned, or
 * NULL to allocate stream-ordered.  Errors: INVALID_ARGUMENT (null pointer,
 * rows < 0, cols < 1), UNSUPPORTED_SHAPE (rows x cols above 2^40),
 * MISALIGNED, WORKSPACE_TOO_SMALL, HIP_ERROR; nothing is launched on error.
 */
int gscan_bias_grad_reduce(const float *grad, int64_t rows, int64_t cols, float *out,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * CIFG matrix-memory update, independent mode (BURT-IMMA CUDA Kernel API
 * Reference, section 2.3 batched_cifg_update with shared_memory_mode =
 * false: section 2.2 cifg_update, steps 1-4, for every sample):
 *   concat = [h_b ; x_b]                                (d_model + d_input)
 *   f      = sigmoid(W_f @ concat + b_f)                (d_model)
 *   C_b[i][j] <- f[i] * C_b[i][j] + (1 - f[i]) * h_b[i] * h_b[j]
 * in place on C_batch [B][d_model][d_model] (fp32 row-major); H [B][d_model],
 * X [B][d_input] (may be NULL when d_input == 0), W_f [d_model][d_model +
 * d_input] (its first d_model columns act on h), b_f [d_model]; all fp32
 * device memory, C_batch, H, X, W_f 16-byte aligned, b_f 4-byte aligned.
 * C_batch must not overlap any input.  Step 5 of cifg_update (the optional
 * spectral clip by a power iteration) and the shared-memory mode are not
 * provided.  Arithmetic is fp32; the gate's dot product is summed in a
 * fixed order (bitwise reproducible).  Errors: INVALID_ARGUMENT (null
 * pointer, B < 1, d_model < 1, d_input < 0, overlap), UNSUPPORTED_SHAPE
 * (d_model or d_input not a multiple of 4, d_model > 16384,
 * B * d_model^2 > 2^40), MISALIGNED, HIP_ERROR; nothing is launched on error.
 */
int gscan_batched_cifg_update(float *C_batch, const float *H, const float *X,
                              const float *W_f, const float *b_f, int64_t B, int64_t d_model,
                              int64_t d_input, hipStream_t stream);

/* Workspace bytes of gscan_bias_grad_reduce (0 for invalid sizes). */
size_t gscan_bias_grad_reduce_workspace_bytes(int64_t rows, int64_t cols);

/*
 * Backward without any allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, kernels and result as
 * gscan_backward_ex, with the weight-gradient partials kept in a static
 * device array of GSCAN_NOALLOC_SCRATCH_BYTES bytes inside the library
 * (one per GPU, held until the process ends) instead of a workspace.  It
 * calls no allocating routine; the array's device address is looked up once
 * per device (the device current at the call).
 *
 * Limit: shapes whose gscan_backward_workspace_bytes() exceeds
 * GSCAN_NOALLOC_SCRATCH_BYTES are rejected with
 * GSCAN_ERR_WORKSPACE_TOO_SMALL before anything is launched (all five
 * named workloads but the widest fit).
 * Concurrency: every call on one GPU uses that GPU's one array, so calls
 * that overlap on a GPU (on different streams, or from different threads
 * without ordering) race; calls ordered on one stream are safe.  The array
 * keeps the last call's partials; nothing in it needs to start at zero.
 * Other arguments, layouts and errors as for gscan_backward_ex.
 */
#define GSCAN_NOALLOC_SCRATCH_BYTES (16u << 20)

int gscan_backward_noalloc(const void *h_history, const void *h_s2,
                           const float *W_A, const float *W_B, const float *W_C,
                           int64_t B, int64_t K, int64_t SH2, int64_t D,
                           const float *d_context, float *dW_A, float *dW_B, float *dW_C,
                           gscan_dtype_t in_dtype, float a_shift, hipStream_t stream);

/* Workspace bytes gscan_backward_ex needs for this shape (0 if unsupported). */
size_t gscan_backward_workspace_bytes(int64_t B, int64_t K, int64_t SH2, int64_t D,
                                      gscan_dtype_t in_dtype);

/* Static description of a status code. */
const char *gscan_status_string(int status);

/* Detail of the calling thread's most recent failure ("" if none). */
const char *gscan_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int gscan_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GSCAN_H */
