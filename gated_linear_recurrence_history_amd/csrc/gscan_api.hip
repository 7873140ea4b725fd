// C ABI of the gated temporal scan (declared in include/gscan.h).
//
// Every call validates all arguments before enqueueing anything (the
// validate-then-launch order of the Kimi-K3 KDA decode launcher page, whose
// entry point checks every length before its first allocation or launch),
// returns a status code instead of aborting, and records a detail string in
// thread-local storage.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "gscan.h"
#include "gscan_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

bool aligned16(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// hipGetLastError() returns and resets the calling thread's most recent HIP
// error, whichever call raised it.  Each entry point clears it once its
// arguments have passed validation and before it enqueues anything, so the
// checks after its own launches report only its own failures.
void clear_stale_error()
{
    (void)hipGetLastError();
}

int check_common(const void *hh, const void *hs2, const float *WA, const float *WB,
                 const float *WC, int64_t B, int64_t K, int64_t SH2, int64_t D, int dtype,
                 gscan::Plan *plan)
{
    if (!hh || !hs2 || !WA || !WB || !WC)
        return fail(GSCAN_ERR_INVALID_ARGUMENT, "null input pointer");
    if (B <= 0 || K <= 0 || SH2 <= 0 || D <= 0)
        return fail(GSCAN_ERR_INVALID_ARGUMENT,
                    "sizes must be positive (B=%lld K=%lld SH2=%lld D=%lld)", (long long)B,
                    (long long)K, (long long)SH2, (long long)D);
    if (dtype != GSCAN_F32 && dtype != GSCAN_BF16)
        return fail(GSCAN_ERR_INVALID_ARGUMENT, "unknown input dtype %d", dtype);
    if (!gscan::make_plan(B, K, SH2, D, dtype, plan))
        return fail(GSCAN_ERR_UNSUPPORTED_SHAPE,
                    "unsupported shape B=%lld K=%lld SH2=%lld D=%lld (need 16<=SH2<=1024, "
                    "SH2%%16==0, 16<=D<=256, D%%16==0)",
                    (long long)B, (long long)K, (long long)SH2, (long long)D);
    if (!aligned16(hh) || !aligned16(hs2) || !aligned16(WA) || !aligned16(WB) || !aligned16(WC))
        return fail(GSCAN_ERR_MISALIGNED, "input pointers must be 16-byte aligned");
    return GSCAN_OK;
}

int check_backward(const void *h_history, const void *h_s2, const float *W_A, const float *W_B,
                   const float *W_C, int64_t B, int64_t K, int64_t SH2, int64_t D,
                   const float *d_context, int dtype, gscan::Plan *plan)
{
    int st = check_common(h_history, h_s2, W_A, W_B, W_C, B, K, SH2, D, dtype, plan);
    if (st != GSCAN_OK) return st;
    if (!d_context) return fail(GSCAN_ERR_INVALID_ARGUMENT, "null d_context");
    if (!aligned16(d_context))
        return fail(GSCAN_ERR_MISALIGNED, "d_context must be 16-byte aligned");
    return GSCAN_OK;
}

int check_outputs(const float *dW_A, const float *dW_B, const float *dW_C)
{
    if (!dW_A || !dW_B || !dW_C) return fail(GSCAN_ERR_INVALID_ARGUMENT, "null dW pointer");
    if (!aligned16(dW_A) || !aligned16(dW_B) || !aligned16(dW_C))
        return fail(GSCAN_ERR_MISALIGNED, "dW pointers must be 16-byte aligned");
    return GSCAN_OK;
}

// Workspace of the backward with input gradients: the partials, then
// dL/dA | dL/dB per row and dL/dC per sample (each 256-byte aligned).
struct FullLayout {
    size_t dab = 0, dc = 0, bytes = 0;
};

FullLayout full_layout(const gscan::Plan &p)
{
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    FullLayout f;
    if (p.fused_dinput()) {  // phase 1 writes the input gradients: partials only
        f.dab = f.dc = 0;
        f.bytes = p.ws_bytes;
        return f;
    }
    if (p.bwd_split || p.generic) {  // the workspace already holds both
        f.dab = p.split_dab;
        f.dc = p.split_dc;
        f.bytes = p.ws_bytes;
        return f;
    }
    f.dab = up(p.ws_bytes);
    f.dc = up(f.dab + (size_t)(p.B * p.K) * (size_t)(2 * p.D) * sizeof(float));
    f.bytes = f.dc + (size_t)p.B * (size_t)p.D * sizeof(float);
    return f;
}

int check_workspace(const void *workspace, size_t workspace_bytes, const gscan::Plan &plan)
{
    if (!workspace) return fail(GSCAN_ERR_INVALID_ARGUMENT, "null workspace");
    if (workspace_bytes < plan.ws_bytes)
        return fail(GSCAN_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu",
                    workspace_bytes, plan.ws_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(GSCAN_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    return GSCAN_OK;
}

// ------------------------------------------- static scratch (no allocation)
// The weight-gradient partials of gscan_backward_noalloc live in this
// file-scope device array instead of caller or runtime memory.  Its host-side
// name is only a stand-in: host code uses the device address that
// hipGetSymbolAddress returns, looked up once per device (with that device
// current) and kept.  Each device holds its own copy for the life of the
// process.
static __device__ __align__(256) unsigned char scratch[GSCAN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`.
int current_scratch(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(GSCAN_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(GSCAN_ERR_HIP, "device index %d outside 0..%d", dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(GSCAN_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s",
                        dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GSCAN_OK;
}

// A caller's forward workspace, checked only where the plan uses one.
int check_forward_workspace(const void *workspace, size_t workspace_bytes,
                            const gscan::Plan &plan)
{
    if (!plan.fwd_scratch || !workspace) return GSCAN_OK;
    if (workspace_bytes < plan.fwd_scratch)
        return fail(GSCAN_ERR_WORKSPACE_TOO_SMALL, "forward workspace %zu bytes < required %zu",
                    workspace_bytes, plan.fwd_scratch);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(GSCAN_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    return GSCAN_OK;
}

// The forward with the scratch its plan asks for (the materialised
// projections of the shapes outside the fused kernels): the caller's
// workspace, or memory from the stream-ordered allocator released on the
// same stream.
int run_forward(const gscan::Plan &plan, const void *hh, const void *hs2, const float *WA,
                const float *WB, const float *WC, float a_shift, const gscan::CtxOut &out,
                void *workspace, hipStream_t stream)
{
    if (plan.fwd_scratch && workspace) {
        hipError_t e = gscan::launch_forward(plan, hh, hs2, WA, WB, WC, a_shift, out, workspace,
                                             stream);
        if (e != hipSuccess)
            return fail(GSCAN_ERR_HIP, "forward launch failed: %s", hipGetErrorString(e));
        return GSCAN_OK;
    }
    void *sc = nullptr;
    if (plan.fwd_scratch) {
        hipError_t e = hipMallocAsync(&sc, plan.fwd_scratch, stream);
        if (e != hipSuccess)
            return fail(GSCAN_ERR_HIP, "forward scratch allocation (%zu bytes) failed: %s",
                        plan.fwd_scratch, hipGetErrorString(e));
    }
    hipError_t e = gscan::launch_forward(plan, hh, hs2, WA, WB, WC, a_shift, out, sc, stream);
    if (sc) {
        hipError_t f = hipFreeAsync(sc, stream);
        if (e == hipSuccess) e = f;
    }
    if (e != hipSuccess)
        return fail(GSCAN_ERR_HIP, "forward launch failed: %s", hipGetErrorString(e));
    return GSCAN_OK;
}

}  // namespace

extern "C" {

int gscan_forward_ex(const void *h_history, const void *h_s2, const float *W_A, const float *W_B,
                     const float *W_C, int64_t B, int64_t K, int64_t SH2, int64_t D,
                     float *context_out, gscan_dtype_t in_dtype, float a_shift,
                     void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    gscan::Plan plan;
    int st = check_common(h_history, h_s2, W_A, W_B, W_C, B, K, SH2, D, (int)in_dtype, &plan);
    if (st != GSCAN_OK) return st;
    if (!context_out) return fail(GSCAN_ERR_INVALID_ARGUMENT, "null context_out");
    if (!aligned16(context_out))
        return fail(GSCAN_ERR_MISALIGNED, "context_out must be 16-byte aligned");
    if ((st = check_forward_workspace(workspace, workspace_bytes, plan)) != GSCAN_OK) return st;
    clear_stale_error();
    gscan::CtxOut out;
    out.ctx = context_out;
    st = run_forward(plan, h_history, h_s2, W_A, W_B, W_C, a_shift, out, workspace, stream);
    if (st != GSCAN_OK) return st;
    g_last_error[0] = '\0';
    return GSCAN_OK;
}

int gscan_forward_enrich(const void *h_history, const void *h_s2, const float *W_A,
                         const float *W_B, const float *W_C, int64_t B, int64_t K, int64_t SH2,
                         int64_t D, float *context_out, float *h_enriched, int64_t ld_enriched,
                         int64_t col_offset, gscan_dtype_t in_dtype, float a_shift,
                         void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    gscan::Plan plan;
    int st = check_common(h_history, h_s2, W_A, W_B, W_C, B, K, SH2, D, (int)in_dtype, &plan);
    if (st != GSCAN_OK) return st;
    if (!h_enriched) return fail(GSCAN_ERR_INVALID_ARGUMENT, "null h_enriched");
    if (ld_enriched < D || col_offset < 0 || col_offset > ld_enriched - D)
        return fail(GSCAN_ERR_INVALID_ARGUMENT,
                    "need ld_enriched >= D and 0 <= col_offset <= ld_enriched - D (ld=%lld "
                    "offset=%lld D=%lld)",
                    (long long)ld_enriched, (long long)col_offset, (long long)D);
    if (ld_enriched > (int64_t(1) << 40) / B)
        return fail(GSCAN_ERR_UNSUPPORTED_SHAPE, "B x ld_enriched above 2^40");
    if ((reinterpret_cast<uintptr_t>(h_enriched) & 3u) != 0)
        return fail(GSCAN_ERR_MISALIGNED, "h_enriched must be 4-byte aligned");
    if (context_out) {
        if (!aligned16(context_out))
            return fail(GSCAN_ERR_MISALIGNED, "context_out must be 16-byte aligned");
        // the two outputs must not overlap (each element has one writer)
        const uintptr_t c0 = reinterpret_cast<uintptr_t>(context_out);
        const uintptr_t c1 = c0 + (uintptr_t)(B * D) * sizeof(float);
        const uintptr_t e0 = reinterpret_cast<uintptr_t>(h_enriched);
        const uintptr_t e1 = e0 + (uintptr_t)((B - 1) * ld_enriched + col_offset + D) * sizeof(float);
        if (c0 < e1 && e0 < c1)
            return fail(GSCAN_ERR_INVALID_ARGUMENT, "context_out overlaps h_enriched");
    }
    if ((st = check_forward_workspace(workspace, workspace_bytes, plan)) != GSCAN_OK) return st;
    clear_stale_error();
    gscan::CtxOut out;
    out.ctx = context_out;
    out.enr = h_enriched + col_offset;
    out.ld = ld_enriched;
    st = run_forward(plan, h_history, h_s2, W_A, W_B, W_C, a_shift, out, workspace, stream);
    if (st != GSCAN_OK) return st;
    g_last_error[0] = '\0';
    return GSCAN_OK;
}

int gscan_forward(const void *h_history, const void *h_s2, const float *W_A, const float *W_B,
                  const float *W_C, int64_t B, int64_t K, int64_t SH2, int64_t D,
                  float *context_out, hipStream_t stream)
{
    return gscan_forward_ex(h_history, h_s2, W_A, W_B, W_C, B, K, SH2, D, context_out, GSCAN_F32,
                            0.0f, nullptr, 0, stream);
}

size_t gscan_forward_workspace_bytes(int64_t B, int64_t K, int64_t SH2, int64_t D,
                                     gscan_dtype_t in_dtype)
{
    if (B <= 0 || K <= 0 || SH2 <= 0 || D <= 0) return 0;
    gscan::Plan plan;
    if (!gscan::make_plan(B, K, SH2, D, (int)in_dtype, &plan)) return 0;
    return plan.fwd_scratch;
}

size_t gscan_backward_workspace_bytes(int64_t B, int64_t K, int64_t SH2, int64_t D,
                                      gscan_dtype_t in_dtype)
{
    gscan::Plan plan;
    if (!gscan::make_plan(B, K, SH2, D, (int)in_dtype, &plan)) return 0;
    return plan.ws_bytes;
}

int gscan_backward_ex(const void *h_history, const void *h_s2, const float *W_A,
                      const float *W_B, const float *W_C, int64_t B, int64_t K, int64_t SH2,
                      int64_t D, const float *d_context, float *dW_A, float *dW_B, float *dW_C,
                      gscan_dtype_t in_dtype, float a_shift, void *workspace,
                      size_t workspace_bytes, hipStream_t stream)
{
    gscan::Plan plan;
    int st = check_backward(h_history, h_s2, W_A, W_B, W_C, B, K, SH2, D, d_context,
                            (int)in_dtype, &plan);
    if (st != GSCAN_OK) return st;
    if ((st = check_outputs(dW_A, dW_B, dW_C)) != GSCAN_OK) return st;
    if (workspace && (st = check_workspace(workspace, workspace_bytes, plan)) != GSCAN_OK)
        return st;
    clear_stale_error();
    void *ws = workspace;
    if (!ws) {
        hipError_t e = hipMallocAsync(&ws, plan.ws_bytes, stream);
        if (e != hipSuccess)
            return fail(GSCAN_ERR_HIP, "workspace allocation of %zu bytes failed: %s",
                        plan.ws_bytes, hipGetErrorString(e));
    }
    float *part = static_cast<float *>(ws);
    hipError_t e = gscan::launch_backward_partials(plan, h_history, h_s2, W_A, W_B, W_C, a_shift,
                                                   d_context, part, nullptr, nullptr, nullptr,
                                                   nullptr, stream);
    if (e == hipSuccess) e = gscan::launch_backward_reduce(plan, part, dW_A, dW_B, dW_C, stream);
    if (!workspace) {
        hipError_t f = hipFreeAsync(ws, stream);
        if (e == hipSuccess) e = f;
    }
    if (e != hipSuccess)
        return fail(GSCAN_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
    g_last_error[0] = '\0';
    return GSCAN_OK;
}

size_t gscan_backward_full_workspace_bytes(int64_t B, int64_t K, int64_t SH2, int64_t D,
                                           gscan_dtype_t in_dtype)
{
    if (B <= 0 || K <= 0 || SH2 <= 0 || D <= 0) return 0;
    gscan::Plan plan;
    if (!gscan::make_plan(B, K, SH2, D, (int)in_dtype, &plan)) return 0;
    return full_layout(plan).bytes;
}

int gscan_backward_full_ex(const void *h_history, const void *h_s2, const float *W_A,
                           const float *W_B, const float *W_C, int64_t B, int64_t K, int64_t SH2,
                           int64_t D, const float *d_context, float *dW_A, float *dW_B,
                           float *dW_C, float *d_h_history, float *d_h_s2,
                           gscan_dtype_t in_dtype, float a_shift, void *workspace,
                           size_t workspace_bytes, hipStream_t stream)
{
    gscan::Plan plan;
    int st = check_backward(h_history, h_s2, W_A, W_B, W_C, B, K, SH2, D, d_context,
                            (int)in_dtype, &plan);
    if (st != GSCAN_OK) return st;
    if ((st = check_outputs(dW_A, dW_B, dW_C)) != GSCAN_OK) return st;
    if (!d_h_history || !d_h_s2)
        return fail(GSCAN_ERR_INVALID_ARGUMENT, "null input-gradient pointer");
    if (!aligned16(d_h_history) || !aligned16(d_h_s2))
        return fail(GSCAN_ERR_MISALIGNED, "input-gradient pointers must be 16-byte aligned");
    const FullLayout lay = full_layout(plan);
    if (workspace) {
        if (workspace_bytes < lay.bytes)
            return fail(GSCAN_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu",
                        workspace_bytes, lay.bytes);
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
            return fail(GSCAN_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    }
    clear_stale_error();
    void *ws = workspace;
    if (!ws) {
        hipError_t e = hipMallocAsync(&ws, lay.bytes, stream);
        if (e != hipSuccess)
            return fail(GSCAN_ERR_HIP, "workspace allocation of %zu bytes failed: %s", lay.bytes,
                        hipGetErrorString(e));
    }
    char *base = static_cast<char *>(ws);
    float *part = reinterpret_cast<float *>(base);
    hipError_t e;
    if (plan.fused_dinput()) {
        // phase 1 writes d_h_history and d_h_s2 itself
        e = gscan::launch_backward_partials(plan, h_history, h_s2, W_A, W_B, W_C, a_shift,
                                            d_context, part, nullptr, nullptr, d_h_history,
                                            d_h_s2, stream);
        if (e == hipSuccess) e = gscan::launch_backward_reduce(plan, part, dW_A, dW_B, dW_C, stream);
    } else {
        float *dab = reinterpret_cast<float *>(base + lay.dab);
        float *dc = reinterpret_cast<float *>(base + lay.dc);
        e = gscan::launch_backward_partials(plan, h_history, h_s2, W_A, W_B, W_C, a_shift,
                                            d_context, part, dab, dc, nullptr, nullptr, stream);
        if (e == hipSuccess) e = gscan::launch_backward_reduce(plan, part, dW_A, dW_B, dW_C, stream);
        if (e == hipSuccess && !plan.adjoints_final())
            e = gscan::launch_adjoint(plan, dab, dc, d_context, a_shift, stream);
        if (e == hipSuccess)
            e = gscan::launch_dinput(dab, W_A, W_B, D, 2 * D, SH2, B * K, d_h_history, stream);
        if (e == hipSuccess) e = gscan::launch_dinput(dc, W_C, nullptr, D, D, SH2, B, d_h_s2, stream);
    }
    if (!workspace) {
        hipError_t f = hipFreeAsync(ws, stream);
        if (e == hipSuccess) e = f;
    }
    if (e != hipSuccess)
        return fail(GSCAN_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
    g_last_error[0] = '\0';
    return GSCAN_OK;
}

size_t gscan_bias_grad_reduce_workspace_bytes(int64_t rows, int64_t cols)
{
    if (rows < 0 || cols < 1 || rows > (int64_t(1) << 40) / cols) return 0;
    return gscan::colsum_workspace_bytes(rows, cols);
}

int gscan_bias_grad_reduce(const float *grad, int64_t rows, int64_t cols, float *out,
                           void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!out || (rows > 0 && !grad))
        return fail(GSCAN_ERR_INVALID_ARGUMENT, "null pointer");
    if (rows < 0 || cols < 1)
        return fail(GSCAN_ERR_INVALID_ARGUMENT, "need rows >= 0 and cols >= 1 (rows=%lld cols=%lld)",
                    (long long)rows, (long long)cols);
    if (rows > (int64_t(1) << 40) / cols)
        return fail(GSCAN_ERR_UNSUPPORTED_SHAPE, "rows x cols above 2^40");
    if ((reinterpret_cast<uintptr_t>(grad) & 3u) != 0 || (reinterpret_cast<uintptr_t>(out) & 3u) != 0)
        return fail(GSCAN_ERR_MISALIGNED, "grad and out must be 4-byte aligned");
    const size_t need = gscan::colsum_workspace_bytes(rows, cols);
    if (workspace) {
        if (workspace_bytes < need)
            return fail(GSCAN_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu",
                        workspace_bytes, need);
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
            return fail(GSCAN_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    }
    clear_stale_error();
    void *ws = workspace;
    if (!ws) {
        hipError_t e = hipMallocAsync(&ws, need, stream);
        if (e != hipSuccess)
            return fail(GSCAN_ERR_HIP, "workspace allocation of %zu bytes failed: %s", need,
                        hipGetErrorString(e));
    }
    hipError_t e = gscan::launch_colsum(grad, rows, cols, out, ws, stream);
    if (!workspace) {
        hipError_t f = hipFreeAsync(ws, stream);
        if (e == hipSuccess) e = f;
    }
    if (e != hipSuccess)
        return fail(GSCAN_ERR_HIP, "bias-gradient reduction launch failed: %s", hipGetErrorString(e));
    g_last_error[0] = '\0';
    return GSCAN_OK;
}

int gscan_backward_partials(const void *h_history, const void *h_s2, const float *W_A,
                            const float *W_B, const float *W_C, int64_t B, int64_t K,
                            int64_t SH2, int64_t D, const float *d_context,
                            gscan_dtype_t in_dtype, float a_shift, void *workspace,
                            size_t workspace_bytes, hipStream_t stream)
{
    gscan::Plan plan;
    int st = check_backward(h_history, h_s2, W_A, W_B, W_C, B, K, SH2, D, d_context,
                            (int)in_dtype, &plan);
    if (st != GSCAN_OK) return st;
    if ((st = check_workspace(workspace, workspace_bytes, plan)) != GSCAN_OK) return st;
    clear_stale_error();
    hipError_t e = gscan::launch_backward_partials(plan, h_history, h_s2, W_A, W_B, W_C, a_shift,
                                                   d_context, static_cast<float *>(workspace),
                                                   nullptr, nullptr, nullptr, nullptr, stream);
    if (e != hipSuccess)
        return fail(GSCAN_ERR_HIP, "backward phase 1 launch failed: %s", hipGetErrorString(e));
    g_last_error[0] = '\0';
    return GSCAN_OK;
}

int gscan_backward_reduce(const void *workspace, size_t workspace_bytes, int64_t B, int64_t K,
                          int64_t SH2, int64_t D, gscan_dtype_t in_dtype, float *dW_A,
                          float *dW_B, float *dW_C, hipStream_t stream)
{
    gscan::Plan plan;
    if (B <= 0 || K <= 0 || SH2 <= 0 || D <= 0)
        return fail(GSCAN_ERR_INVALID_ARGUMENT, "sizes must be positive");
    if (in_dtype != GSCAN_F32 && in_dtype != GSCAN_BF16)
        return fail(GSCAN_ERR_INVALID_ARGUMENT, "unknown input dtype %d", (int)in_dtype);
    if (!gscan::make_plan(B, K, SH2, D, (int)in_dtype, &plan))
        return fail(GSCAN_ERR_UNSUPPORTED_SHAPE, "unsupported shape");
    int st;
    if ((st = check_workspace(workspace, workspace_bytes, plan)) != GSCAN_OK) return st;
    if ((st = check_outputs(dW_A, dW_B, dW_C)) != GSCAN_OK) return st;
    clear_stale_error();
    hipError_t e = gscan::launch_backward_reduce(plan, static_cast<const float *>(workspace), dW_A,
                                                 dW_B, dW_C, stream);
    if (e != hipSuccess)
        return fail(GSCAN_ERR_HIP, "backward phase 2 launch failed: %s", hipGetErrorString(e));
    g_last_error[0] = '\0';
    return GSCAN_OK;
}

int gscan_backward_noalloc(const void *h_history, const void *h_s2, const float *W_A,
                           const float *W_B, const float *W_C, int64_t B, int64_t K, int64_t SH2,
                           int64_t D, const float *d_context, float *dW_A, float *dW_B,
                           float *dW_C, gscan_dtype_t in_dtype, float a_shift,
                           hipStream_t stream)
{
    gscan::Plan plan;
    int st = check_backward(h_history, h_s2, W_A, W_B, W_C, B, K, SH2, D, d_context,
                            (int)in_dtype, &plan);
    if (st != GSCAN_OK) return st;
    if ((st = check_outputs(dW_A, dW_B, dW_C)) != GSCAN_OK) return st;
    if (plan.ws_bytes > (size_t)GSCAN_NOALLOC_SCRATCH_BYTES)
        return fail(GSCAN_ERR_WORKSPACE_TOO_SMALL,
                    "shape B=%lld K=%lld SH2=%lld D=%lld needs %zu bytes of partials, more than "
                    "the %zu-byte static scratch of gscan_backward_noalloc (use "
                    "gscan_backward_ex with a workspace)",
                    (long long)B, (long long)K, (long long)SH2, (long long)D, plan.ws_bytes,
                    (size_t)GSCAN_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if ((st = current_scratch(&ws)) != GSCAN_OK) return st;
    clear_stale_error();
    // phase 1 overwrites every partial it leaves for phase 2: nothing in the
    // scratch needs to start at zero
    float *part = static_cast<float *>(ws);
    hipError_t e = gscan::launch_backward_partials(plan, h_history, h_s2, W_A, W_B, W_C, a_shift,
                                                   d_context, part, nullptr, nullptr, nullptr,
                                                   nullptr, stream);
    if (e == hipSuccess) e = gscan::launch_backward_reduce(plan, part, dW_A, dW_B, dW_C, stream);
    if (e != hipSuccess)
        return fail(GSCAN_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
    g_last_error[0] = '\0';
    return GSCAN_OK;
}

int gscan_backward(const void *h_history, const void *h_s2, const float *W_A, const float *W_B,
                   const float *W_C, int64_t B, int64_t K, int64_t SH2, int64_t D,
                   const float *d_context, float *dW_A, float *dW_B, float *dW_C,
                   hipStream_t stream)
{
    return gscan_backward_ex(h_history, h_s2, W_A, W_B, W_C, B, K, SH2, D, d_context, dW_A, dW_B,
                             dW_C, GSCAN_F32, 0.0f, nullptr, 0, stream);
}

int gscan_batched_cifg_update(float *C_batch, const float *H, const float *X, const float *W_f,
                              const float *b_f, int64_t B, int64_t d_model, int64_t d_input,
                              hipStream_t stream)
{
    if (!C_batch || !H || !W_f || !b_f || (d_input > 0 && !X))
        return fail(GSCAN_ERR_INVALID_ARGUMENT, "null pointer");
    if (B < 1 || d_model < 1 || d_input < 0)
        return fail(GSCAN_ERR_INVALID_ARGUMENT,
                    "need B >= 1, d_model >= 1, d_input >= 0 (B=%lld d_model=%lld d_input=%lld)",
                    (long long)B, (long long)d_model, (long long)d_input);
    if (d_model % 4 != 0 || d_input % 4 != 0 || d_model > 16384 || d_input > (int64_t(1) << 24) ||
        B > (int64_t(1) << 40) / (d_model * d_model))
        return fail(GSCAN_ERR_UNSUPPORTED_SHAPE,
                    "unsupported shape B=%lld d_model=%lld d_input=%lld (need d_model and d_input "
                    "multiples of 4, d_model <= 16384, B*d_model^2 <= 2^40)",
                    (long long)B, (long long)d_model, (long long)d_input);
    if (!aligned16(C_batch) || !aligned16(H) || (d_input > 0 && !aligned16(X)) ||
        !aligned16(W_f) || (reinterpret_cast<uintptr_t>(b_f) & 3u) != 0)
        return fail(GSCAN_ERR_MISALIGNED,
                    "C_batch, H, X, W_f must be 16-byte aligned and b_f 4-byte aligned");
    // C_batch is updated in place and must not overlap any input
    const uintptr_t c0 = reinterpret_cast<uintptr_t>(C_batch);
    const uintptr_t c1 = c0 + (uintptr_t)(B * d_model * d_model) * sizeof(float);
    auto overlaps = [&](const void *p, int64_t n) {
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(p);
        return p && n > 0 && a0 < c1 && c0 < a0 + (uintptr_t)n * sizeof(float);
    };
    if (overlaps(H, B * d_model) || overlaps(X, B * d_input) ||
        overlaps(W_f, d_model * (d_model + d_input)) || overlaps(b_f, d_model))
        return fail(GSCAN_ERR_INVALID_ARGUMENT, "C_batch overlaps an input");
    clear_stale_error();
    hipError_t e = gscan::launch_cifg(C_batch, H, d_input > 0 ? X : H, W_f, b_f, B, d_model,
                                      d_input, stream);
    if (e != hipSuccess)
        return fail(GSCAN_ERR_HIP, "CIFG update launch failed: %s", hipGetErrorString(e));
    g_last_error[0] = '\0';
    return GSCAN_OK;
}

const char *gscan_status_string(int status)
{
    switch (status) {
    case GSCAN_OK: return "ok";
    case GSCAN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case GSCAN_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case GSCAN_ERR_MISALIGNED: return "misaligned pointer";
    case GSCAN_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case GSCAN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char *gscan_last_error(void)
{
    return g_last_error;
}

int gscan_version(void)
{
    return 100;  // 0.1.0
}

}  // extern "C"
