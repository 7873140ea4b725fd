// Batch-parallel bias-gradient reduction: out[j] = sum over rows of
// grad[r][j] for a row-major [rows][cols] fp32 gradient (design spec section
// "IQN Bias Grad Reduce": block partials, then a reduction of the partials;
// the KAN and Q-denoise bias gradients follow the same pattern).
//
// Phase 1: workgroup b sums a contiguous range of rows into one fp64 partial
// per column.  For cols <= 256 the 256 threads form P = 256 / cols row
// phases x cols columns, so consecutive threads read consecutive addresses;
// the P phase sums of a column are then added in phase order.  For wider
// gradients each thread owns columns t, t+256, ... over all rows of the range.
// Phase 2: one workgroup per column adds the partials in a fixed tree order
// (fp64) and rounds once to fp32.  No atomics: bitwise reproducible.
#include <cstdint>

#include "gscan_internal.h"

namespace gscan {
namespace {

constexpr int kColThreads = 256;

__global__ void __launch_bounds__(kColThreads)
gscan_colsum_partial_kernel(const float *__restrict__ grad, int64_t rows, int64_t cols,
                            int64_t rows_per_block, double *__restrict__ part)
{
    __shared__ double red[kColThreads];
    const int t = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < rows ? r0 + rows_per_block : rows;
    double *out = part + (int64_t)blockIdx.x * cols;
    if (cols <= kColThreads) {
        const int c = (int)cols;
        const int P = kColThreads / c;
        const int j = t % c, q = t / c;
        double acc = 0.0;
        if (q < P) {
            int64_t r = r0 + q;
            // four rows in flight, added in row order
            for (; r + 3 * P < r1; r += 4 * P) {
                const float v0 = grad[r * c + j], v1 = grad[(r + P) * c + j];
                const float v2 = grad[(r + 2 * P) * c + j], v3 = grad[(r + 3 * P) * c + j];
                acc += (double)v0;
                acc += (double)v1;
                acc += (double)v2;
                acc += (double)v3;
            }
            for (; r < r1; r += P) acc += (double)grad[r * c + j];
        }
        red[t] = acc;
        __syncthreads();
        if (t < c) {
            double s = 0.0;
            for (int p = 0; p < P; ++p) s += red[p * c + t];
            out[t] = s;
        }
    } else {
        for (int64_t j = t; j < cols; j += kColThreads) {
            double acc = 0.0;
            for (int64_t r = r0; r < r1; ++r) acc += (double)grad[r * cols + j];
            out[j] = acc;
        }
    }
}

// workgroup b takes columns b, b + gridDim.x, ... (the grid is capped, so any
// column count the validation admits is covered)
__global__ void __launch_bounds__(kColThreads)
gscan_colsum_final_kernel(const double *__restrict__ part, int64_t nparts, int64_t cols,
                          float *__restrict__ out)
{
    __shared__ double red[kColThreads];
    const int t = threadIdx.x;
    for (int64_t j = blockIdx.x; j < cols; j += gridDim.x) {
        double s = 0.0;
        for (int64_t p = t; p < nparts; p += kColThreads) s += part[p * cols + j];
        red[t] = s;
        __syncthreads();
        for (int w = kColThreads / 2; w > 0; w >>= 1) {
            if (t < w) red[t] += red[t + w];
            __syncthreads();
        }
        if (t == 0) out[j] = (float)red[0];
        __syncthreads();  // red is rewritten for the next column
    }
}

constexpr int64_t kFinalMaxGrid = 65536;

// rows per phase-1 workgroup: about 4096 elements each, at most 1024 groups
int64_t colsum_blocks(int64_t rows, int64_t cols, int64_t *rows_per_block)
{
    const int64_t elems = rows * cols;
    int64_t g = (elems + 4095) / 4096;
    if (g > 1024) g = 1024;
    if (g < 1) g = 1;
    int64_t rpb = (rows + g - 1) / g;
    if (rpb < 1) rpb = 1;
    g = rows > 0 ? (rows + rpb - 1) / rpb : 1;
    *rows_per_block = rpb;
    return g;
}

}  // namespace

size_t colsum_workspace_bytes(int64_t rows, int64_t cols)
{
    int64_t rpb;
    const int64_t g = colsum_blocks(rows, cols, &rpb);
    return (size_t)(g * cols) * sizeof(double);
}

hipError_t launch_colsum(const float *grad, int64_t rows, int64_t cols, float *out,
                         void *workspace, hipStream_t st)
{
    int64_t rpb;
    const int64_t g = colsum_blocks(rows, cols, &rpb);
    double *part = static_cast<double *>(workspace);
    hipLaunchKernelGGL(gscan_colsum_partial_kernel, dim3((unsigned)g), dim3(kColThreads), 0, st,
                       grad, rows, cols, rpb, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t fg = cols < kFinalMaxGrid ? cols : kFinalMaxGrid;
    hipLaunchKernelGGL(gscan_colsum_final_kernel, dim3((unsigned)fg), dim3(kColThreads), 0, st,
                       part, g, cols, out);
    return hipGetLastError();
}

}  // namespace gscan
