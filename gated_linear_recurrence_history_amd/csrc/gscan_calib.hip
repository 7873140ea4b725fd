// Measurement helper, not part of the scan: a read-only stream over a
// device buffer, the ceiling against which the scan's read-dominated passes
// are compared (bench.py).  Each thread reads 16-byte pieces in a
// grid-stride loop, four in flight, and folds them into one word per
// workgroup so that no load can be dropped.  Built as libgscan_calib.so,
// separate from the scan library.
#include <cstddef>
#include <cstdint>
#include <hip/hip_runtime.h>

namespace {

constexpr int kThreads = 256;

typedef unsigned int u4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kThreads)
gscan_calib_read_kernel(const u4 *__restrict__ p, int64_t n, unsigned *__restrict__ out)
{
    __shared__ unsigned red[kThreads];
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    u4 acc = {0u, 0u, 0u, 0u};
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n; i += stride) acc ^= p[i];
    red[threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] ^= red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

}  // namespace

extern "C" {

// Words written to `out` by gscan_calib_read (one per workgroup).
int gscan_calib_read_grid(void)
{
    return 4096;
}

// Reads `bytes` bytes (a multiple of 16, 16-byte aligned) at device pointer
// `p` once; writes gscan_calib_read_grid() words to device memory `out`.
// Returns 0, or a HIP error code.
int gscan_calib_read(const void *p, size_t bytes, unsigned *out, hipStream_t stream)
{
    if (!p || !out || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(p) & 15u) != 0)
        return (int)hipErrorInvalidValue;
    (void)hipGetLastError();
    hipLaunchKernelGGL(gscan_calib_read_kernel, dim3(4096), dim3(kThreads), 0, stream,
                       static_cast<const u4 *>(p), (int64_t)(bytes / 16), out);
    return (int)hipGetLastError();
}

}  // extern "C"
