// Measurement helper, not part of the scan: a read-only stream over a
// device buffer, the ceiling against which the scan's read-dominated passes
// are compared (bench.py).  Each workgroup reads one contiguous chunk of the
// buffer, sixteen 16-byte pieces in flight per thread, and folds them into
// one word so that no load can be dropped (of the layouts tried on the
// MI355X -- grid-strided or chunked, 4 to 16 loads in flight, 512 to 16384
// workgroups, with or without non-temporal loads -- this one read fastest).
// Built as libgscan_calib.so, separate from the scan library.
#include <cstddef>
#include <cstdint>
#include <hip/hip_runtime.h>

namespace {

constexpr int kThreads = 256;
constexpr int kGrid = 2048;
constexpr int kUnroll = 16;

typedef unsigned int u4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kThreads)
gscan_calib_read_kernel(const u4 *__restrict__ p, int64_t n, unsigned *__restrict__ out)
{
    __shared__ unsigned red[kThreads];
    // workgroup b: pieces [b * n / grid, (b + 1) * n / grid)
    const int64_t lo = (int64_t)blockIdx.x * n / gridDim.x;
    const int64_t hi = (int64_t)(blockIdx.x + 1) * n / gridDim.x;
    const u4 *q = p + lo;
    const int64_t m = hi - lo;
    u4 acc = {0u, 0u, 0u, 0u};
    for (int64_t i = threadIdx.x; i < m; i += (int64_t)kThreads * kUnroll) {
        u4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = i + u * kThreads < m ? q[i + u * kThreads] : u4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
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
    return kGrid;
}

// Reads `bytes` bytes (a multiple of 16, 16-byte aligned) at device pointer
// `p` once; writes gscan_calib_read_grid() words to device memory `out`.
// Returns 0, or a HIP error code.
int gscan_calib_read(const void *p, size_t bytes, unsigned *out, hipStream_t stream)
{
    if (!p || !out || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(p) & 15u) != 0)
        return (int)hipErrorInvalidValue;
    (void)hipGetLastError();
    hipLaunchKernelGGL(gscan_calib_read_kernel, dim3(kGrid), dim3(kThreads), 0, stream,
                       static_cast<const u4 *>(p), (int64_t)(bytes / 16), out);
    return (int)hipGetLastError();
}

}  // extern "C"
