// probe.hip -- measurement probes: a plain device copy (the known-size
// reference that hardware byte counters are scaled by) and a read-only stream
// (the achievable read bandwidth, with as little arithmetic as possible).
// Both take 16-byte aligned pointers; the caller checks that.
#include "device_common.hpp"
#include "launch.hpp"

namespace libred {

constexpr int kProbeBlock = 256;

__global__ __launch_bounds__(kProbeBlock) void copy_f32_kernel(const float* __restrict__ x,
                                                               float* __restrict__ y, size_t n) {
    const size_t nvec = n / 4;
    const f32x4* __restrict__ xv = reinterpret_cast<const f32x4*>(x);
    f32x4* __restrict__ yv = reinterpret_cast<f32x4*>(y);
    const size_t stride = (size_t)gridDim.x * kProbeBlock;
    for (size_t i = (size_t)blockIdx.x * kProbeBlock + threadIdx.x; i < nvec; i += stride)
        yv[i] = xv[i];
    if (blockIdx.x == 0 && threadIdx.x < n - 4 * nvec) y[4 * nvec + threadIdx.x] = x[4 * nvec + threadIdx.x];
}

// Folds every 32-bit word into an xor; stores it only if it equals a value
// chosen at run time, so the loads cannot be removed and nothing is written.
__global__ __launch_bounds__(kProbeBlock) void read_f32_kernel(const float* __restrict__ x, size_t n,
                                                               unsigned int* __restrict__ sink,
                                                               unsigned int magic) {
    const size_t nvec = n / 4;
    const i32x4* __restrict__ xv = reinterpret_cast<const i32x4*>(x);
    const size_t stride = (size_t)gridDim.x * kProbeBlock;
    unsigned int a = 0, b = 0, c = 0, d = 0;
    size_t i = (size_t)blockIdx.x * kProbeBlock + threadIdx.x;
    for (; i + 3 * stride < nvec; i += 4 * stride) {
        const i32x4 v0 = xv[i], v1 = xv[i + stride], v2 = xv[i + 2 * stride], v3 = xv[i + 3 * stride];
        a ^= v0.x ^ v1.x ^ v2.x ^ v3.x;
        b ^= v0.y ^ v1.y ^ v2.y ^ v3.y;
        c ^= v0.z ^ v1.z ^ v2.z ^ v3.z;
        d ^= v0.w ^ v1.w ^ v2.w ^ v3.w;
    }
    for (; i < nvec; i += stride) {
        const i32x4 v = xv[i];
        a ^= v.x; b ^= v.y; c ^= v.z; d ^= v.w;
    }
    const unsigned int h = a ^ (b << 1) ^ (c << 2) ^ (d << 3);
    if (h == magic) sink[0] = h;
}

hipError_t launch_copy_f32(const float* x, float* y, size_t n, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(copy_f32_kernel, dim3(grid), dim3(kProbeBlock), 0, stream, x, y, n);
    return hipGetLastError();
}

hipError_t launch_read_f32(const float* x, size_t n, unsigned int* sink, int grid,
                           hipStream_t stream) {
    hipLaunchKernelGGL(read_f32_kernel, dim3(grid), dim3(kProbeBlock), 0, stream, x, n, sink,
                       0x9E3779B9u);
    return hipGetLastError();
}

}  // namespace libred
