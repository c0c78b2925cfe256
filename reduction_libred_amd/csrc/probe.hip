// probe.hip -- a plain device copy: the known-size reference that hardware
// byte counters are scaled by. It takes 16-byte aligned pointers; the caller
// checks that. (The read-only probe is the single-value kernel with an xor
// fold; see flat_reduce.hip.)
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

hipError_t launch_copy_f32(const float* x, float* y, size_t n, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(copy_f32_kernel, dim3(grid), dim3(kProbeBlock), 0, stream, x, y, n);
    return hipGetLastError();
}

}  // namespace libred
