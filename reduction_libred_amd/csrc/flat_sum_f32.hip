// flat_sum_f32.hip -- the float32 sum (the headline path), its partials-only
// form, the workspace zero-fill and the launch-shape check. The kernel
// template and its steps are in flat_reduce.hpp.
#include "flat_reduce.hpp"

namespace libred {

__global__ void zero_words_kernel(unsigned int* p, size_t words) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

hipError_t launch_zero_words(unsigned int* p, size_t words, hipStream_t stream) {
    hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, stream, p, words);
    return hipGetLastError();
}

bool flat_policy_supported(const FlatPolicy& p) {
    if (p.blocks_per_cu < 1 || (p.nontemporal != 0 && p.nontemporal != 1)) return false;
    if (p.combine != (int)kCombineTicket && p.combine != (int)kCombineTwoPass) return false;
    if (p.layout == kGridStride) {
        const bool b = p.block == 256 || p.block == 1024;
        const bool u = p.unroll == 1 || p.unroll == 4 || p.unroll == 8;
        return b && u && p.prefetch == 0;
    }
    if (p.layout == kWaveTiles) {
        const bool b = p.block == 64 || p.block == 256 || p.block == 1024;
        const bool u = p.unroll == 4 || p.unroll == 8 || p.unroll == 16;
        return b && u && (p.prefetch == 0 || p.prefetch == 1);
    }
    return false;
}

hipError_t launch_sum_f32(const float* x, size_t n, float* out, int grid, const FlatPolicy& p,
                          const Workspace& ws, hipStream_t stream) {
    return launch_op<SumF32>(x, n, out, grid, p, ws, stream);
}

hipError_t launch_sum_f32_partials(const float* x, size_t n, double* partials, int grid,
                                   const FlatPolicy& p, hipStream_t stream) {
    Workspace ws;
    ws.ticket = nullptr;
    ws.partials = partials;
    ws.max_partials = (size_t)grid;
    return launch_op<SumF32>(x, n, nullptr, grid, p, ws, stream);
}

}  // namespace libred
