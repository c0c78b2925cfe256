// probe.hip -- a plain device copy: the known-size reference that hardware
// byte counters are scaled by (it takes 16-byte aligned pointers; the caller
// checks that); the LDS bank probe; the cross-lane primitives alone; and a
// fill of library scratch with a poison word. (The load-only read probe is
// in read_probe.hip.)
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

// LDS bank probe (the reduction lesson's demo 1, for a 64-lane wave): LDS word
// i holds i; lane l reads word (l * stride) mod kLdsProbeWords, or l / 2 for
// stride -1, `iters` times. Each address also depends on the previous value
// read through `zero` (0 at run time), so the loads cannot be hoisted out of
// the loop. The lanes' totals are summed into *sink with one atomic per
// lane. Reading SQ_LDS_BANK_CONFLICT against SQ_INSTS_LDS for each stride
// gives the bank geometry.
__global__ __launch_bounds__(64) void lds_stride_kernel(int stride, int iters, unsigned int zero,
                                                        unsigned int* __restrict__ sink) {
    __shared__ unsigned int lds[kLdsProbeWords];
    for (int i = threadIdx.x; i < kLdsProbeWords; i += 64) lds[i] = (unsigned int)i;
    __syncthreads();
    const unsigned int lane = threadIdx.x;
    const unsigned int base =
        stride < 0 ? lane / 2 : (lane * (unsigned int)stride) % (unsigned int)kLdsProbeWords;
    unsigned int acc = 0;
    for (int k = 0; k < iters; ++k) acc += lds[base + (acc & zero)];
    atomicAdd(sink, acc);
}

hipError_t launch_lds_stride(int stride, int iters, unsigned int* sink, hipStream_t stream) {
    hipLaunchKernelGGL(lds_stride_kernel, dim3(1), dim3(64), 0, stream, stride, iters, 0u, sink);
    return hipGetLastError();
}

// The production wave reduce on its own: wave w reduces in[64w .. 64w + 63]
// with the DPP sequence of wave_reduce<Op> and lane 0 stores out[w].
template <class Op>
__global__ __launch_bounds__(64) void wave_reduce_probe_kernel(const typename Op::acc_t* __restrict__ in,
                                                               typename Op::acc_t* __restrict__ out) {
    const typename Op::acc_t v = wave_reduce<Op>(in[(size_t)blockIdx.x * 64 + threadIdx.x]);
    if (threadIdx.x == 0) out[blockIdx.x] = v;
}

hipError_t launch_wave_reduce_probe(int op, const void* in, size_t nwaves, void* out, hipStream_t stream) {
    const dim3 grid((unsigned)nwaves), block(64);
    switch (op) {
        case 0:
            hipLaunchKernelGGL(wave_reduce_probe_kernel<SumF32>, grid, block, 0, stream,
                               static_cast<const double*>(in), static_cast<double*>(out));
            break;
        case 1:
            hipLaunchKernelGGL(wave_reduce_probe_kernel<SumI32>, grid, block, 0, stream,
                               static_cast<const int64_t*>(in), static_cast<int64_t*>(out));
            break;
        case 2:
            hipLaunchKernelGGL(wave_reduce_probe_kernel<MaxF32>, grid, block, 0, stream,
                               static_cast<const float*>(in), static_cast<float*>(out));
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The register shuffle rung 5 uses: out[l] = value of lane l + offset, or the
// lane's own value when l + offset is past the wave.
__global__ __launch_bounds__(64) void shfl_down_probe_kernel(const float* __restrict__ in, int offset,
                                                             float* __restrict__ out) {
    out[threadIdx.x] = __shfl_down(in[threadIdx.x], (unsigned)offset, kWave);
}

hipError_t launch_shfl_down_probe(const float* in, int offset, float* out, hipStream_t stream) {
    hipLaunchKernelGGL(shfl_down_probe_kernel, dim3(1), dim3(64), 0, stream, in, offset, out);
    return hipGetLastError();
}

// p[i] = value for i < words, with ordinary vector stores.
__global__ void fill_words_kernel(unsigned int* __restrict__ p, size_t words, unsigned int value) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x)
        p[i] = value;
}

hipError_t launch_fill_words(unsigned int* p, size_t words, unsigned int value, hipStream_t stream) {
    hipLaunchKernelGGL(fill_words_kernel, dim3(256), dim3(256), 0, stream, p, words, value);
    return hipGetLastError();
}

hipError_t launch_copy_f32(const float* x, float* y, size_t n, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(copy_f32_kernel, dim3(grid), dim3(kProbeBlock), 0, stream, x, y, n);
    return hipGetLastError();
}

}  // namespace libred
