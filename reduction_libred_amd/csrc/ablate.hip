// ablate.hip -- the reduction lesson's five block-reduction versions
// ("03_shared_memory_sync_reduction.py", demo 3), rebuilt for gfx950 as an
// ablation ladder. Each rung writes one float32 partial per 256-thread block
// through an LDS tree, the way the lesson does; rung k differs from rung k-1
// by the one change the lesson makes:
//   1 interleaved addressing: at step s only threads with tid % 2s == 0 add,
//     so most lanes of every wave sit idle (divergence);
//   2 interleaved addressing by consecutive threads: thread t adds at index
//     2*s*t, so the lanes are busy but hit LDS at stride 2s (bank conflicts);
//   3 sequential addressing: the first s threads add s[t + s] into s[t]
//     (contiguous, conflict-free), but half the threads idle from step one;
//   4 first add during load: each block covers 2*256 elements and each
//     thread adds two loads before the tree;
//   5 version 4, but the tree stops at 128 values and wave 0 finishes with
//     register shuffles: lanes fold 128 -> 64, then shuffle-down by 32, 16,
//     8, 4, 2, 1 (the lesson folds to a 32-lane warp and shuffles five times;
//     a gfx950 wave has 64 lanes, so here it is one fold and six shuffles).
// Elements past n read as 0 (the lesson's ladder assumes n is a multiple of
// the block's span; here any n works). The partials are then summed in
// float64 and rounded once, as the lesson's host does (by the library's own
// float sum, in the C ABI layer).
#include "device_common.hpp"
#include "launch.hpp"

namespace libred {

constexpr int B = kRungBlock;

__device__ __forceinline__ float load_or_zero(const float* __restrict__ x, size_t i, size_t n) {
    return i < n ? x[i] : 0.0f;
}

__global__ __launch_bounds__(B) void rung1_divergent(const float* __restrict__ x, size_t n,
                                                     float* __restrict__ partials) {
    __shared__ float s[B];
    const unsigned t = threadIdx.x;
    s[t] = load_or_zero(x, (size_t)blockIdx.x * B + t, n);
    __syncthreads();
    for (unsigned k = 1; k < B; k *= 2) {
        if (t % (2 * k) == 0) s[t] += s[t + k];
        __syncthreads();
    }
    if (t == 0) partials[blockIdx.x] = s[0];
}

__global__ __launch_bounds__(B) void rung2_strided(const float* __restrict__ x, size_t n,
                                                   float* __restrict__ partials) {
    __shared__ float s[B];
    const unsigned t = threadIdx.x;
    s[t] = load_or_zero(x, (size_t)blockIdx.x * B + t, n);
    __syncthreads();
    for (unsigned k = 1; k < B; k *= 2) {
        const unsigned idx = 2 * k * t;
        if (idx < B) s[idx] += s[idx + k];
        __syncthreads();
    }
    if (t == 0) partials[blockIdx.x] = s[0];
}

// The sequential tree: for k = B/2, B/4, ..., stop the first k threads add
// s[t + k] into s[t], one barrier per step.
__device__ __forceinline__ void sequential_tree(float* s, unsigned t, unsigned stop) {
    for (unsigned k = B / 2; k >= stop; k >>= 1) {
        if (t < k) s[t] += s[t + k];
        __syncthreads();
    }
}

__global__ __launch_bounds__(B) void rung3_sequential(const float* __restrict__ x, size_t n,
                                                      float* __restrict__ partials) {
    __shared__ float s[B];
    const unsigned t = threadIdx.x;
    s[t] = load_or_zero(x, (size_t)blockIdx.x * B + t, n);
    __syncthreads();
    sequential_tree(s, t, 1);
    if (t == 0) partials[blockIdx.x] = s[0];
}

__global__ __launch_bounds__(B) void rung4_first_add(const float* __restrict__ x, size_t n,
                                                     float* __restrict__ partials) {
    __shared__ float s[B];
    const unsigned t = threadIdx.x;
    const size_t i = (size_t)blockIdx.x * (2 * B) + t;
    s[t] = load_or_zero(x, i, n) + load_or_zero(x, i + B, n);
    __syncthreads();
    sequential_tree(s, t, 1);
    if (t == 0) partials[blockIdx.x] = s[0];
}

__global__ __launch_bounds__(B) void rung5_wave_shuffle(const float* __restrict__ x, size_t n,
                                                        float* __restrict__ partials) {
    __shared__ float s[B];
    const unsigned t = threadIdx.x;
    const size_t i = (size_t)blockIdx.x * (2 * B) + t;
    s[t] = load_or_zero(x, i, n) + load_or_zero(x, i + B, n);
    __syncthreads();
    sequential_tree(s, t, 2 * kWave);   // down to 128 values
    if (t < kWave) {                    // wave 0 only (wave-uniform branch)
        float v = s[t] + s[t + kWave];
        for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_down(v, off, kWave);
        if (t == 0) partials[blockIdx.x] = v;
    }
}

size_t rung_elems_per_block(int rung) { return (rung == 4 || rung == 5) ? 2 * B : B; }

hipError_t launch_rung(int rung, const float* x, size_t n, float* partials, size_t nblocks,
                       hipStream_t stream) {
    const dim3 grid((unsigned)nblocks), block(B);
    switch (rung) {
        case 1: hipLaunchKernelGGL(rung1_divergent, grid, block, 0, stream, x, n, partials); break;
        case 2: hipLaunchKernelGGL(rung2_strided, grid, block, 0, stream, x, n, partials); break;
        case 3: hipLaunchKernelGGL(rung3_sequential, grid, block, 0, stream, x, n, partials); break;
        case 4: hipLaunchKernelGGL(rung4_first_add, grid, block, 0, stream, x, n, partials); break;
        case 5: hipLaunchKernelGGL(rung5_wave_shuffle, grid, block, 0, stream, x, n, partials); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace libred
