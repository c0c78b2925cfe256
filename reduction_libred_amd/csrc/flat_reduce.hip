// flat_reduce.hip -- single-value reductions (sum f32, sum i32->i64, max f32).
//
// One launch does the whole reduction. The steps follow the block-partial
// scheme of the reduction lesson ("03_shared_memory_sync_reduction.py",
// demo 3), redesigned for wave64 and a persistent grid:
//   1. grid-stride loop of 16-byte loads, `UNROLL` in flight per thread,
//      every element folded into four private accumulators as it arrives
//      (the lesson's version 4 adds while loading; here every load does);
//   2. the misaligned head and the ragged tail (< 4 elements each) are read
//      with scalar loads by block 0; out-of-range lanes contribute nothing;
//   3. wave reduce 64 -> 1 with DPP (the lesson's version 5 does this step
//      with warp shuffles);
//   4. one LDS word per wave, one barrier, wave 0 combines the waves;
//   5. thread 0 stores the block partial;
//   6. the block that finishes last (a counter bumped once per block) combines
//      all partials in index order and stores the result. The lesson notes
//      that blocks cannot wait for each other inside a kernel; the counter
//      lets the last one to arrive do the final step without a second launch,
//      and the fixed index order makes the result independent of which block
//      that is (the simulator page "simt_lab.py", section 5, asks that a
//      kernel's result never depend on block order).
#include "device_common.hpp"
#include "launch.hpp"

namespace libred {

template <class Op, int BLOCK, int UNROLL, bool NT>
__global__ __launch_bounds__(BLOCK) void flat_reduce_kernel(
    const typename Op::elem_t* __restrict__ x, size_t n,
    typename Op::acc_t* __restrict__ partials, unsigned int* __restrict__ ticket,
    typename Op::out_t* __restrict__ out) {
    using acc_t = typename Op::acc_t;
    using vec_t = typename Op::vec_t;
    using elem_t = typename Op::elem_t;
    __shared__ acc_t lds[BLOCK / kWave];
    __shared__ int is_last;

    // Split x into head (scalar), 16-byte aligned body, tail (scalar).
    const size_t head = head_elems(x, sizeof(elem_t), n);
    const size_t nvec = (n - head) / 4;
    const size_t tail0 = head + 4 * nvec;
    const vec_t* __restrict__ xv = reinterpret_cast<const vec_t*>(x + head);

    acc_t acc[4] = {Op::identity(), Op::identity(), Op::identity(), Op::identity()};

    // Step 1: grid-stride body. Each load of a wave covers 1 KiB contiguous.
    const size_t stride = (size_t)gridDim.x * BLOCK;
    size_t i = (size_t)blockIdx.x * BLOCK + threadIdx.x;
    for (; i + (size_t)(UNROLL - 1) * stride < nvec; i += (size_t)UNROLL * stride) {
        vec_t v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = load_vec<NT>(xv + i + (size_t)u * stride);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) accumulate4<Op>(acc, v[u]);
    }
    for (; i < nvec; i += stride) accumulate4<Op>(acc, load_vec<NT>(xv + i));

    // Step 2: head and tail.
    if (blockIdx.x == 0) {
        if (threadIdx.x < head) acc[0] = Op::combine(acc[0], Op::lift(x[threadIdx.x]));
        if (threadIdx.x < n - tail0) acc[1] = Op::combine(acc[1], Op::lift(x[tail0 + threadIdx.x]));
    }

    // Steps 3-4: thread -> wave -> block.
    acc_t v = Op::combine(Op::combine(acc[0], acc[1]), Op::combine(acc[2], acc[3]));
    v = block_reduce<Op, BLOCK>(v, lds);

    if (gridDim.x == 1) {
        if (threadIdx.x == 0) out[0] = Op::finish(v);
        return;
    }

    // Step 5: publish the partial, then take a ticket. The release fence
    // orders the partial before the counter update for every other block.
    if (threadIdx.x == 0) {
        __hip_atomic_store(&partials[blockIdx.x], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const unsigned int prev =
            __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = (prev == gridDim.x - 1);
    }
    __syncthreads();
    if (!is_last) return;  // block-uniform: the whole block leaves together

    // Step 6: the last block. The acquire fence makes every partial visible.
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    acc_t w = Op::identity();
    for (unsigned int j = threadIdx.x; j < gridDim.x; j += BLOCK)
        w = Op::combine(w, __hip_atomic_load(&partials[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    w = block_reduce<Op, BLOCK>(w, lds);
    if (threadIdx.x == 0) {
        out[0] = Op::finish(w);
        __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__global__ void zero_words_kernel(unsigned int* p, size_t words) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

hipError_t launch_zero_words(unsigned int* p, size_t words, hipStream_t stream) {
    hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, stream, p, words);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Policy dispatch: the (block, unroll, nontemporal) triples compiled in.
// ---------------------------------------------------------------------------
bool flat_policy_supported(const FlatPolicy& p) {
    const bool b = p.block == 256 || p.block == 512 || p.block == 1024;
    const bool u = p.unroll == 1 || p.unroll == 2 || p.unroll == 4 || p.unroll == 8 || p.unroll == 16;
    return b && u && (p.nontemporal == 0 || p.nontemporal == 1) && p.blocks_per_cu >= 1;
}

template <class Op, int BLOCK, int UNROLL>
static hipError_t launch_bu(const typename Op::elem_t* x, size_t n, typename Op::out_t* out,
                            int grid, bool nt, const Workspace& ws, hipStream_t stream) {
    auto* partials = static_cast<typename Op::acc_t*>(ws.partials);
    if (nt)
        hipLaunchKernelGGL((flat_reduce_kernel<Op, BLOCK, UNROLL, true>), dim3(grid), dim3(BLOCK), 0,
                           stream, x, n, partials, ws.ticket, out);
    else
        hipLaunchKernelGGL((flat_reduce_kernel<Op, BLOCK, UNROLL, false>), dim3(grid), dim3(BLOCK), 0,
                           stream, x, n, partials, ws.ticket, out);
    return hipGetLastError();
}

template <class Op, int BLOCK>
static hipError_t launch_b(const typename Op::elem_t* x, size_t n, typename Op::out_t* out,
                           int grid, const FlatPolicy& p, const Workspace& ws, hipStream_t stream) {
    const bool nt = p.nontemporal != 0;
    switch (p.unroll) {
        case 1: return launch_bu<Op, BLOCK, 1>(x, n, out, grid, nt, ws, stream);
        case 2: return launch_bu<Op, BLOCK, 2>(x, n, out, grid, nt, ws, stream);
        case 4: return launch_bu<Op, BLOCK, 4>(x, n, out, grid, nt, ws, stream);
        case 8: return launch_bu<Op, BLOCK, 8>(x, n, out, grid, nt, ws, stream);
        case 16: return launch_bu<Op, BLOCK, 16>(x, n, out, grid, nt, ws, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class Op>
static hipError_t launch_op(const typename Op::elem_t* x, size_t n, typename Op::out_t* out,
                            int grid, const FlatPolicy& p, const Workspace& ws, hipStream_t stream) {
    switch (p.block) {
        case 256: return launch_b<Op, 256>(x, n, out, grid, p, ws, stream);
        case 512: return launch_b<Op, 512>(x, n, out, grid, p, ws, stream);
        case 1024: return launch_b<Op, 1024>(x, n, out, grid, p, ws, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_sum_f32(const float* x, size_t n, float* out, int grid, const FlatPolicy& p,
                          const Workspace& ws, hipStream_t stream) {
    return launch_op<SumF32>(x, n, out, grid, p, ws, stream);
}

hipError_t launch_sum_i32_i64(const int32_t* x, size_t n, int64_t* out, int grid,
                              const FlatPolicy& p, const Workspace& ws, hipStream_t stream) {
    return launch_op<SumI32>(x, n, out, grid, p, ws, stream);
}

hipError_t launch_max_f32(const float* x, size_t n, float* out, int grid, const FlatPolicy& p,
                          const Workspace& ws, hipStream_t stream) {
    return launch_op<MaxF32>(x, n, out, grid, p, ws, stream);
}

}  // namespace libred
