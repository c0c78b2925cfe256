// flat_reduce.hpp -- the single-value reduction kernel and its launch-shape
// dispatch, as templates over the reduction operator; the flat_*.hip
// translation units instantiate them for their operators.
//
// The steps follow the block-partial scheme of the reduction lesson
// ("03_shared_memory_sync_reduction.py", demo 3), redesigned for wave64 and a
// persistent grid:
//   1. stream the 16-byte aligned body with `UNROLL` loads in flight per lane,
//      folding every element into four private accumulators as it arrives
//      (the lesson's version 4 adds while loading; here every load does);
//   2. the misaligned head and the ragged tail (< 4 elements each) are read
//      with scalar loads by block 0; lanes with nothing to read add nothing;
//   3. wave reduce 64 -> 1 with DPP (the lesson's version 5 does this step
//      with warp shuffles);
//   4. one LDS word per wave, one barrier, wave 0 combines the waves;
//   5. thread 0 stores the block partial;
//   6. the partials are combined in index order, either by the block that
//      finishes last in the same launch (a counter bumped once per block
//      tells it that it is last), or by a one-block second launch. The lesson
//      notes that blocks cannot wait for each other inside a kernel; both
//      forms respect that, and the fixed index order makes the result
//      independent of which block finishes when (the simulator page
//      "simt_lab.py", section 5, asks that a kernel's result never depend on
//      block order).
//
// Two layouts of step 1 are compiled:
//   kGridStride: thread i of the grid reads vectors i, i + G*T, i + 2*G*T, ...
//       (UNROLL of them per loop trip), so each wave load covers 1 KiB and the
//       grid sweeps the array front to back in G*T*16-byte slabs;
//   kWaveTiles: the body is cut into tiles of 64*UNROLL vectors (UNROLL KiB);
//       wave w of the grid reads tiles w, w + nwaves, ... whole, one 16-byte
//       vector per lane per load, so each wave streams contiguous memory.
//       With `PREFETCH`, the next tile's loads are issued before the current
//       tile is folded, keeping 2*UNROLL KiB in flight per wave.
#pragma once

#include "device_common.hpp"
#include "launch.hpp"

namespace libred {

// Element number of the first element of body vector i (after the head).
#define LIBRED_ELEM(i) (head + (size_t)(i) * Op::kPerVec)

template <class Op, int BLOCK, int UNROLL, bool NT>
__device__ __forceinline__ void body_grid_stride(const typename Op::vec_t* __restrict__ xv, size_t nvec,
                                                 size_t head, typename Op::acc_t (&acc)[4]) {
    using vec_t = typename Op::vec_t;
    const size_t stride = (size_t)gridDim.x * BLOCK;
    size_t i = (size_t)blockIdx.x * BLOCK + threadIdx.x;
    for (; i + (size_t)(UNROLL - 1) * stride < nvec; i += (size_t)UNROLL * stride) {
        vec_t v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = load_vec<NT>(xv + i + (size_t)u * stride);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) fold_vec<Op>(acc, v[u], LIBRED_ELEM(i + (size_t)u * stride));
    }
    for (; i < nvec; i += stride) fold_vec<Op>(acc, load_vec<NT>(xv + i), LIBRED_ELEM(i));
}

// One tile of a wave: UNROLL loads, each of 64 lanes x 16 bytes = 1 KiB.
// With GROUP the loads are held together by a scheduling barrier: for the
// int32 sum the compiler otherwise split the next tile's loads around the
// fold of the current one, leaving half of them in flight during its waits
// (1 GiB: 6.6 -> 7.3 TB/s with the barrier). The other operators keep the
// compiler's own order.
template <class Op>
struct GroupLoads : std::false_type {};
template <>
struct GroupLoads<SumI32> : std::true_type {};

template <bool NT, bool GROUP = false, class V, int UNROLL>
__device__ __forceinline__ void load_tile(V (&v)[UNROLL], const V* __restrict__ p) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = load_vec<NT>(p + u * kWave);
    if constexpr (GROUP) __builtin_amdgcn_sched_barrier(0);
}

// Fold a tile loaded from body vector index v0 (lane's first vector).
// An operator with its own tile fold gets the element number of vector 0's
// first element (vector u starts 64 * kPerVec elements later per step).
template <class Op, int UNROLL>
__device__ __forceinline__ void fold_tile(typename Op::acc_t (&acc)[4],
                                          const typename Op::vec_t (&v)[UNROLL], size_t v0, size_t head) {
    if constexpr (HasTileFold<Op>::value) {
        Op::template fold_tile<UNROLL>(acc, v, LIBRED_ELEM(v0));
    } else {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) fold_vec<Op>(acc, v[u], LIBRED_ELEM(v0 + (size_t)u * kWave));
    }
}

template <class Op, int BLOCK, int UNROLL, bool NT, bool PREFETCH>
__device__ __forceinline__ void body_wave_tiles(const typename Op::vec_t* __restrict__ xv, size_t nvec,
                                                size_t head, typename Op::acc_t (&acc)[4]) {
    using vec_t = typename Op::vec_t;
    constexpr int W = BLOCK / kWave;
    constexpr size_t TILE = (size_t)kWave * UNROLL;  // vectors per tile
    const int lane = threadIdx.x % kWave;
    const size_t wave = (size_t)__builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const size_t nwaves = (size_t)gridDim.x * W;
    const size_t ntiles = nvec / TILE;
    size_t t = (size_t)blockIdx.x * W + wave;  // wave-uniform

    if constexpr (!PREFETCH) {
        for (; t < ntiles; t += nwaves) {
            const vec_t* __restrict__ p = xv + t * TILE + lane;
            vec_t v[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) v[u] = load_vec<NT>(p + u * kWave);
            fold_tile<Op>(acc, v, t * TILE + lane, head);
        }
    } else if (t < ntiles) {
        // Two register buffers, a and b, alternate: the loads of the next
        // tile go into one while the other is folded, so the wait before a
        // fold leaves the next tile's loads in flight.
        constexpr bool G = GroupLoads<Op>::value;
        vec_t a[UNROLL], b[UNROLL];
        load_tile<NT, G>(a, xv + t * TILE + lane);
        while (true) {
            if (t + nwaves >= ntiles) {
                fold_tile<Op>(acc, a, t * TILE + lane, head);
                break;
            }
            load_tile<NT, G>(b, xv + (t + nwaves) * TILE + lane);
            fold_tile<Op>(acc, a, t * TILE + lane, head);
            t += nwaves;
            if (t + nwaves >= ntiles) {
                fold_tile<Op>(acc, b, t * TILE + lane, head);
                break;
            }
            load_tile<NT, G>(a, xv + (t + nwaves) * TILE + lane);
            fold_tile<Op>(acc, b, t * TILE + lane, head);
            t += nwaves;
        }
    }
    // Vectors after the last whole tile (fewer than one tile).
    const size_t w = (size_t)blockIdx.x * W + wave;
    for (size_t i = ntiles * TILE + w * kWave + lane; i < nvec; i += nwaves * kWave)
        fold_vec<Op>(acc, load_vec<NT>(xv + i), LIBRED_ELEM(i));
}

// mode: kCombineTicket (the last block combines), kCombineTwoPass (each
// block stores its partial; combine_partials_kernel runs next; a grid of one
// block stores the result directly) or kPartialsOnly (every block, even a
// lone one, stores its partial).
enum { kPartialsOnly = 2 };

template <class Op, int BLOCK, int UNROLL, bool NT, int LAYOUT, bool PREFETCH>
__global__ __launch_bounds__(BLOCK) void flat_reduce_kernel(
    const typename Op::elem_t* __restrict__ x, size_t n,
    typename Op::acc_t* __restrict__ partials, unsigned int* __restrict__ ticket,
    typename Op::out_t* __restrict__ out, int mode) {
    using acc_t = typename Op::acc_t;
    using vec_t = typename Op::vec_t;
    using elem_t = typename Op::elem_t;
    __shared__ acc_t lds[BLOCK / kWave > 0 ? BLOCK / kWave : 1];
    __shared__ int is_last;

    // Split x into head (scalar), 16-byte aligned body, tail (scalar).
    const size_t head = head_elems(x, sizeof(elem_t), n);
    const size_t nvec = (n - head) / Op::kPerVec;
    const size_t tail0 = head + (size_t)Op::kPerVec * nvec;
    const vec_t* __restrict__ xv = reinterpret_cast<const vec_t*>(x + head);

    acc_t acc[4] = {Op::identity(), Op::identity(), Op::identity(), Op::identity()};

    // Step 1: the body.
    if constexpr (LAYOUT == kGridStride)
        body_grid_stride<Op, BLOCK, UNROLL, NT>(xv, nvec, head, acc);
    else
        body_wave_tiles<Op, BLOCK, UNROLL, NT, PREFETCH>(xv, nvec, head, acc);

    // An operator that deferred part of its fold finishes it here.
    if constexpr (HasResolve<Op>::value) Op::template resolve<UNROLL, NT>(acc, x);

    // Step 2: head and tail.
    if (blockIdx.x == 0) {
        if (threadIdx.x < head) acc[0] = Op::combine(acc[0], Op::lift(x[threadIdx.x], threadIdx.x));
        if (threadIdx.x < n - tail0)
            acc[1] = Op::combine(acc[1], Op::lift(x[tail0 + threadIdx.x], tail0 + threadIdx.x));
    }

    // Steps 3-4: thread -> wave -> block.
    acc_t v = Op::combine(Op::combine(acc[0], acc[1]), Op::combine(acc[2], acc[3]));
    v = block_reduce<Op, BLOCK>(v, lds);

    if (mode == kPartialsOnly) {
        if (threadIdx.x == 0) partials[blockIdx.x] = v;
        return;
    }
    if (gridDim.x == 1) {
        if (threadIdx.x == 0) out[0] = Op::finish(v);
        return;
    }
    if (mode == kCombineTwoPass) {
        if (threadIdx.x == 0) partials[blockIdx.x] = v;
        return;
    }

    // Step 5: publish the partial, then take a ticket. The release fence
    // orders the partial before the counter update for every other block; the
    // block that draws the last ticket acquires before it reads any partial.
    if (threadIdx.x == 0) {
        partials[blockIdx.x] = v;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const unsigned int prev =
            __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = (prev == gridDim.x - 1);
        if (is_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    if (!is_last) return;  // block-uniform: the whole block leaves together

    // Step 6: the last block combines the partials in index order.
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    acc_t w = Op::identity();
    for (unsigned int j = threadIdx.x; j < gridDim.x; j += BLOCK) w = Op::combine(w, partials[j]);
    w = block_reduce<Op, BLOCK>(w, lds);
    if (threadIdx.x == 0) {
        out[0] = Op::finish(w);
        __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Step 6 as a second launch: one wave combines the np partials in a fixed
// order. Lane l takes partials l, l + 64, l + 128, ... with eight loads in
// flight at a time (one memory latency for up to 512 partials), then the wave
// reduce combines the lanes. No LDS and no barrier.
constexpr int kCombineBlock = kWave;
constexpr int kCombineBatch = 8;

template <class Op>
__global__ __launch_bounds__(kCombineBlock) void combine_partials_kernel(
    const typename Op::acc_t* __restrict__ partials, unsigned int np, typename Op::out_t* __restrict__ out) {
    using acc_t = typename Op::acc_t;
    const unsigned int lane = threadIdx.x;
    acc_t w = Op::identity();
    for (unsigned int j0 = 0; j0 < np; j0 += kWave * kCombineBatch) {
        acc_t v[kCombineBatch];
#pragma unroll
        for (int k = 0; k < kCombineBatch; ++k) {
            const unsigned int j = j0 + k * kWave + lane;
            v[k] = j < np ? partials[j] : Op::identity();
        }
#pragma unroll
        for (int k = 0; k < kCombineBatch; ++k) w = Op::combine(w, v[k]);
    }
    w = wave_reduce<Op>(w);
    if (lane == 0) out[0] = Op::finish(w);
}

// ---------------------------------------------------------------------------
// Policy dispatch: the (layout, block, unroll, nontemporal, prefetch) shapes
// compiled in: the default shapes and a small set around them for the
// launch-shape comparisons.
//   grid-stride: block 256 / 1024, unroll 1 / 4 / 8
//   wave tiles:  block 64 / 256 / 1024, unroll 4 / 8 / 16, prefetch 0 / 1
// ---------------------------------------------------------------------------
template <class Op, int BLOCK, int UNROLL, int LAYOUT, bool PREFETCH>
inline hipError_t launch_shape(const typename Op::elem_t* x, size_t n, typename Op::out_t* out,
                               int grid, const FlatPolicy& p, const Workspace& ws, hipStream_t stream) {
    auto* partials = static_cast<typename Op::acc_t*>(ws.partials);
    const int mode = out == nullptr ? (int)kPartialsOnly : p.combine;
    if (p.nontemporal)
        hipLaunchKernelGGL((flat_reduce_kernel<Op, BLOCK, UNROLL, true, LAYOUT, PREFETCH>), dim3(grid),
                           dim3(BLOCK), 0, stream, x, n, partials, ws.ticket, out, mode);
    else
        hipLaunchKernelGGL((flat_reduce_kernel<Op, BLOCK, UNROLL, false, LAYOUT, PREFETCH>), dim3(grid),
                           dim3(BLOCK), 0, stream, x, n, partials, ws.ticket, out, mode);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || grid == 1 || mode != (int)kCombineTwoPass) return e;
    hipLaunchKernelGGL((combine_partials_kernel<Op>), dim3(1), dim3(kCombineBlock), 0, stream,
                       partials, (unsigned int)grid, out);
    return hipGetLastError();
}

template <class Op, int BLOCK>
inline hipError_t launch_grid_stride(const typename Op::elem_t* x, size_t n, typename Op::out_t* out,
                                     int grid, const FlatPolicy& p, const Workspace& ws,
                                     hipStream_t stream) {
    switch (p.unroll) {
        case 1: return launch_shape<Op, BLOCK, 1, kGridStride, false>(x, n, out, grid, p, ws, stream);
        case 4: return launch_shape<Op, BLOCK, 4, kGridStride, false>(x, n, out, grid, p, ws, stream);
        case 8: return launch_shape<Op, BLOCK, 8, kGridStride, false>(x, n, out, grid, p, ws, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class Op, int BLOCK, bool PREFETCH>
inline hipError_t launch_tiles_p(const typename Op::elem_t* x, size_t n, typename Op::out_t* out,
                                 int grid, const FlatPolicy& p, const Workspace& ws, hipStream_t stream) {
    switch (p.unroll) {
        case 4: return launch_shape<Op, BLOCK, 4, kWaveTiles, PREFETCH>(x, n, out, grid, p, ws, stream);
        case 8: return launch_shape<Op, BLOCK, 8, kWaveTiles, PREFETCH>(x, n, out, grid, p, ws, stream);
        case 16: return launch_shape<Op, BLOCK, 16, kWaveTiles, PREFETCH>(x, n, out, grid, p, ws, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class Op, int BLOCK>
inline hipError_t launch_tiles(const typename Op::elem_t* x, size_t n, typename Op::out_t* out,
                               int grid, const FlatPolicy& p, const Workspace& ws, hipStream_t stream) {
    if (p.prefetch) return launch_tiles_p<Op, BLOCK, true>(x, n, out, grid, p, ws, stream);
    return launch_tiles_p<Op, BLOCK, false>(x, n, out, grid, p, ws, stream);
}

template <class Op>
inline hipError_t launch_op(const typename Op::elem_t* x, size_t n, typename Op::out_t* out,
                            int grid, const FlatPolicy& p, const Workspace& ws, hipStream_t stream) {
    if (p.layout == kGridStride) {
        switch (p.block) {
            case 256: return launch_grid_stride<Op, 256>(x, n, out, grid, p, ws, stream);
            case 1024: return launch_grid_stride<Op, 1024>(x, n, out, grid, p, ws, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (p.block) {
        case 64: return launch_tiles<Op, 64>(x, n, out, grid, p, ws, stream);
        case 256: return launch_tiles<Op, 256>(x, n, out, grid, p, ws, stream);
        case 1024: return launch_tiles<Op, 1024>(x, n, out, grid, p, ws, stream);
        default: return hipErrorInvalidValue;
    }
}

#undef LIBRED_ELEM

}  // namespace libred
