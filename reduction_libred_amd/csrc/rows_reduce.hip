// rows_reduce.hip -- per-row (segmented) sum and max of a row-major matrix.
//
// One 64-lane wave owns one row at a time: no LDS, no barrier and no
// cross-block combine. This is the lesson's "one output per block segment"
// ("03_shared_memory_sync_reduction.py", demo 3) with the segment shrunk to
// a wave, which suits rows of a few thousand elements: a 4096-float row is
// 16 KiB, i.e. 16 aligned 16-byte loads per lane. Each row's start may be
// misaligned when cols is not a multiple of 4, so every row peels its own
// head and tail. Sums accumulate in float64 and round once per row.
#include "device_common.hpp"
#include "launch.hpp"

namespace libred {

template <class Op, int BLOCK, int UNROLL, bool NT>
__global__ __launch_bounds__(BLOCK) void rows_reduce_kernel(const typename Op::elem_t* __restrict__ x,
                                                            size_t rows, size_t cols,
                                                            typename Op::out_t* __restrict__ out) {
    using acc_t = typename Op::acc_t;
    using vec_t = typename Op::vec_t;
    using elem_t = typename Op::elem_t;
    constexpr int W = BLOCK / kWave;
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

    // Wave-uniform loop over rows: all 64 lanes stay active at the wave reduce.
    for (size_t r = (size_t)blockIdx.x * W + wave; r < rows; r += (size_t)gridDim.x * W) {
        const elem_t* row = x + r * cols;
        const size_t head = head_elems(row, sizeof(elem_t), cols);
        const size_t nvec = (cols - head) / 4;
        const size_t tail0 = head + 4 * nvec;
        const vec_t* __restrict__ rv = reinterpret_cast<const vec_t*>(row + head);

        acc_t acc[4] = {Op::identity(), Op::identity(), Op::identity(), Op::identity()};
        size_t j = lane;
        for (; j + (size_t)(UNROLL - 1) * kWave < nvec; j += (size_t)UNROLL * kWave) {
            vec_t v[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) v[u] = load_vec<NT>(rv + j + (size_t)u * kWave);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) accumulate4<Op>(acc, v[u]);
        }
        for (; j < nvec; j += kWave) accumulate4<Op>(acc, load_vec<NT>(rv + j));
        if ((size_t)lane < head) acc[0] = Op::combine(acc[0], Op::lift(row[lane]));
        if ((size_t)lane < cols - tail0) acc[1] = Op::combine(acc[1], Op::lift(row[tail0 + lane]));

        acc_t v = Op::combine(Op::combine(acc[0], acc[1]), Op::combine(acc[2], acc[3]));
        v = wave_reduce<Op>(v);
        if (lane == 0) out[r] = Op::finish(v);
    }
}

bool rows_policy_supported(const RowsPolicy& p) {
    const bool b = p.block == 64 || p.block == 128 || p.block == 256 || p.block == 512;
    const bool u = p.unroll == 1 || p.unroll == 2 || p.unroll == 4 || p.unroll == 8 || p.unroll == 16;
    return b && u && (p.nontemporal == 0 || p.nontemporal == 1) && p.max_blocks >= 1;
}

template <class Op, int BLOCK, int UNROLL>
static hipError_t rows_bu(const typename Op::elem_t* x, size_t rows, size_t cols,
                          typename Op::out_t* out, int grid, bool nt, hipStream_t stream) {
    if (nt)
        hipLaunchKernelGGL((rows_reduce_kernel<Op, BLOCK, UNROLL, true>), dim3(grid), dim3(BLOCK), 0,
                           stream, x, rows, cols, out);
    else
        hipLaunchKernelGGL((rows_reduce_kernel<Op, BLOCK, UNROLL, false>), dim3(grid), dim3(BLOCK), 0,
                           stream, x, rows, cols, out);
    return hipGetLastError();
}

template <class Op, int BLOCK>
static hipError_t rows_b(const typename Op::elem_t* x, size_t rows, size_t cols,
                         typename Op::out_t* out, int grid, const RowsPolicy& p, hipStream_t stream) {
    const bool nt = p.nontemporal != 0;
    switch (p.unroll) {
        case 1: return rows_bu<Op, BLOCK, 1>(x, rows, cols, out, grid, nt, stream);
        case 2: return rows_bu<Op, BLOCK, 2>(x, rows, cols, out, grid, nt, stream);
        case 4: return rows_bu<Op, BLOCK, 4>(x, rows, cols, out, grid, nt, stream);
        case 8: return rows_bu<Op, BLOCK, 8>(x, rows, cols, out, grid, nt, stream);
        case 16: return rows_bu<Op, BLOCK, 16>(x, rows, cols, out, grid, nt, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class Op>
static hipError_t rows_op(const typename Op::elem_t* x, size_t rows, size_t cols,
                          typename Op::out_t* out, int grid, const RowsPolicy& p, hipStream_t stream) {
    switch (p.block) {
        case 64: return rows_b<Op, 64>(x, rows, cols, out, grid, p, stream);
        case 128: return rows_b<Op, 128>(x, rows, cols, out, grid, p, stream);
        case 256: return rows_b<Op, 256>(x, rows, cols, out, grid, p, stream);
        case 512: return rows_b<Op, 512>(x, rows, cols, out, grid, p, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rows_sum_f32(const float* x, size_t rows, size_t cols, float* out, int grid,
                               const RowsPolicy& p, hipStream_t stream) {
    return rows_op<SumF32>(x, rows, cols, out, grid, p, stream);
}

hipError_t launch_rows_max_f32(const float* x, size_t rows, size_t cols, float* out, int grid,
                               const RowsPolicy& p, hipStream_t stream) {
    return rows_op<MaxF32>(x, rows, cols, out, grid, p, stream);
}

}  // namespace libred
