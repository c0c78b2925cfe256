// rows_reduce.hip -- per-row (segmented) sum and max of a row-major matrix
// whose rows start `ld` elements apart (ld >= cols; ld == cols is the dense
// case).
//
// The lesson's reduction gives one output per block segment
// ("03_shared_memory_sync_reduction.py", demo 3). Here the segment is a row,
// and two layouts cover the shapes:
//   one wave per row (many rows): a 64-lane wave owns one row at a time, with
//       no LDS, no barrier and no cross-block combine; a 4096-float row is
//       16 KiB, i.e. 16 aligned 16-byte loads per lane;
//   split rows (few long rows): each row is cut across `gx` single-wave
//       blocks that stream tiles of 64*UNROLL vectors dealt round-robin, each
//       storing one partial; a second launch combines each row's partials in
//       index order with one wave per row.
// A row's start may be misaligned when ld is not a multiple of 4, so every
// row peels its own head and tail. Sums accumulate in float64 and round once
// per row.
#include "device_common.hpp"
#include "launch.hpp"

namespace libred {

// Fold row `row` (cols elements) into acc: vectors v0, v0 + vstep, ... of the
// aligned body in loop trips of UNROLL loads spaced 64 vectors apart, with the
// head and tail only when `edges` is set. Wave-uniform arguments.
template <class Op, int UNROLL, bool NT>
__device__ __forceinline__ void fold_row_span(const typename Op::elem_t* __restrict__ row, size_t cols,
                                              size_t first_tile, size_t tile_step, bool edges,
                                              typename Op::acc_t (&acc)[4]) {
    using vec_t = typename Op::vec_t;
    constexpr size_t TILE = (size_t)kWave * UNROLL;
    const int lane = threadIdx.x % kWave;
    const size_t head = head_elems(row, sizeof(typename Op::elem_t), cols);
    const size_t nvec = (cols - head) / Op::kPerVec;
    const size_t tail0 = head + (size_t)Op::kPerVec * nvec;
    const vec_t* __restrict__ rv = reinterpret_cast<const vec_t*>(row + head);
    const size_t ntiles = nvec / TILE;
    for (size_t t = first_tile; t < ntiles; t += tile_step) {
        const vec_t* __restrict__ p = rv + t * TILE + lane;
        vec_t v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = load_vec<NT>(p + u * kWave);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            fold_vec<Op>(acc, v[u], head + (t * TILE + lane + (size_t)u * kWave) * Op::kPerVec);
    }
    for (size_t i = ntiles * TILE + first_tile * kWave + lane; i < nvec; i += tile_step * kWave)
        fold_vec<Op>(acc, load_vec<NT>(rv + i), head + i * Op::kPerVec);
    if (edges) {
        if ((size_t)lane < head) acc[0] = Op::combine(acc[0], Op::lift(row[lane], lane));
        if ((size_t)lane < cols - tail0)
            acc[1] = Op::combine(acc[1], Op::lift(row[tail0 + lane], tail0 + lane));
    }
}

template <class Op, int BLOCK, int UNROLL, bool NT>
__global__ __launch_bounds__(BLOCK) void rows_reduce_kernel(const typename Op::elem_t* __restrict__ x,
                                                            size_t rows, size_t cols, size_t ld,
                                                            typename Op::out_t* __restrict__ out) {
    using acc_t = typename Op::acc_t;
    constexpr int W = BLOCK / kWave;
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

    // Wave-uniform loop over rows: all 64 lanes stay active at the wave reduce.
    for (size_t r = (size_t)blockIdx.x * W + wave; r < rows; r += (size_t)gridDim.x * W) {
        acc_t acc[4] = {Op::identity(), Op::identity(), Op::identity(), Op::identity()};
        fold_row_span<Op, UNROLL, NT>(x + r * ld, cols, 0, 1, true, acc);
        acc_t v = Op::combine(Op::combine(acc[0], acc[1]), Op::combine(acc[2], acc[3]));
        v = wave_reduce<Op>(v);
        if (lane == 0) out[r] = Op::finish(v);
    }
}

// Split rows: block b is split s = b % gx of row r = b / gx.
template <class Op, int UNROLL, bool NT>
__global__ __launch_bounds__(kWave) void rows_split_kernel(const typename Op::elem_t* __restrict__ x,
                                                           size_t cols, size_t ld, unsigned int gx,
                                                           typename Op::acc_t* __restrict__ partials) {
    using acc_t = typename Op::acc_t;
    const size_t r = blockIdx.x / gx;
    const size_t s = blockIdx.x % gx;
    acc_t acc[4] = {Op::identity(), Op::identity(), Op::identity(), Op::identity()};
    fold_row_span<Op, UNROLL, NT>(x + r * ld, cols, s, gx, s == 0, acc);
    acc_t v = Op::combine(Op::combine(acc[0], acc[1]), Op::combine(acc[2], acc[3]));
    v = wave_reduce<Op>(v);
    if (threadIdx.x == 0) partials[blockIdx.x] = v;
}

// One wave per row adds that row's gx partials in index order.
constexpr int kRowsCombineBlock = 256;

template <class Op>
__global__ __launch_bounds__(kRowsCombineBlock) void rows_combine_kernel(
    const typename Op::acc_t* __restrict__ partials, size_t rows, unsigned int gx,
    typename Op::out_t* __restrict__ out) {
    using acc_t = typename Op::acc_t;
    constexpr int W = kRowsCombineBlock / kWave;
    const int lane = threadIdx.x % kWave;
    const size_t r = (size_t)blockIdx.x * W + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (r >= rows) return;  // wave-uniform
    acc_t v = Op::identity();
    for (unsigned int j = lane; j < gx; j += kWave) v = Op::combine(v, partials[r * gx + j]);
    v = wave_reduce<Op>(v);
    if (lane == 0) out[r] = Op::finish(v);
}

bool rows_policy_supported(const RowsPolicy& p) {
    const bool b = p.block == 64 || p.block == 128 || p.block == 256 || p.block == 512;
    const bool u = p.unroll == 1 || p.unroll == 2 || p.unroll == 4 || p.unroll == 8 || p.unroll == 16;
    return b && u && (p.nontemporal == 0 || p.nontemporal == 1) && p.max_blocks >= 1 && p.split >= 0 &&
           p.split <= 2;
}

template <class Op, int BLOCK, int UNROLL>
static hipError_t rows_bu(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                          typename Op::out_t* out, int grid, bool nt, hipStream_t stream) {
    if (nt)
        hipLaunchKernelGGL((rows_reduce_kernel<Op, BLOCK, UNROLL, true>), dim3(grid), dim3(BLOCK), 0,
                           stream, x, rows, cols, ld, out);
    else
        hipLaunchKernelGGL((rows_reduce_kernel<Op, BLOCK, UNROLL, false>), dim3(grid), dim3(BLOCK), 0,
                           stream, x, rows, cols, ld, out);
    return hipGetLastError();
}

template <class Op, int BLOCK>
static hipError_t rows_b(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                         typename Op::out_t* out, int grid, const RowsPolicy& p, hipStream_t stream) {
    const bool nt = p.nontemporal != 0;
    switch (p.unroll) {
        case 1: return rows_bu<Op, BLOCK, 1>(x, rows, cols, ld, out, grid, nt, stream);
        case 2: return rows_bu<Op, BLOCK, 2>(x, rows, cols, ld, out, grid, nt, stream);
        case 4: return rows_bu<Op, BLOCK, 4>(x, rows, cols, ld, out, grid, nt, stream);
        case 8: return rows_bu<Op, BLOCK, 8>(x, rows, cols, ld, out, grid, nt, stream);
        case 16: return rows_bu<Op, BLOCK, 16>(x, rows, cols, ld, out, grid, nt, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class Op, int UNROLL>
static hipError_t rows_split_u(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                               typename Op::out_t* out, unsigned int gx, bool nt, void* ws_partials,
                               hipStream_t stream) {
    auto* partials = static_cast<typename Op::acc_t*>(ws_partials);
    const dim3 grid((unsigned int)(rows * gx));
    if (nt)
        hipLaunchKernelGGL((rows_split_kernel<Op, UNROLL, true>), grid, dim3(kWave), 0, stream, x, cols, ld,
                           gx, partials);
    else
        hipLaunchKernelGGL((rows_split_kernel<Op, UNROLL, false>), grid, dim3(kWave), 0, stream, x, cols, ld,
                           gx, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t W = kRowsCombineBlock / kWave;
    hipLaunchKernelGGL((rows_combine_kernel<Op>), dim3((unsigned int)((rows + W - 1) / W)),
                       dim3(kRowsCombineBlock), 0, stream, partials, rows, gx, out);
    return hipGetLastError();
}

template <class Op>
static hipError_t rows_op(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                          typename Op::out_t* out, const RowsLaunch& L, const RowsPolicy& p,
                          hipStream_t stream) {
    if (L.split_gx > 0) {
        const bool nt = p.nontemporal != 0;
        switch (p.unroll) {
            case 1: return rows_split_u<Op, 1>(x, rows, cols, ld, out, L.split_gx, nt, L.partials, stream);
            case 2: return rows_split_u<Op, 2>(x, rows, cols, ld, out, L.split_gx, nt, L.partials, stream);
            case 4: return rows_split_u<Op, 4>(x, rows, cols, ld, out, L.split_gx, nt, L.partials, stream);
            case 8: return rows_split_u<Op, 8>(x, rows, cols, ld, out, L.split_gx, nt, L.partials, stream);
            case 16: return rows_split_u<Op, 16>(x, rows, cols, ld, out, L.split_gx, nt, L.partials, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (p.block) {
        case 64: return rows_b<Op, 64>(x, rows, cols, ld, out, L.grid, p, stream);
        case 128: return rows_b<Op, 128>(x, rows, cols, ld, out, L.grid, p, stream);
        case 256: return rows_b<Op, 256>(x, rows, cols, ld, out, L.grid, p, stream);
        case 512: return rows_b<Op, 512>(x, rows, cols, ld, out, L.grid, p, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rows_sum_f32(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                               const RowsLaunch& L, const RowsPolicy& p, hipStream_t stream) {
    return rows_op<SumF32>(x, rows, cols, ld, out, L, p, stream);
}

hipError_t launch_rows_max_f32(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                               const RowsLaunch& L, const RowsPolicy& p, hipStream_t stream) {
    return rows_op<MaxF32>(x, rows, cols, ld, out, L, p, stream);
}

}  // namespace libred
