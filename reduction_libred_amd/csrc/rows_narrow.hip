// rows_narrow.hip -- per-row sum and max of rows of 1, 2 or 4 floats of a
// contiguous, 16-byte aligned row-major matrix, in registers only.
//
// One output per segment, as the lesson's block partials are one output per
// block ("03_shared_memory_sync_reduction.py", demo 3); here a segment is a
// row of C floats, a quarter of a 16-byte vector or less. Each lane's vector
// holds M = 4 / C whole rows: the lane folds them in order (float64 for the
// sum, the strictly-greater rule for the max) and stores its M results side
// by side. The matrix is cut into tiles of U * 64 vectors; a wave reads a
// tile with U loads per lane, each a coalesced 1 KiB, and writes its
// U * 64 * M results with U stores of 256 * M contiguous bytes, whole
// 128-byte lines when out is 128-byte aligned. Nothing goes through LDS and
// no lane talks to another.
//
// Tiles are dealt to the waves round-robin, and the next tile's loads are
// issued before the current tile is folded and stored. The rows after the
// last whole tile (fewer than U * 64 * M) are reduced by one wave, element
// by element.
#include "device_common.hpp"
#include "launch.hpp"

namespace libred {

namespace {

template <class Op, int C, int U, bool NT>
__global__ __launch_bounds__(kWave) void rows_narrow_kernel(const float* __restrict__ x, size_t rows,
                                                            float* __restrict__ out) {
    static_assert(C == 1 || C == 2 || C == 4, "one vector must hold whole rows");
    using acc_t = typename Op::acc_t;
    constexpr int M = 4 / C;                                 // rows per vector
    constexpr size_t kTileRows = (size_t)U * kWave * M;
    const unsigned int lane = threadIdx.x;
    const f32x4* __restrict__ xv = reinterpret_cast<const f32x4*>(x);
    const size_t ntiles = rows / kTileRows;
    const size_t G = gridDim.x;
    const bool out16 = ((uintptr_t)out & 15) == 0;

    auto load = [&](f32x4 (&v)[U], size_t t) {
        const f32x4* __restrict__ p = xv + t * U * kWave + lane;
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = load_vec<NT>(p + u * kWave);
    };
    auto fold_store = [&](const f32x4 (&v)[U], size_t t) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float res[M];
#pragma unroll
            for (int r = 0; r < M; ++r) {
                acc_t a = Op::identity();
#pragma unroll
                for (int c = 0; c < C; ++c) a = Op::combine(a, Op::lift(v[u][r * C + c], (size_t)c));
                res[r] = Op::finish(a);
            }
            float* __restrict__ o = out + ((t * U + u) * kWave + lane) * M;
            if constexpr (M == 4) {
                if (out16) {
                    f32x4 w = {res[0], res[1], res[2], res[3]};
                    *reinterpret_cast<f32x4*>(o) = w;
                    continue;
                }
            }
#pragma unroll
            for (int r = 0; r < M; ++r) o[r] = res[r];
        }
    };

    // The wave's tiles t0, t0 + G, ... two per loop pass, one register
    // buffer each, the next tile's loads in flight while one is folded.
    size_t t0 = blockIdx.x;  // wave-uniform
    if (t0 < ntiles) {
        size_t n = (ntiles - t0 + G - 1) / G;
        f32x4 a[U], b[U];
        load(a, t0);
        for (; n > 2; n -= 2, t0 += 2 * G) {
            load(b, t0 + G);
            fold_store(a, t0);
            load(a, t0 + 2 * G);
            fold_store(b, t0 + G);
        }
        if (n == 2) {
            load(b, t0 + G);
            fold_store(a, t0);
            fold_store(b, t0 + G);
        } else {
            fold_store(a, t0);
        }
    }
    // Rows after the last whole tile: the wave that would take tile ntiles.
    if (blockIdx.x == ntiles % G) {
        for (size_t r = ntiles * kTileRows + lane; r < rows; r += kWave) {
            acc_t a = Op::identity();
#pragma unroll
            for (int c = 0; c < C; ++c) a = Op::combine(a, Op::lift(x[r * C + c], (size_t)c));
            out[r] = Op::finish(a);
        }
    }
}

template <class Op, int C>
hipError_t launch_c(const float* x, size_t rows, float* out, int grid, bool nt, hipStream_t stream) {
    constexpr int U = kNarrowTileLoads;
    if (nt)
        hipLaunchKernelGGL((rows_narrow_kernel<Op, C, U, true>), dim3(grid), dim3(kWave), 0, stream, x, rows, out);
    else
        hipLaunchKernelGGL((rows_narrow_kernel<Op, C, U, false>), dim3(grid), dim3(kWave), 0, stream, x, rows,
                           out);
    return hipGetLastError();
}

template <class Op>
hipError_t launch_op(const float* x, size_t rows, size_t cols, float* out, int grid, bool nt, hipStream_t stream) {
    switch (cols) {
        case 1: return launch_c<Op, 1>(x, rows, out, grid, nt, stream);
        case 2: return launch_c<Op, 2>(x, rows, out, grid, nt, stream);
        case 4: return launch_c<Op, 4>(x, rows, out, grid, nt, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t rows_narrow_tile_rows(size_t cols) {
    if (cols != 1 && cols != 2 && cols != 4) return 0;
    return (size_t)kNarrowTileLoads * kWave * (4 / cols);
}

hipError_t launch_rows_narrow(int op, const float* x, size_t rows, size_t cols, float* out, int grid, bool nt,
                              hipStream_t stream) {
    if (op == 0) return launch_op<SumF32>(x, rows, cols, out, grid, nt, stream);
    if (op == 1) return launch_op<MaxF32>(x, rows, cols, out, grid, nt, stream);
    return hipErrorInvalidValue;
}

}  // namespace libred
