// rows_narrow.hip -- per-row sum and max of narrow rows (1 to 32 floats) of
// a contiguous, 16-byte aligned row-major matrix, each lane folding whole
// rows.
//
// One output per segment, as the lesson's block partials are one output per
// block ("03_shared_memory_sync_reduction.py", demo 3); here a segment is a
// row of C floats, far shorter than a wave. Each lane owns M = 4 / gcd(C, 4)
// consecutive rows, whose M * C floats are V = M * C / 4 whole 16-byte
// vectors (C = 1: four rows in one vector; C = 3: four rows in three; C = 16:
// one row in four). A wave step covers 64 * M consecutive rows; a tile is U
// steps, U = ceil(8 / V), so that about eight 16-byte loads per lane are in
// flight. The lane folds each of its rows in order (float64 for the sum, the
// strictly-greater rule for the max) and stores its M results side by side:
// a store instruction writes 256 * M contiguous bytes, whole 128-byte lines
// when out is 128-byte aligned. With NT the loads are non-temporal, and so are
// the result stores where a lane stores several results.
//
// A tile is read with coalesced loads (lane l takes vectors l, l + 64, ...,
// 1 KiB per instruction). With V = 1 each lane's vector already holds its
// rows. With V > 1 the tile goes through LDS as it arrived and each lane
// reads back its own V consecutive vectors with 16-byte LDS reads (lanes
// 16 * V bytes apart: for odd V, which covers every width but the multiples
// of 8, no two lanes of a 16-lane pass share a bank). Reading each lane's
// vectors straight from memory instead, 16 * V bytes apart, touched many
// lines per load instruction for little data and ran 2.5 times slower.
//
// Tiles are dealt to the waves round-robin, and the next tile's loads are
// issued before the current tile is folded and stored. The rows after the
// last whole tile (fewer than U * 64 * M) are reduced by one wave, element
// by element.
#include "device_common.hpp"
#include "launch.hpp"

namespace libred {

namespace {

template <int C>
struct NarrowShape {
    static constexpr int M = C % 4 == 0 ? 1 : (C % 2 == 0 ? 2 : 4);  // rows per lane per step
    static constexpr int V = C * M / 4;                               // 16-byte vectors per lane per step
    static constexpr int U = (kNarrowTileLoads + V - 1) / V;          // steps per tile
    static constexpr int L = U * V;                                   // loads per lane per tile
};

template <class Op, int C, bool NT>
__global__ __launch_bounds__(kWave) void rows_narrow_kernel(const float* __restrict__ x, size_t rows,
                                                            float* __restrict__ out) {
    using acc_t = typename Op::acc_t;
    using S = NarrowShape<C>;
    constexpr int M = S::M, V = S::V, U = S::U, L = S::L;
    constexpr size_t kTileRows = (size_t)U * kWave * M;
    // Non-temporal result stores where a lane stores several results (rows
    // of one float: the copy probe's stores gained 5-7% so; 3 floats 5.9 ->
    // 6.5 TB/s); plain ones where it stores one (4 floats: 6.4 plain, 6.0-6.2
    // non-temporal).
    constexpr bool NT_STORE = NT && M > 1;
    __shared__ f32x4 stage[V > 1 ? kWave * L : 1];
    const unsigned int lane = threadIdx.x;
    const f32x4* __restrict__ xv = reinterpret_cast<const f32x4*>(x);
    const size_t ntiles = rows / kTileRows;
    const size_t G = gridDim.x;
    const bool out16 = ((uintptr_t)out & 15) == 0;

    auto load = [&](f32x4 (&v)[L], size_t t) {
        const f32x4* __restrict__ p = xv + t * L * kWave + lane;
#pragma unroll
        for (int i = 0; i < L; ++i) v[i] = load_vec<NT>(p + i * kWave);
    };
    auto fold_store = [&](const f32x4 (&v)[L], size_t t) {
        f32x4 w[L];  // the lane's own vectors: step u's are w[u * V .. u * V + V)
        if constexpr (V == 1) {
#pragma unroll
            for (int i = 0; i < L; ++i) w[i] = v[i];
        } else {
#pragma unroll
            for (int i = 0; i < L; ++i) stage[i * kWave + lane] = v[i];
            __syncthreads();
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < V; ++j) w[u * V + j] = stage[u * kWave * V + lane * V + j];
            __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float res[M];
#pragma unroll
            for (int r = 0; r < M; ++r) {
                acc_t a = Op::identity();
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const int e = r * C + c;
                    a = Op::combine(a, Op::lift(w[u * V + e / 4][e % 4], (size_t)c));
                }
                res[r] = Op::finish(a);
            }
            float* __restrict__ o = out + ((t * U + u) * kWave + lane) * M;
            if constexpr (M == 4) {
                if (out16) {
                    f32x4 q = {res[0], res[1], res[2], res[3]};
                    store_vec<NT_STORE>(reinterpret_cast<f32x4*>(o), q);
                    continue;
                }
            }
#pragma unroll
            for (int r = 0; r < M; ++r) store_vec<NT_STORE>(o + r, res[r]);
        }
    };

    // The wave's tiles t0, t0 + G, ... two per loop pass, one register
    // buffer each, the next tile's loads in flight while one is folded.
    // Tiles of more than 16 loads per lane (odd widths from 21 floats) take
    // one buffer: two would not fit in registers.
    size_t t0 = blockIdx.x;  // wave-uniform
    if constexpr (L > 16) {
        for (; t0 < ntiles; t0 += G) {
            f32x4 a[L];
            load(a, t0);
            fold_store(a, t0);
        }
    } else if (t0 < ntiles) {
        size_t n = (ntiles - t0 + G - 1) / G;
        f32x4 a[L], b[L];
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
    if (nt)
        hipLaunchKernelGGL((rows_narrow_kernel<Op, C, true>), dim3(grid), dim3(kWave), 0, stream, x, rows, out);
    else
        hipLaunchKernelGGL((rows_narrow_kernel<Op, C, false>), dim3(grid), dim3(kWave), 0, stream, x, rows, out);
    return hipGetLastError();
}

template <class Op>
hipError_t launch_op(const float* x, size_t rows, size_t cols, float* out, int grid, bool nt, hipStream_t stream) {
    switch (cols) {
        case 1: return launch_c<Op, 1>(x, rows, out, grid, nt, stream);
        case 2: return launch_c<Op, 2>(x, rows, out, grid, nt, stream);
        case 3: return launch_c<Op, 3>(x, rows, out, grid, nt, stream);
        case 4: return launch_c<Op, 4>(x, rows, out, grid, nt, stream);
        case 5: return launch_c<Op, 5>(x, rows, out, grid, nt, stream);
        case 6: return launch_c<Op, 6>(x, rows, out, grid, nt, stream);
        case 7: return launch_c<Op, 7>(x, rows, out, grid, nt, stream);
        case 8: return launch_c<Op, 8>(x, rows, out, grid, nt, stream);
        case 9: return launch_c<Op, 9>(x, rows, out, grid, nt, stream);
        case 10: return launch_c<Op, 10>(x, rows, out, grid, nt, stream);
        case 11: return launch_c<Op, 11>(x, rows, out, grid, nt, stream);
        case 12: return launch_c<Op, 12>(x, rows, out, grid, nt, stream);
        case 13: return launch_c<Op, 13>(x, rows, out, grid, nt, stream);
        case 14: return launch_c<Op, 14>(x, rows, out, grid, nt, stream);
        case 15: return launch_c<Op, 15>(x, rows, out, grid, nt, stream);
        case 16: return launch_c<Op, 16>(x, rows, out, grid, nt, stream);
        case 17: return launch_c<Op, 17>(x, rows, out, grid, nt, stream);
        case 18: return launch_c<Op, 18>(x, rows, out, grid, nt, stream);
        case 19: return launch_c<Op, 19>(x, rows, out, grid, nt, stream);
        case 20: return launch_c<Op, 20>(x, rows, out, grid, nt, stream);
        case 21: return launch_c<Op, 21>(x, rows, out, grid, nt, stream);
        case 22: return launch_c<Op, 22>(x, rows, out, grid, nt, stream);
        case 23: return launch_c<Op, 23>(x, rows, out, grid, nt, stream);
        case 24: return launch_c<Op, 24>(x, rows, out, grid, nt, stream);
        case 25: return launch_c<Op, 25>(x, rows, out, grid, nt, stream);
        case 26: return launch_c<Op, 26>(x, rows, out, grid, nt, stream);
        case 27: return launch_c<Op, 27>(x, rows, out, grid, nt, stream);
        case 28: return launch_c<Op, 28>(x, rows, out, grid, nt, stream);
        case 29: return launch_c<Op, 29>(x, rows, out, grid, nt, stream);
        case 30: return launch_c<Op, 30>(x, rows, out, grid, nt, stream);
        case 31: return launch_c<Op, 31>(x, rows, out, grid, nt, stream);
        case 32: return launch_c<Op, 32>(x, rows, out, grid, nt, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t rows_narrow_tile_rows(size_t cols) {
    if (cols < 1 || cols > kNarrowMaxCols) return 0;
    const size_t m = cols % 4 == 0 ? 1 : (cols % 2 == 0 ? 2 : 4);
    const size_t v = cols * m / 4;
    const size_t u = (kNarrowTileLoads + v - 1) / v;
    return u * kWave * m;
}

hipError_t launch_rows_narrow(int op, const float* x, size_t rows, size_t cols, float* out, int grid, bool nt,
                              hipStream_t stream) {
    if (op == 0) return launch_op<SumF32>(x, rows, cols, out, grid, nt, stream);
    if (op == 1) return launch_op<MaxF32>(x, rows, cols, out, grid, nt, stream);
    return hipErrorInvalidValue;
}

}  // namespace libred
