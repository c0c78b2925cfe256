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
//
// With HOLD, a wave writes its results into LDS instead and stores them in
// bursts, every H of its tiles (H * U * 64 * M results, at most
// kNarrowHoldBytes), with 16-byte stores of whole tiles' runs. A result
// store between the loads of a read stream costs more than its bytes: a
// probe that reads 8 KiB per wave step and writes 1/16 of that ran at 5.4
// TB/s of reads and writes storing every step, 6.5 storing every 16 steps
// and 6.9 every 64 (512 waves, 1 GiB).
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace libred {

namespace {

// Rows of c floats: m rows per lane per step, v 16-byte vectors per lane per
// step, u steps per tile, l = u * v loads per lane per tile.
struct NarrowDims {
    int m, v, u, l;
};

constexpr NarrowDims narrow_dims(size_t c) {
    const int m = c % 4 == 0 ? 1 : (c % 2 == 0 ? 2 : 4);
    const int v = (int)c * m / 4;
    const int u = (kNarrowTileLoads + v - 1) / v;
    return {m, v, u, u * v};
}

template <int C>
struct NarrowShape {
    static constexpr NarrowDims d = narrow_dims(C);
    static constexpr int M = d.m, V = d.v, U = d.u, L = d.l;
};

// How a lane folds a row for the max. The compare-and-select
// ((b > a) ? b : a) passes every compare through VCC with wait states before
// the select; at some widths that stalls the fold and the max ran well
// behind the sum (17 floats: 6.1 TB/s of input and output against 6.8).
// There each element is first made canonical (a signalling NaN becomes a
// quiet one), then folded with fmaxf (v_max_f32 / v_max3_f32): a quiet NaN
// operand never wins such a maximum, and the accumulator starts at -inf and
// never holds a NaN, so the result is the same value as the
// compare-and-select fold (of two equal values of opposite sign, either
// zero may be returned). Without the explicit canonicalization the compiler
// fed loaded elements to v_max3_f32 as they were, and a signalling NaN won.
// Two runs, compare-and-select against this fold: 17 floats 6.1 -> 6.9-7.1,
// 19: 6.4 -> 6.9-7.1, 21: 6.5 -> 6.9-7.0, 23: 6.7-6.8 -> 6.9, 31: 6.6 -> 6.7,
// 32: 6.9 -> 7.1-7.2; at the other widths fmaxf (before canonicalization was
// added) ran up to 10% slower (18-28 even: 6.5-7.1 -> 6.3-6.5; 9: 6.9 ->
// 6.6), and folding in four chains instead of one changed nothing.
constexpr bool narrow_max_by_fmax(int c) { return c == 17 || c == 19 || c == 21 || c == 23 || c == 31 || c == 32; }

template <class Op, int C>
__device__ __forceinline__ typename Op::acc_t narrow_combine(typename Op::acc_t a, typename Op::acc_t b) {
    if constexpr (std::is_same_v<Op, MaxF32> && narrow_max_by_fmax(C))
        return __builtin_fmaxf(a, __builtin_canonicalizef(b));
    else
        return Op::combine(a, b);
}

// Results a wave holds in LDS before a burst of stores, in bytes.
constexpr size_t kNarrowHoldBytes = 48 * 1024;

// Tiles whose results a wave holds before a burst (1 without HOLD).
constexpr int narrow_hold_tiles(size_t c, bool hold) {
    const NarrowDims d = narrow_dims(c);
    const size_t h = kNarrowHoldBytes / ((size_t)d.u * kWave * d.m * sizeof(float));
    return !hold ? 1 : h < 1 ? 1 : h > 64 ? 64 : (int)h;
}

// Static LDS of one block: the staging tile (v > 1) and the held results.
constexpr size_t narrow_lds_bytes(size_t c, bool hold) {
    const NarrowDims d = narrow_dims(c);
    const size_t stage = d.v > 1 ? (size_t)kWave * d.l * 16 : 0;
    const size_t held = hold ? (size_t)narrow_hold_tiles(c, hold) * d.u * kWave * d.m * sizeof(float) : 0;
    return stage + held;
}

template <class Op, int C, bool NT, bool HOLD>
__global__ __launch_bounds__(kWave) void rows_narrow_kernel(const float* __restrict__ x, size_t rows,
                                                            float* __restrict__ out) {
    using acc_t = typename Op::acc_t;
    using S = NarrowShape<C>;
    constexpr int M = S::M, V = S::V, U = S::U, L = S::L;
    constexpr size_t kTileRows = (size_t)U * kWave * M;
    constexpr int H = narrow_hold_tiles(C, HOLD);
    constexpr size_t kTileVecs = kTileRows / 4;  // kTileRows is a multiple of 64
    __shared__ f32x4 held_v[HOLD ? H * kTileVecs : 1];
    float* const held = reinterpret_cast<float*>(held_v);
    size_t first = 0;      // the first held tile (wave-uniform)
    unsigned int nheld = 0;  // tiles held: first, first + G, ... (wave-uniform)
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
    // Store the held results: tile first + i * G's run of kTileRows results
    // from held[i * kTileRows ...), as 16-byte vectors when out allows.
    auto flush = [&]() {
        __syncthreads();
        if (out16) {
            const size_t nv = (size_t)nheld * kTileVecs;
            for (size_t q = lane; q < nv; q += kWave) {
                const size_t i = q / kTileVecs, k = q - i * kTileVecs;
                store_vec<NT>(reinterpret_cast<f32x4*>(out + (first + i * G) * kTileRows) + k, held_v[q]);
            }
        } else {
            const size_t nf = (size_t)nheld * kTileRows;
            for (size_t q = lane; q < nf; q += kWave) {
                const size_t i = q / kTileRows, k = q - i * kTileRows;
                store_vec<NT>(out + (first + i * G) * kTileRows + k, held[q]);
            }
        }
        __syncthreads();
        nheld = 0;
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
                    a = narrow_combine<Op, C>(a, Op::lift(w[u * V + e / 4][e % 4], (size_t)c));
                }
                res[r] = Op::finish(a);
            }
            if constexpr (HOLD) {
                float* o = held + nheld * kTileRows + (u * kWave + lane) * M;
                if constexpr (M == 4) {
                    *reinterpret_cast<f32x4*>(o) = f32x4{res[0], res[1], res[2], res[3]};
                } else {
#pragma unroll
                    for (int r = 0; r < M; ++r) o[r] = res[r];
                }
                continue;
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
        if constexpr (HOLD) {
            if (nheld == 0) first = t;
            if (++nheld == H) flush();
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
    if constexpr (HOLD) {
        if (nheld > 0) flush();
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
hipError_t launch_c(const float* x, size_t rows, float* out, int grid, bool nt, bool hold, hipStream_t stream) {
    if (hold && nt)
        hipLaunchKernelGGL((rows_narrow_kernel<Op, C, true, true>), dim3(grid), dim3(kWave), 0, stream, x, rows, out);
    else if (hold)
        hipLaunchKernelGGL((rows_narrow_kernel<Op, C, false, true>), dim3(grid), dim3(kWave), 0, stream, x, rows, out);
    else if (nt)
        hipLaunchKernelGGL((rows_narrow_kernel<Op, C, true, false>), dim3(grid), dim3(kWave), 0, stream, x, rows, out);
    else
        hipLaunchKernelGGL((rows_narrow_kernel<Op, C, false, false>), dim3(grid), dim3(kWave), 0, stream, x, rows,
                           out);
    return hipGetLastError();
}

template <class Op>
hipError_t launch_op(const float* x, size_t rows, size_t cols, float* out, int grid, bool nt, bool hold,
                     hipStream_t stream) {
    switch (cols) {
        case 1: return launch_c<Op, 1>(x, rows, out, grid, nt, hold, stream);
        case 2: return launch_c<Op, 2>(x, rows, out, grid, nt, hold, stream);
        case 3: return launch_c<Op, 3>(x, rows, out, grid, nt, hold, stream);
        case 4: return launch_c<Op, 4>(x, rows, out, grid, nt, hold, stream);
        case 5: return launch_c<Op, 5>(x, rows, out, grid, nt, hold, stream);
        case 6: return launch_c<Op, 6>(x, rows, out, grid, nt, hold, stream);
        case 7: return launch_c<Op, 7>(x, rows, out, grid, nt, hold, stream);
        case 8: return launch_c<Op, 8>(x, rows, out, grid, nt, hold, stream);
        case 9: return launch_c<Op, 9>(x, rows, out, grid, nt, hold, stream);
        case 10: return launch_c<Op, 10>(x, rows, out, grid, nt, hold, stream);
        case 11: return launch_c<Op, 11>(x, rows, out, grid, nt, hold, stream);
        case 12: return launch_c<Op, 12>(x, rows, out, grid, nt, hold, stream);
        case 13: return launch_c<Op, 13>(x, rows, out, grid, nt, hold, stream);
        case 14: return launch_c<Op, 14>(x, rows, out, grid, nt, hold, stream);
        case 15: return launch_c<Op, 15>(x, rows, out, grid, nt, hold, stream);
        case 16: return launch_c<Op, 16>(x, rows, out, grid, nt, hold, stream);
        case 17: return launch_c<Op, 17>(x, rows, out, grid, nt, hold, stream);
        case 18: return launch_c<Op, 18>(x, rows, out, grid, nt, hold, stream);
        case 19: return launch_c<Op, 19>(x, rows, out, grid, nt, hold, stream);
        case 20: return launch_c<Op, 20>(x, rows, out, grid, nt, hold, stream);
        case 21: return launch_c<Op, 21>(x, rows, out, grid, nt, hold, stream);
        case 22: return launch_c<Op, 22>(x, rows, out, grid, nt, hold, stream);
        case 23: return launch_c<Op, 23>(x, rows, out, grid, nt, hold, stream);
        case 24: return launch_c<Op, 24>(x, rows, out, grid, nt, hold, stream);
        case 25: return launch_c<Op, 25>(x, rows, out, grid, nt, hold, stream);
        case 26: return launch_c<Op, 26>(x, rows, out, grid, nt, hold, stream);
        case 27: return launch_c<Op, 27>(x, rows, out, grid, nt, hold, stream);
        case 28: return launch_c<Op, 28>(x, rows, out, grid, nt, hold, stream);
        case 29: return launch_c<Op, 29>(x, rows, out, grid, nt, hold, stream);
        case 30: return launch_c<Op, 30>(x, rows, out, grid, nt, hold, stream);
        case 31: return launch_c<Op, 31>(x, rows, out, grid, nt, hold, stream);
        case 32: return launch_c<Op, 32>(x, rows, out, grid, nt, hold, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t rows_narrow_tile_rows(size_t cols) {
    if (cols < 1 || cols > kNarrowMaxCols) return 0;
    const NarrowDims d = narrow_dims(cols);
    return (size_t)d.u * kWave * d.m;
}

size_t rows_narrow_lds_bytes(size_t cols, bool hold) {
    if (cols < 1 || cols > kNarrowMaxCols) return 0;
    return narrow_lds_bytes(cols, hold);
}

hipError_t launch_rows_narrow(int op, const float* x, size_t rows, size_t cols, float* out, int grid, bool nt,
                              bool hold, hipStream_t stream) {
    if (op == 0) return launch_op<SumF32>(x, rows, cols, out, grid, nt, hold, stream);
    if (op == 1) return launch_op<MaxF32>(x, rows, cols, out, grid, nt, hold, stream);
    return hipErrorInvalidValue;
}

}  // namespace libred
