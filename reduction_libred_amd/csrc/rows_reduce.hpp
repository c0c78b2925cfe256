// rows_reduce.hpp -- per-row (segmented) sum and max of a row-major matrix
// whose rows start `ld` elements apart (ld >= cols; ld == cols is the dense
// case), as templates over the operator; rows_sum.hip and rows_max.hip
// instantiate them for the sum and the max, so the two compile in parallel.
//
// The lesson's reduction gives one output per block segment
// ("03_shared_memory_sync_reduction.py", demo 3). Here the segment is a row,
// and the kernels, in the order of this file, cover the shapes:
//   rows_reduce_kernel, one wave per row (many long rows): a 64-lane wave
//       owns one row at a time, with no LDS, no barrier and no cross-block
//       combine; a 4096-float row is 16 KiB, i.e. 16 aligned 16-byte loads
//       per lane;
//   rows_cover_kernel, the same for rows that do not start 16-byte aligned
//       (x unaligned, or ld not a multiple of 4): a row is read as the
//       aligned 16-byte vectors that cover it, elements outside the row
//       masked when folded; rows_stream_kernel reads rows the same way with
//       the next tile always in flight across rows (a policy option);
//   rows_packed_kernel, short strided or unaligned rows: several rows per
//       load, a segment of lanes per row;
//   rows_staged_kernel, short rows of a contiguous matrix: tiles of whole
//       rows loaded as 16-byte vectors into LDS and reduced from there;
//   rows_split_kernel + rows_combine_kernel, few long rows: each row is cut
//       across `gx` single-wave blocks that stream tiles of 64*UNROLL
//       vectors, each storing one partial; a second launch combines each
//       row's partials in index order with one wave per row.
// rows_reduce_kernel and the split kernel peel an unaligned row's head and
// tail element by element (none when aligned). Sums accumulate in float64
// and round once per row.
#pragma once

#include "device_common.hpp"
#include "launch.hpp"

namespace libred {

// The block index a grid-stride row kernel works as. With chunk C > 0, the
// indices are dealt to the XCDs (the launch deals block b to XCD b mod
// kXcds) in runs of C consecutive ones, the runs in turn, gridDim.x a
// multiple of kXcds * C: neighbouring rows (or tiles), which share the
// 128-byte line where one ends and the next begins, are then read into one
// XCD's L2 but at the end of a run, while the blocks running at any time
// still hold one band of consecutive indices.
__device__ __forceinline__ size_t work_block(int chunk) {
    if (chunk <= 0) return blockIdx.x;
    const size_t c = (size_t)chunk, i = blockIdx.x / kXcds;
    return i / c * (kXcds * c) + (blockIdx.x % kXcds) * c + i % c;
}

template <bool NT, class V, int UNROLL>
__device__ __forceinline__ void load_tile_rows(V (&v)[UNROLL], const V* __restrict__ p) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = load_vec<NT>(p + u * kWave);
}

// Fold body vectors i = begin + lane, begin + lane + step, ... (< nvec) of a
// row into acc, UNROLL loads at a time: a lane issues all of a batch's loads
// before it folds any, so the vectors after a row's last whole tile cost one
// memory latency, not one per vector. (The loads stay under a lane mask here:
// loading a stand-in vector instead, as the short-row kernels do, made the
// compiler wait for every outstanding memory operation at the top of each
// row in the one-wave-per-row kernel, 11% slower on 65536 x 4096.)
template <class Op, int UNROLL, bool NT>
__device__ __forceinline__ void fold_remainder(typename Op::acc_t (&acc)[4], const typename Op::vec_t* __restrict__ rv,
                                               size_t head, size_t begin, size_t nvec, size_t step) {
    using vec_t = typename Op::vec_t;
    const size_t lane = threadIdx.x % kWave;
    for (size_t i0 = begin + lane; i0 < nvec; i0 += step * UNROLL) {
        vec_t v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const size_t i = i0 + (size_t)u * step;
            if (i < nvec) v[u] = load_vec<NT>(rv + i);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const size_t i = i0 + (size_t)u * step;
            if (i < nvec) fold_vec<Op>(acc, v[u], head + i * Op::kPerVec);
        }
    }
}

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
    fold_remainder<Op, UNROLL, NT>(acc, rv, head, ntiles * TILE + first_tile * kWave, nvec, tile_step * kWave);
    if (edges) {
        if ((size_t)lane < head) acc[0] = Op::combine(acc[0], Op::lift(row[lane], lane));
        if ((size_t)lane < cols - tail0)
            acc[1] = Op::combine(acc[1], Op::lift(row[tail0 + lane], tail0 + lane));
    }
}

template <class Op, int BLOCK, int UNROLL, bool NT>
__global__ __launch_bounds__(BLOCK) void rows_reduce_kernel(const typename Op::elem_t* __restrict__ x,
                                                            size_t rows, size_t cols, size_t ld,
                                                            typename Op::out_t* __restrict__ out, int xmap) {
    using acc_t = typename Op::acc_t;
    constexpr int W = BLOCK / kWave;
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

    // Wave-uniform loop over rows: all 64 lanes stay active at the wave reduce.
    for (size_t r = work_block(xmap) * W + wave; r < rows; r += (size_t)gridDim.x * W) {
        acc_t acc[4] = {Op::identity(), Op::identity(), Op::identity(), Op::identity()};
        fold_row_span<Op, UNROLL, NT>(x + r * ld, cols, 0, 1, true, acc);
        acc_t v = Op::combine(Op::combine(acc[0], acc[1]), Op::combine(acc[2], acc[3]));
        v = wave_reduce<Op>(v);
        if (lane == 0) out[r] = Op::finish(v);
    }
}

// One wave per row, streaming. A row is read as the aligned 16-byte vectors
// that cover it: vector 0 holds the row's first element at position s (0-3),
// and the cover has nv = ceil((s + cols) / 4) vectors, cut into tiles of
// 64 * UNROLL. A wave's work is the sequence of (row, tile) items of rows
// r, r + G, r + 2G, ... (G waves in all); the loads of the next item (which may
// be the first tile of the wave's next row) are issued before the current
// item is folded, and every load is unconditional: an index past the row's
// last vector is clamped to it, and elements outside the row are replaced by
// the identity when folded, never masked at the load. Only the first and last
// tiles of a row need that masking. A cover vector that would reach outside
// the array (before x when x is not 16-byte aligned, or past the end of the
// last row) is not loaded as a vector; its elements of the row are read one
// by one when the row is finished. Rows hold at least 16 elements.
template <class Op>
struct CoverGeom {
    const typename Op::vec_t* vb;  // the aligned vector holding the row's first element
    size_t nv;                     // vectors of the cover
    size_t ntiles;                 // tiles of 64 * UNROLL vectors
    size_t vlo, vhi;               // vectors [vlo, vhi) are loaded as vectors
    unsigned int s;                // position of the row's first element in vector 0
};

template <class Op, int UNROLL>
__device__ __forceinline__ CoverGeom<Op> cover_geom(const typename Op::elem_t* __restrict__ x, size_t r,
                                                    size_t cols, size_t ld, uintptr_t end) {
    using elem_t = typename Op::elem_t;
    constexpr size_t E = Op::kPerVec;
    const elem_t* row = x + r * ld;
    CoverGeom<Op> g;
    g.s = (unsigned int)(((uintptr_t)row & 15u) / sizeof(elem_t));
    // Pointer arithmetic from x (not an integer cast) keeps the loads global.
    g.vb = reinterpret_cast<const typename Op::vec_t*>(row - g.s);
    g.nv = (g.s + cols + E - 1) / E;
    g.ntiles = (g.nv + (size_t)kWave * UNROLL - 1) / ((size_t)kWave * UNROLL);
    g.vlo = (uintptr_t)g.vb < (uintptr_t)x ? 1 : 0;
    g.vhi = (uintptr_t)(g.vb + g.nv) > end ? g.nv - 1 : g.nv;
    return g;
}

// The element that leaves a row reduction unchanged: 0 for the sum, -inf for
// the max (which skips NaN and keeps its incumbent on ties).
template <class Op>
struct RowNeutral;
template <>
struct RowNeutral<SumF32> {
    static __device__ __forceinline__ float value() { return 0.0f; }
};
template <>
struct RowNeutral<MaxF32> {
    static __device__ __forceinline__ float value() { return -__builtin_inff(); }
};

// Fold row r through its cover (see above), one tile at a time: the tile's
// loads are unconditional (indices clamped into [vlo, vhi)), load slots of
// the last tile that hold no vector of the row are skipped (a wave-uniform
// test), and the first and last tiles are folded with the elements outside
// the row replaced by the identity. Then the edge elements of a cover vector
// that was not loaded as a vector.
template <class Op, int UNROLL, bool NT>
__device__ __forceinline__ void fold_row_cover(const typename Op::elem_t* __restrict__ x, size_t r, size_t cols,
                                               size_t ld, uintptr_t end, typename Op::acc_t (&acc)[4]) {
    using vec_t = typename Op::vec_t;
    constexpr size_t E = Op::kPerVec;
    constexpr size_t TILE = (size_t)kWave * UNROLL;
    const unsigned int lane = threadIdx.x % kWave;
    const CoverGeom<Op> g = cover_geom<Op, UNROLL>(x, r, cols, ld, end);
    // Only cover vector 0 (elements before position s) and the last cover
    // vector (elements from position s + cols on) can hold elements outside
    // the row; a vector outside [vlo, vhi) holds none of the row. Those
    // elements become the operator's neutral element.
    const unsigned int k_end = (unsigned int)(g.s + cols - (g.nv - 1) * E);  // 1..E
    for (size_t t = 0; t < g.ntiles; ++t) {
        vec_t v[UNROLL];
        if (t != 0 && t + 1 != g.ntiles) {  // wave-uniform: a tile inside the row, read as is
            const vec_t* __restrict__ p = g.vb + t * TILE + lane;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) v[u] = load_vec<NT>(p + u * kWave);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                fold_vec<Op>(acc, v[u], (t * TILE + (size_t)u * kWave + lane) * E - g.s);
        } else {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                size_t i = t * TILE + (size_t)u * kWave + lane;
                i = i < g.vlo ? g.vlo : i;
                i = i >= g.vhi ? g.vhi - 1 : i;
                v[u] = load_vec<NT>(g.vb + i);
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const size_t i = t * TILE + (size_t)u * kWave + lane;
                unsigned int lo = i == 0 ? g.s : 0u;
                unsigned int hi = i + 1 == g.nv ? k_end : (unsigned int)E;
                if (i < g.vlo || i >= g.vhi) hi = 0;
                vec_t w = v[u];
#pragma unroll
                for (int k = 0; k < (int)E; ++k)
                    w[k] = ((unsigned int)k >= lo && (unsigned int)k < hi) ? w[k] : RowNeutral<Op>::value();
                fold_vec<Op>(acc, w, i * E - g.s);
            }
        }
    }
    const typename Op::elem_t* row = x + r * ld;
    if (g.vlo != 0) {
        const size_t nfirst = E - g.s;
        if (lane < nfirst) acc[0] = Op::combine(acc[0], Op::lift(row[lane], lane));
    }
    if (g.vhi != g.nv) {
        const size_t e0 = (g.nv - 1) * E - g.s;
        if (lane < cols - e0) acc[1] = Op::combine(acc[1], Op::lift(row[e0 + lane], e0 + lane));
    }
}

template <class Op, int BLOCK, int UNROLL, bool NT>
__global__ __launch_bounds__(BLOCK) void rows_cover_kernel(const typename Op::elem_t* __restrict__ x,
                                                           size_t rows, size_t cols, size_t ld,
                                                           typename Op::out_t* __restrict__ out, int xmap) {
    using acc_t = typename Op::acc_t;
    constexpr int W = BLOCK / kWave;
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uintptr_t end = (uintptr_t)(x + (rows - 1) * ld + cols);
    for (size_t r = work_block(xmap) * W + wave; r < rows; r += (size_t)gridDim.x * W) {
        acc_t acc[4] = {Op::identity(), Op::identity(), Op::identity(), Op::identity()};
        fold_row_cover<Op, UNROLL, NT>(x, r, cols, ld, end, acc);
        acc_t v = Op::combine(Op::combine(acc[0], acc[1]), Op::combine(acc[2], acc[3]));
        v = wave_reduce<Op>(v);
        if (lane == 0) out[r] = Op::finish(v);
    }
}

template <class Op, int UNROLL, bool NT>
__global__ __launch_bounds__(kWave) void rows_stream_kernel(const typename Op::elem_t* __restrict__ x,
                                                            size_t rows, size_t cols, size_t ld,
                                                            typename Op::out_t* __restrict__ out, int xmap) {
    using acc_t = typename Op::acc_t;
    using vec_t = typename Op::vec_t;
    using elem_t = typename Op::elem_t;
    constexpr size_t E = Op::kPerVec;
    constexpr size_t TILE = (size_t)kWave * UNROLL;
    const unsigned int lane = threadIdx.x;
    const size_t G = gridDim.x;
    const uintptr_t end = (uintptr_t)(x + (rows - 1) * ld + cols);
    size_t r = work_block(xmap);  // wave-uniform
    if (r >= rows) return;
    CoverGeom<Op> g = cover_geom<Op, UNROLL>(x, r, cols, ld, end);
    size_t t = 0;
    acc_t acc[4] = {Op::identity(), Op::identity(), Op::identity(), Op::identity()};

    auto load_item = [&](vec_t (&v)[UNROLL], const CoverGeom<Op>& h, size_t tt) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            size_t i = tt * TILE + (size_t)u * kWave + lane;
            i = i < h.vlo ? h.vlo : i;
            i = i >= h.vhi ? h.vhi - 1 : i;
            v[u] = load_vec<NT>(h.vb + i);
        }
    };
    auto fold_item = [&](const vec_t (&v)[UNROLL]) {
        if (t != 0 && t + 1 != g.ntiles) {  // wave-uniform: a tile inside the row
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                fold_vec<Op>(acc, v[u], (t * TILE + (size_t)u * kWave + lane) * E - g.s);
        } else {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const size_t i = t * TILE + (size_t)u * kWave + lane;
                const bool live = i >= g.vlo && i < g.vhi;
#pragma unroll
                for (int k = 0; k < (int)E; ++k) {
                    const size_t e = i * E + k;  // position in the cover; the row is [s, s + cols)
                    const bool in = live && e >= g.s && e < g.s + cols;
                    acc[k & 3] = Op::combine(acc[k & 3], in ? Op::lift(v[u][k], e - g.s) : Op::identity());
                }
            }
        }
    };
    auto finish_row = [&]() {
        const elem_t* row = x + r * ld;
        if (g.vlo != 0) {  // the row's elements in cover vector 0, read one by one
            const size_t nfirst = E - g.s;
            if (lane < nfirst) acc[0] = Op::combine(acc[0], Op::lift(row[lane], lane));
        }
        if (g.vhi != g.nv) {  // and those in the last cover vector
            const size_t e0 = (g.nv - 1) * E - g.s;
            if (lane < cols - e0) acc[1] = Op::combine(acc[1], Op::lift(row[e0 + lane], e0 + lane));
        }
        acc_t v = Op::combine(Op::combine(acc[0], acc[1]), Op::combine(acc[2], acc[3]));
        v = wave_reduce<Op>(v);
        if (lane == 0) out[r] = Op::finish(v);
        acc[0] = acc[1] = acc[2] = acc[3] = Op::identity();
    };
    // One item: load the next one, fold this one, finish the row after its
    // last tile. Returns false when the wave has no item left (its final
    // loads then re-read the current tile, which stays in bounds).
    auto step = [&](const vec_t (&cur)[UNROLL], vec_t (&nxt)[UNROLL]) -> bool {
        size_t rn = r, tn = t + 1;
        CoverGeom<Op> gn = g;
        const bool row_done = tn >= g.ntiles;
        if (row_done) {
            rn = r + G;
            tn = 0;
            if (rn < rows) gn = cover_geom<Op, UNROLL>(x, rn, cols, ld, end);
        }
        const bool more = rn < rows;
        load_item(nxt, more ? gn : g, more ? tn : t);
        fold_item(cur);
        if (row_done) finish_row();
        r = rn;
        t = tn;
        g = gn;
        return more;
    };
    vec_t a[UNROLL], b[UNROLL];
    load_item(a, g, 0);
    while (step(a, b) && step(b, a)) {
    }
}

// Packed short rows (at most 512 floats): a row gets a segment of
// L = 2^LOG2L lanes, lane j taking the row's load units j, j + L, ..., up to
// V of them, so one load instruction covers P = 64 / L rows. A unit is a
// 16-byte vector when every row starts on a 16-byte boundary and holds whole
// vectors (x 16-byte aligned, cols and ld multiples of 4; L <= 16), else one
// element (L <= 64), which serves rows of any width and alignment. Each lane
// folds its units, the L lanes of a segment are combined with the first
// LOG2L steps of the DPP wave reduce, and the segment's leader stores the
// row. A wave takes groups of P rows w, w + G, w + 2G, ... (G = grid size),
// U groups per trip (16 vectors or 32 elements in flight per lane) with all
// their loads issued first, and the next trip's loads issued before the
// current trip is reduced and stored.
//
// After the first four steps (quad_perm x 2, row_half_mirror, row_mirror)
// every lane of a 16-lane row holds the row's total; row_bcast:15 into rows 1
// and 3 then leaves 32-lane totals in lanes 16-31 and 48-63, and
// row_bcast:31 into rows 2 and 3 leaves the 64-lane total in lanes 48-63. So
// the leader is lane 0 of a segment of up to 16 lanes and the last lane of a
// 32- or 64-lane segment.
template <class Op, int LOG2L>
__device__ __forceinline__ typename Op::acc_t segment_reduce(typename Op::acc_t v) {
    using T = typename Op::acc_t;
    const T id = Op::identity();
    if constexpr (LOG2L >= 1) v = Op::combine(v, dpp_move<0xB1, 0xF>(id, v));   // quad_perm:[1,0,3,2]
    if constexpr (LOG2L >= 2) v = Op::combine(v, dpp_move<0x4E, 0xF>(id, v));   // quad_perm:[2,3,0,1]
    if constexpr (LOG2L >= 3) v = Op::combine(v, dpp_move<0x141, 0xF>(id, v));  // row_half_mirror
    if constexpr (LOG2L >= 4) v = Op::combine(v, dpp_move<0x140, 0xF>(id, v));  // row_mirror
    if constexpr (LOG2L >= 5) v = Op::combine(v, dpp_move<0x142, 0xA>(id, v));  // row_bcast:15 -> rows 1, 3
    if constexpr (LOG2L >= 6) v = Op::combine(v, dpp_move<0x143, 0xC>(id, v));  // row_bcast:31 -> rows 2, 3
    return v;
}

template <class Op, int LOG2L, int V, bool SCALAR, bool NT>
__global__ __launch_bounds__(kWave) void rows_packed_kernel(const typename Op::elem_t* __restrict__ x,
                                                            size_t rows, size_t cols, size_t ld,
                                                            typename Op::out_t* __restrict__ out, int xmap) {
    using acc_t = typename Op::acc_t;
    using unit_t = std::conditional_t<SCALAR, typename Op::elem_t, typename Op::vec_t>;
    constexpr size_t E = SCALAR ? 1 : Op::kPerVec;  // elements per unit
    constexpr int L = 1 << LOG2L;
    constexpr int P = kWave / L;
    constexpr int U = (SCALAR ? 32 : 16) / V;
    const int lane = threadIdx.x;
    const size_t q = (size_t)(lane >> LOG2L);
    const size_t j = (size_t)(lane & (L - 1));
    const bool leader = LOG2L <= 4 ? j == 0 : j == (size_t)L - 1;
    const size_t nunits = cols / E;
    const size_t ldu = ld / E;
    const unit_t* __restrict__ xu = reinterpret_cast<const unit_t*>(x);
    const size_t G = gridDim.x;
    const size_t ngroups = (rows + P - 1) / P;
    // A lane with nothing to read (past the last row, or past its row's last
    // unit) reads unit 0 of the matrix instead and folds nothing: no load
    // sits under a lane mask (that would make the compiler wait for every
    // earlier load first).
    auto load_trip = [&](unit_t (&v)[U][V], size_t g0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t r = (g0 + (size_t)u * G) * P + q;
            const bool live = r < rows;
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const size_t i = j + (size_t)k * L;
                v[u][k] = load_vec<NT>(xu + (live && i < nunits ? r * ldu + i : 0));
            }
        }
    };
    auto reduce_trip = [&](const unit_t (&v)[U][V], size_t g0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t g = g0 + (size_t)u * G;
            if (g >= ngroups) break;  // wave-uniform
            const size_t r = g * P + q;
            const bool live = r < rows;
            acc_t acc[4] = {Op::identity(), Op::identity(), Op::identity(), Op::identity()};
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const size_t i = j + (size_t)k * L;
                if (live && i < nunits) {
                    if constexpr (SCALAR)
                        acc[k & 3] = Op::combine(acc[k & 3], Op::lift(v[u][k], i));
                    else
                        fold_vec<Op>(acc, v[u][k], i * E);
                }
            }
            acc_t a = Op::combine(Op::combine(acc[0], acc[1]), Op::combine(acc[2], acc[3]));
            a = segment_reduce<Op, LOG2L>(a);
            if (live && leader) out[r] = Op::finish(a);
        }
    };
    // Trips alternate between two register buffers: the next trip's loads
    // are issued before the current trip is reduced and stored, so the loads
    // stay in flight across trips (and, memory operations completing in
    // order, waiting for them never waits for the stores that follow). The
    // wave's n trips run two per loop pass with the odd or last two after
    // the loop, which then has a single exit: with an exit after each half,
    // the compiler joins the exits in a block that also leads back to the
    // loop head, and on that path the other buffer's loads are still in
    // flight, so the head waited for them before issuing the next loads.
    size_t g0 = work_block(xmap);  // wave-uniform
    if (g0 >= ngroups) return;
    const size_t step = G * U;
    size_t n = (ngroups - g0 + step - 1) / step;
    unit_t a[U][V], b[U][V];
    load_trip(a, g0);
    for (; n > 2; n -= 2, g0 += 2 * step) {
        load_trip(b, g0 + step);
        reduce_trip(a, g0);
        load_trip(a, g0 + 2 * step);
        reduce_trip(b, g0 + step);
    }
    if (n == 2) {
        load_trip(b, g0 + step);
        reduce_trip(a, g0);
        reduce_trip(b, g0 + step);
    } else {
        reduce_trip(a, g0);
    }
}

// Short rows, staged through LDS: rows starting ld >= cols elements apart,
// x at any element. A tile is R consecutive rows; its span, from its first
// row's first element to its last row's last, is loaded as the aligned
// 16-byte vectors that cover it (coalesced whatever the row length or
// stride), at most U per lane, and stored to LDS, where the tile's first
// element lands at `off` (0-3, the span's offset within its first vector)
// and row r at off + r * ld. The vectors a tile loads beyond its own span
// hold elements of its neighbours or of the gaps between rows, all inside
// the matrix, and are never read. Two vectors may reach outside the matrix:
// the first, when x is not 16-byte aligned (it starts sh elements before
// x), and the last, when the matrix ends inside it; neither is loaded as a
// vector, and their elements of the matrix are read one by one. (For a
// contiguous, 16-byte aligned matrix, R is a multiple of 4 / gcd(cols, 4),
// so every tile starts 16-byte aligned and off is 0.) The wave then reduces
// the tile's rows 64 / S at a time with S = 2^LOG2S lanes per row: lane s of
// a row adds elements s, s + S, ... in order (with SPREAD, from a starting
// element that differs between the rows of a pass), then the segment reduce; with
// VREAD (rows of whole vectors, off always 0 and ld a multiple of 4) lane s
// reads vectors s, s + S, ... of its row. Tiles are dealt round-robin to the
// waves, and the next tile's loads are issued before the current tile is
// reduced. A load slot with no vector of the tile reads the first whole
// vector of the matrix instead (no load sits under a lane mask).
//
// With HOLD, a wave keeps its row results in LDS (dynamic shared memory, at
// least R times the wave's tile count) and stores them all after its last
// tile. (A template parameter: with a run-time choice the compiler merges the
// LDS store and the global store into one flat store, which counts against
// both the LDS and the memory counters, so every LDS wait became a wait for
// all loads in flight.) Small stores spread through the read stream cost
// far more HBM time than their bytes: on 1 GiB of 64-float rows, 16 MiB of
// results stored as each tile was reduced took about 20 us more than no
// stores at all, against about 2 us when they all went out at the end.
//
// The host ensures that a tile's span plus 3 fits 256 * U elements, that the
// matrix spans at least 8 elements, and that R * ld >= 4.
// FMAX (maxima only): each lane folds its elements with a hardware max of the
// canonicalized element (a signalling NaN made quiet, so that a NaN never
// wins, as with the compare-and-select), not a compare and a select through
// VCC.
template <class Op, int LOG2S, int U, bool NT, bool VREAD, bool HOLD, bool SPREAD, bool FMAX = false>
__global__ __launch_bounds__(kWave) void rows_staged_kernel(const typename Op::elem_t* __restrict__ x,
                                                            size_t rows, size_t cols, size_t ld,
                                                            unsigned int sh, unsigned int R,
                                                            typename Op::out_t* __restrict__ out, int xmap) {
    using acc_t = typename Op::acc_t;
    using elem_t = typename Op::elem_t;
    using vec_t = typename Op::vec_t;
    constexpr int S = 1 << LOG2S;
    constexpr int P = kWave / S;
    constexpr size_t E = Op::kPerVec;
    // Element reads keep eight LDS reads in flight where the combine is a
    // cheap 32-bit one and a row has 4 or more lanes: such a loop has too
    // little arithmetic to cover four reads' latency (1 GiB, maxima of 100,
    // 256 and 384 floats: 6.1-6.5 -> 6.6-6.9 TB/s). Float64 sums, and maxima
    // with one or two lanes per row, measured as fast or faster with four.
    constexpr bool kEightReads = sizeof(acc_t) == 4 && LOG2S >= 2;
    static_assert(!FMAX || std::is_same_v<Op, MaxF32>, "the fmax fold is the float32 max's");
    auto fold = [](acc_t a, acc_t b) -> acc_t {
        if constexpr (FMAX)
            return __builtin_fmaxf(a, __builtin_canonicalizef(b));
        else
            return Op::combine(a, b);
    };
    __shared__ vec_t stage[kWave * U];
    extern __shared__ __align__(16) unsigned char rows_staged_held[];
    typename Op::out_t* held = reinterpret_cast<typename Op::out_t*>(rows_staged_held);
    elem_t* lds = reinterpret_cast<elem_t*>(stage);
    const unsigned int lane = threadIdx.x;
    const unsigned int s = lane & (S - 1);
    const bool leader = LOG2S <= 4 ? s == 0 : s == (unsigned int)S - 1;
    const size_t ntiles = (rows + R - 1) / R;
    const size_t G = gridDim.x;
    // Vectors of the aligned cover, counted from x - sh.
    const vec_t* __restrict__ xv = reinterpret_cast<const vec_t*>(x - sh);
    const size_t end = (size_t)sh + (rows - 1) * ld + cols;  // one past the matrix, from x - sh
    const size_t vlast = (end - 1) / E;                       // the cover's last vector
    const bool cut_last = end % E != 0;                       // ... reaches past the matrix
    const size_t safe = sh > 0 ? 1 : 0;                       // a vector wholly inside
    // With SPREAD (element reads), lane s of a pass's row q reads its m
    // elements s, s + S, ... starting from number q mod m and wrapping round:
    // rows at a stride of a multiple of 16 or 32 words would otherwise put
    // many rows of a pass on the same LDS banks at every step.
    const unsigned int Cw = (unsigned int)cols;
    const unsigned int m_lane = s < Cw ? ((Cw - 1 - s) >> LOG2S) + 1 : 0u;
    const unsigned int wrap_back = m_lane << LOG2S;
    const unsigned int j_first = m_lane > 0 ? s + (((lane >> LOG2S) % m_lane) << LOG2S) : s;
    auto rows_in = [&](size_t t) -> unsigned int {  // rows of tile t (0 past the last tile)
        return t + 1 < ntiles ? R : t + 1 == ntiles ? (unsigned int)(rows - t * R) : 0u;
    };
    auto first_vec = [&](size_t t) -> size_t { return ((size_t)sh + t * R * ld) / E; };
    auto end_vec = [&](size_t t) -> size_t {  // one past the tile's last cover vector
        return ((size_t)sh + (t * R + rows_in(t) - 1) * ld + cols + E - 1) / E;
    };
    auto load_tile = [&](vec_t (&v)[U], size_t t) {
        // Slots [lo, hi) load the tile's cover vectors vb + slot (wave-uniform
        // bounds); the matrix's first vector (when x is not 16-byte aligned)
        // and its last (when the matrix ends inside it) are left out.
        const size_t vb = first_vec(t), ve = end_vec(t);
        const unsigned int lo = vb == 0 && sh > 0 ? 1u : 0u;
        const unsigned int hi = (unsigned int)(ve - vb) - (cut_last && ve - 1 == vlast ? 1u : 0u);
        const vec_t* __restrict__ tv = xv + vb;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const unsigned int slot = lane + (unsigned int)(u * kWave);
            v[u] = load_vec<NT>(slot >= lo && slot < hi ? tv + slot : xv + safe);
        }
    };
    auto reduce_tile = [&](const vec_t (&v)[U], size_t t, size_t k) {  // k: the wave's tile number
        const size_t vb = first_vec(t);
        const unsigned int off = (unsigned int)((size_t)sh + t * R * ld - vb * E);
#pragma unroll
        for (int u = 0; u < U; ++u) stage[lane + u * kWave] = v[u];
        // The vectors left out: their elements of the matrix, one by one
        // (LDS position = cover position - vb * E). The last one may belong
        // to the covers of the last two tiles.
        if (vb == 0 && sh > 0 && lane < E - sh) lds[sh + lane] = x[lane];
        if (cut_last && end_vec(t) - 1 == vlast) {
            const size_t c0 = vlast * E;  // cover position of the last vector
            if (lane < end - c0) lds[c0 - vb * E + lane] = x[c0 + lane - sh];
        }
        __syncthreads();
        const unsigned int rows_t = rows_in(t);
        const unsigned int C = (unsigned int)cols;
        const unsigned int L = (unsigned int)ld;
        for (unsigned int r0 = 0; r0 < rows_t; r0 += P) {
            const unsigned int r = r0 + (lane >> LOG2S);
            acc_t a = Op::identity();
            if constexpr (VREAD) {
                // Rows of whole 16-byte vectors, read a vector at a time:
                // lane s takes vectors s, s + S, ... of its row. With S no
                // smaller than the row's vectors, the lanes of a pass read one
                // contiguous run of LDS (no bank conflicts); element reads at
                // a stride of cols words put rows on the same banks whenever
                // cols is a multiple of 16.
                if (r < rows_t) {
                    const unsigned int V = C / (unsigned int)E;
                    const vec_t* rowv = stage + r * (L / (unsigned int)E);
                    unsigned int j = s;
                    // A cheap 32-bit combine leaves one read's latency
                    // exposed: two reads in flight (maxima of 64 floats
                    // 6.3 -> 6.8 TB/s, 44 and 48 floats 2% faster, 52-60 2%
                    // slower with a single read left over at the end; a
                    // run-time test for that case cost them 6%).
                    if constexpr (sizeof(acc_t) == 4) {
                        for (; j + S < V; j += 2 * S) {
                            const vec_t v0 = rowv[j], v1 = rowv[j + S];
#pragma unroll
                            for (int k = 0; k < (int)E; ++k) a = fold(a, Op::lift(v0[k], j * E + k));
#pragma unroll
                            for (int k = 0; k < (int)E; ++k) a = fold(a, Op::lift(v1[k], (j + S) * E + k));
                        }
                    }
                    for (; j < V; j += S) {
                        const vec_t v = rowv[j];
#pragma unroll
                        for (int k = 0; k < (int)E; ++k) a = fold(a, Op::lift(v[k], j * E + k));
                    }
                }
            } else if constexpr (SPREAD) {
                if (r < rows_t) {
                    const elem_t* row = lds + off + r * L;
                    auto next = [&](unsigned int j) { return j + S >= C ? j + S - wrap_back : j + S; };
                    unsigned int j = j_first, i = 0;
                    for (; i + 4 <= m_lane; i += 4) {
                        const unsigned int j1 = next(j), j2 = next(j1), j3 = next(j2);
                        const elem_t e0 = row[j], e1 = row[j1], e2 = row[j2], e3 = row[j3];
                        a = fold(a, Op::lift(e0, j));
                        a = fold(a, Op::lift(e1, j1));
                        a = fold(a, Op::lift(e2, j2));
                        a = fold(a, Op::lift(e3, j3));
                        j = next(j3);
                    }
                    for (; i < m_lane; ++i) {
                        a = fold(a, Op::lift(row[j], j));
                        j = next(j);
                    }
                }
            } else if (r < rows_t) {
                const elem_t* row = lds + off + r * L;
                unsigned int j = s;
                if constexpr (kEightReads) {
                    for (; j + 7 * S < C; j += 8 * S) {  // eight LDS reads in flight
                        elem_t e[8];
#pragma unroll
                        for (int k = 0; k < 8; ++k) e[k] = row[j + k * S];
#pragma unroll
                        for (int k = 0; k < 8; ++k) a = fold(a, Op::lift(e[k], j + k * S));
                    }
                }
                for (; j + 3 * S < C; j += 4 * S) {  // four LDS reads in flight
                    const elem_t e0 = row[j], e1 = row[j + S], e2 = row[j + 2 * S], e3 = row[j + 3 * S];
                    a = fold(a, Op::lift(e0, j));
                    a = fold(a, Op::lift(e1, j + S));
                    a = fold(a, Op::lift(e2, j + 2 * S));
                    a = fold(a, Op::lift(e3, j + 3 * S));
                }
                for (; j < C; j += S) a = fold(a, Op::lift(row[j], j));
            }
            a = segment_reduce<Op, LOG2S>(a);
            if (r < rows_t && leader) {
                if constexpr (HOLD)
                    held[k * R + r] = Op::finish(a);
                else
                    out[t * R + r] = Op::finish(a);
            }
        }
        __syncthreads();
    };
    // The wave's n tiles t0, t0 + G, ... run two per loop pass, one register
    // buffer each, with the odd or last two after the loop (a loop with one
    // exit, as in rows_packed_kernel, so that its head never waits for loads).
    const size_t first = work_block(xmap);  // wave-uniform
    if (first >= ntiles) return;
    const size_t mine = (ntiles - first + G - 1) / G;
    size_t n = mine, k = 0, t0 = first;
    vec_t a[U], b[U];
    load_tile(a, t0);
    for (; n > 2; n -= 2, k += 2, t0 += 2 * G) {
        load_tile(b, t0 + G);
        reduce_tile(a, t0, k);
        load_tile(a, t0 + 2 * G);
        reduce_tile(b, t0 + G, k + 1);
    }
    if (n == 2) {
        load_tile(b, t0 + G);
        reduce_tile(a, t0, k);
        reduce_tile(b, t0 + G, k + 1);
    } else {
        reduce_tile(a, t0, k);
    }
    if constexpr (HOLD) {
        // Held result i is row i % R of the wave's tile i / R.
        const unsigned int total = (unsigned int)(mine * R);
        for (unsigned int i = lane; i < total; i += kWave) {
            const unsigned int q = i / R, r = i - q * R;
            const size_t t = first + (size_t)q * G;
            if (r < rows_in(t)) out[t * R + r] = held[i];
        }
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

template <class Op, int BLOCK, int UNROLL>
inline hipError_t rows_bu(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                          typename Op::out_t* out, int grid, bool nt, bool pf, bool cover, int xmap,
                          hipStream_t stream) {
    const int xm = xmap > 0 && grid % (kXcds * xmap) == 0 ? xmap : 0;
    if (cover && !pf) {
        if (nt)
            hipLaunchKernelGGL((rows_cover_kernel<Op, BLOCK, UNROLL, true>), dim3(grid), dim3(BLOCK), 0, stream, x,
                               rows, cols, ld, out, xm);
        else
            hipLaunchKernelGGL((rows_cover_kernel<Op, BLOCK, UNROLL, false>), dim3(grid), dim3(BLOCK), 0, stream,
                               x, rows, cols, ld, out, xm);
        return hipGetLastError();
    }
    if (pf) {
        // The streaming kernel runs single-wave blocks: as many waves as the
        // BLOCK-thread grid holds, at most one per row.
        size_t waves = (size_t)grid * (BLOCK / kWave);
        if (waves > rows) waves = rows;
        const int xw = xmap > 0 && waves % (kXcds * (size_t)xmap) == 0 ? xmap : 0;
        if (nt)
            hipLaunchKernelGGL((rows_stream_kernel<Op, UNROLL, true>), dim3((unsigned int)waves), dim3(kWave), 0,
                               stream, x, rows, cols, ld, out, xw);
        else
            hipLaunchKernelGGL((rows_stream_kernel<Op, UNROLL, false>), dim3((unsigned int)waves), dim3(kWave), 0,
                               stream, x, rows, cols, ld, out, xw);
    } else if (nt) {
        hipLaunchKernelGGL((rows_reduce_kernel<Op, BLOCK, UNROLL, true>), dim3(grid), dim3(BLOCK), 0,
                           stream, x, rows, cols, ld, out, xm);
    } else {
        hipLaunchKernelGGL((rows_reduce_kernel<Op, BLOCK, UNROLL, false>), dim3(grid), dim3(BLOCK), 0,
                           stream, x, rows, cols, ld, out, xm);
    }
    return hipGetLastError();
}

template <class Op, int BLOCK>
inline hipError_t rows_b(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                         typename Op::out_t* out, int grid, bool cover, int xmap, const RowsPolicy& p,
                         hipStream_t stream) {
    const bool nt = p.nontemporal != 0;
    const bool pf = p.prefetch != 0;
    switch (p.unroll) {
        case 1: return rows_bu<Op, BLOCK, 1>(x, rows, cols, ld, out, grid, nt, pf, cover, xmap, stream);
        case 2: return rows_bu<Op, BLOCK, 2>(x, rows, cols, ld, out, grid, nt, pf, cover, xmap, stream);
        case 4: return rows_bu<Op, BLOCK, 4>(x, rows, cols, ld, out, grid, nt, pf, cover, xmap, stream);
        case 8: return rows_bu<Op, BLOCK, 8>(x, rows, cols, ld, out, grid, nt, pf, cover, xmap, stream);
        case 16: return rows_bu<Op, BLOCK, 16>(x, rows, cols, ld, out, grid, nt, pf, cover, xmap, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class Op, int UNROLL>
inline hipError_t rows_split_u(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
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

template <class Op, int LOG2L, int V, bool SCALAR>
inline hipError_t rows_packed_lv(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                                 typename Op::out_t* out, int grid, bool nt, int xmap, hipStream_t stream) {
    const int xm = xmap > 0 && grid % (kXcds * xmap) == 0 ? xmap : 0;
    if (nt)
        hipLaunchKernelGGL((rows_packed_kernel<Op, LOG2L, V, SCALAR, true>), dim3(grid), dim3(kWave), 0, stream,
                           x, rows, cols, ld, out, xm);
    else
        hipLaunchKernelGGL((rows_packed_kernel<Op, LOG2L, V, SCALAR, false>), dim3(grid), dim3(kWave), 0, stream,
                           x, rows, cols, ld, out, xm);
    return hipGetLastError();
}

// Several units per lane only with the widest segment (16 lanes for vectors,
// 64 for elements); narrower segments always take one.
template <class Op, int LOG2L, bool SCALAR>
inline hipError_t rows_packed_v(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                                typename Op::out_t* out, const RowsLaunch& L, bool nt, hipStream_t stream) {
    if constexpr (LOG2L == (SCALAR ? 6 : 4)) {
        switch (L.packed_v) {
            case 1: return rows_packed_lv<Op, LOG2L, 1, SCALAR>(x, rows, cols, ld, out, L.grid, nt, L.xmap, stream);
            case 2: return rows_packed_lv<Op, LOG2L, 2, SCALAR>(x, rows, cols, ld, out, L.grid, nt, L.xmap, stream);
            case 4: return rows_packed_lv<Op, LOG2L, 4, SCALAR>(x, rows, cols, ld, out, L.grid, nt, L.xmap, stream);
            case 8: return rows_packed_lv<Op, LOG2L, 8, SCALAR>(x, rows, cols, ld, out, L.grid, nt, L.xmap, stream);
            default: return hipErrorInvalidValue;
        }
    } else {
        if (L.packed_v != 1) return hipErrorInvalidValue;
        return rows_packed_lv<Op, LOG2L, 1, SCALAR>(x, rows, cols, ld, out, L.grid, nt, L.xmap, stream);
    }
}

template <class Op, bool SCALAR>
inline hipError_t rows_packed_s(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                                typename Op::out_t* out, const RowsLaunch& L, bool nt, hipStream_t stream) {
    switch (L.packed_log2l) {
        case 0: return rows_packed_v<Op, 0, SCALAR>(x, rows, cols, ld, out, L, nt, stream);
        case 1: return rows_packed_v<Op, 1, SCALAR>(x, rows, cols, ld, out, L, nt, stream);
        case 2: return rows_packed_v<Op, 2, SCALAR>(x, rows, cols, ld, out, L, nt, stream);
        case 3: return rows_packed_v<Op, 3, SCALAR>(x, rows, cols, ld, out, L, nt, stream);
        case 4: return rows_packed_v<Op, 4, SCALAR>(x, rows, cols, ld, out, L, nt, stream);
        default:
            if constexpr (SCALAR) {
                if (L.packed_log2l == 5) return rows_packed_v<Op, 5, SCALAR>(x, rows, cols, ld, out, L, nt, stream);
                if (L.packed_log2l == 6) return rows_packed_v<Op, 6, SCALAR>(x, rows, cols, ld, out, L, nt, stream);
            }
            return hipErrorInvalidValue;
    }
}

template <class Op, int LOG2S, int U, bool VREAD, bool SPREAD>
inline hipError_t rows_staged_go(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld, typename Op::out_t* out,
                                 const RowsLaunch& L, bool nt, hipStream_t stream) {
    const size_t held_bytes = (size_t)L.staged_hold * sizeof(typename Op::out_t);
    // x's offset, in elements, from the 16-byte boundary before it.
    const unsigned int sh = (unsigned int)(((uintptr_t)x % 16) / sizeof(typename Op::elem_t));
    // The staged tiles are always loaded non-temporally (the default of every
    // row shape): built only that way, which halves this kernel's variants.
    (void)nt;
    const int xm = L.xmap > 0 && L.grid % (kXcds * L.xmap) == 0 ? L.xmap : 0;
    // The hardware max fold is built for up to 4 lanes per row (the default
    // takes it with at most 2); wider segments fold with the compare and
    // select, which gives the same results.
    if constexpr (std::is_same_v<Op, MaxF32> && LOG2S <= 2) {
        if (L.staged_fmax) {
            if (L.staged_hold > 0)
                hipLaunchKernelGGL((rows_staged_kernel<Op, LOG2S, U, true, VREAD, true, SPREAD, true>), dim3(L.grid),
                                   dim3(kWave), held_bytes, stream, x, rows, cols, ld, sh, L.staged_rows, out, xm);
            else
                hipLaunchKernelGGL((rows_staged_kernel<Op, LOG2S, U, true, VREAD, false, SPREAD, true>), dim3(L.grid),
                                   dim3(kWave), 0, stream, x, rows, cols, ld, sh, L.staged_rows, out, xm);
            return hipGetLastError();
        }
    }
    if (L.staged_hold > 0)
        hipLaunchKernelGGL((rows_staged_kernel<Op, LOG2S, U, true, VREAD, true, SPREAD>), dim3(L.grid),
                           dim3(kWave), held_bytes, stream, x, rows, cols, ld, sh, L.staged_rows, out, xm);
    else
        hipLaunchKernelGGL((rows_staged_kernel<Op, LOG2S, U, true, VREAD, false, SPREAD>), dim3(L.grid),
                           dim3(kWave), 0, stream, x, rows, cols, ld, sh, L.staged_rows, out, xm);
    return hipGetLastError();
}

// Spread element reads are built only where the host asks for them: one or
// two lanes per row (32 or more rows per pass).
template <class Op, int LOG2S, int U, bool VREAD>
inline hipError_t rows_staged_suv(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld, typename Op::out_t* out,
                                  const RowsLaunch& L, bool nt, hipStream_t stream) {
    if constexpr (!VREAD && LOG2S <= 1) {
        if (L.staged_spread) return rows_staged_go<Op, LOG2S, U, false, true>(x, rows, cols, ld, out, L, nt, stream);
    } else {
        if (L.staged_spread) return hipErrorInvalidValue;
    }
    return rows_staged_go<Op, LOG2S, U, VREAD, false>(x, rows, cols, ld, out, L, nt, stream);
}

template <class Op, int LOG2S, int U>
inline hipError_t rows_staged_su(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld, typename Op::out_t* out,
                                 const RowsLaunch& L, bool nt, hipStream_t stream) {
    if (L.staged_vread) return rows_staged_suv<Op, LOG2S, U, true>(x, rows, cols, ld, out, L, nt, stream);
    return rows_staged_suv<Op, LOG2S, U, false>(x, rows, cols, ld, out, L, nt, stream);
}

template <class Op, int LOG2S>
inline hipError_t rows_staged_s(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld, typename Op::out_t* out,
                                const RowsLaunch& L, bool nt, hipStream_t stream) {
    switch (L.staged_u) {
        case 4: return rows_staged_su<Op, LOG2S, 4>(x, rows, cols, ld, out, L, nt, stream);
        case 8: return rows_staged_su<Op, LOG2S, 8>(x, rows, cols, ld, out, L, nt, stream);
        case 16: return rows_staged_su<Op, LOG2S, 16>(x, rows, cols, ld, out, L, nt, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class Op>
inline hipError_t rows_staged(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld, typename Op::out_t* out,
                              const RowsLaunch& L, bool nt, hipStream_t stream) {
    switch (L.staged_log2s) {
        case 0: return rows_staged_s<Op, 0>(x, rows, cols, ld, out, L, nt, stream);
        case 1: return rows_staged_s<Op, 1>(x, rows, cols, ld, out, L, nt, stream);
        case 2: return rows_staged_s<Op, 2>(x, rows, cols, ld, out, L, nt, stream);
        case 3: return rows_staged_s<Op, 3>(x, rows, cols, ld, out, L, nt, stream);
        case 4: return rows_staged_s<Op, 4>(x, rows, cols, ld, out, L, nt, stream);
        case 5: return rows_staged_s<Op, 5>(x, rows, cols, ld, out, L, nt, stream);
        case 6: return rows_staged_s<Op, 6>(x, rows, cols, ld, out, L, nt, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class Op>
inline hipError_t rows_op(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                          typename Op::out_t* out, const RowsLaunch& L, const RowsPolicy& p,
                          hipStream_t stream) {
    if (L.staged_u > 0) return rows_staged<Op>(x, rows, cols, ld, out, L, p.nontemporal != 0, stream);
    if (L.packed_v > 0) {
        if (L.packed_scalar) return rows_packed_s<Op, true>(x, rows, cols, ld, out, L, p.nontemporal != 0, stream);
        return rows_packed_s<Op, false>(x, rows, cols, ld, out, L, p.nontemporal != 0, stream);
    }
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
        case 64: return rows_b<Op, 64>(x, rows, cols, ld, out, L.grid, L.cover != 0, L.xmap, p, stream);
        case 128: return rows_b<Op, 128>(x, rows, cols, ld, out, L.grid, L.cover != 0, L.xmap, p, stream);
        case 256: return rows_b<Op, 256>(x, rows, cols, ld, out, L.grid, L.cover != 0, L.xmap, p, stream);
        case 512: return rows_b<Op, 512>(x, rows, cols, ld, out, L.grid, L.cover != 0, L.xmap, p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace libred
