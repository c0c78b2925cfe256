// cols_reduce.hip -- per-column sum and max of a row-major matrix (rows
// starting ld elements apart): out[c] = reduction over r of x[r*ld + c].
//
// The lesson's reduction folds contiguous data; here each output gathers one
// element from every row. A wave still reads contiguous memory: lane l owns
// VEC adjacent columns (one 16-byte load when VEC == 4), so a wave covers
// 64*VEC columns of a row per load (or several short rows at once when the
// matrix is narrow), and walks down its rows with UNROLL loads in flight. For
// parallelism when there are few columns, the rows are dealt round-robin to
// `nchunks` row phases; pass 1 stores one partial per (phase, column), and
// pass 2 adds each column's partials in a fixed order (deterministic): one
// wave per column (cols_combine_kernel), or one thread per column when there
// are many columns and few partials each (cols_combine_wide_kernel). With a
// single phase pass 1 stores the result directly. A contiguous matrix may be
// read as rows / m rows of m * cols columns (the host picks m; the kernels
// see an ordinary matrix): then pass 2 also adds the m partial columns of
// each column and the last rows % m rows (cols_fold_combine_kernel, or the
// wide kernel).
#include "device_common.hpp"
#include "launch.hpp"

namespace libred {

template <int VEC, class Op>
struct ColVec;
template <class Op>
struct ColVec<1, Op> {
    using type = typename Op::elem_t;
};
template <class Op>
struct ColVec<4, Op> {
    using type = typename Op::vec_t;
};

// One element into a column's accumulator. With FMAX (maxima only) the fold
// is a hardware max of the canonicalized element (a signalling NaN is made
// quiet first, so a NaN never wins; between -0 and +0 either may remain, as
// the max rule allows) instead of a compare and a select.
template <class Op, bool FMAX>
__device__ __forceinline__ typename Op::acc_t col_combine(typename Op::acc_t a, typename Op::elem_t e) {
    if constexpr (FMAX)
        return __builtin_fmaxf(a, __builtin_canonicalizef(e));
    else
        return Op::combine(a, Op::lift(e, 0));
}

template <class Op, int VEC, bool FMAX = false>
__device__ __forceinline__ void col_fold(typename Op::acc_t (&acc)[VEC], typename ColVec<VEC, Op>::type v) {
    if constexpr (VEC == 1) {
        acc[0] = col_combine<Op, FMAX>(acc[0], v);
    } else {
        acc[0] = col_combine<Op, FMAX>(acc[0], v.x);
        acc[1] = col_combine<Op, FMAX>(acc[1], v.y);
        acc[2] = col_combine<Op, FMAX>(acc[2], v.z);
        acc[3] = col_combine<Op, FMAX>(acc[3], v.w);
    }
}

// The four columns a lane owns in a row whose first of them sits at position
// s (0-3) of aligned vector v0: elements s..3 of v0, then 0..s-1 of v1 (the
// next aligned vector).
// The choice is made with bit masks (bitfield inserts), not branches: as a
// chain of conditionals on s the compiler branched on every element. The
// vectors are reinterpreted whole (a bit cast of one vector component, as
// in __builtin_bit_cast(uint32_t, v.y), compiled to a read of component 0).
template <class Op, bool FMAX = false>
__device__ __forceinline__ void col_fold_shift(typename Op::acc_t (&acc)[4], typename Op::vec_t v0,
                                               typename Op::vec_t v1, unsigned int s) {
    using elem_t = typename Op::elem_t;
    static_assert(sizeof(typename Op::vec_t) == sizeof(u32x4), "four four-byte elements");
    const u32x4 w0 = __builtin_bit_cast(u32x4, v0), w1 = __builtin_bit_cast(u32x4, v1);
    const uint32_t e[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    const uint32_t m1 = 0u - (s & 1u), m2 = 0u - ((s >> 1) & 1u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (e[i + 1] & m1) | (e[i] & ~m1);      // element i + (s & 1)
        const uint32_t hi = (e[i + 3] & m1) | (e[i + 2] & ~m1);  // element i + 2 + (s & 1)
        const elem_t t = __builtin_bit_cast(elem_t, (hi & m2) | (lo & ~m2));
        acc[i] = col_combine<Op, FMAX>(acc[i], t);
    }
}

// Lane l + 1's vector v (a DPP rotate of the wave by one lane, wave_rol:1);
// lane 63 gets lane 0's vector `after` instead. A lane whose source lane is
// inactive gets 0.
template <class V>
__device__ __forceinline__ V next_lane_vec(V v, V after, unsigned int lane) {
    static_assert(sizeof(V) == sizeof(u32x4), "four four-byte elements");
    constexpr int kWaveRol1 = 0x134;
    const u32x4 a = __builtin_bit_cast(u32x4, v), b = __builtin_bit_cast(u32x4, after);
    const bool first = lane == 0;  // lane 0 lends `after` to lane 63
    u32x4 r;
    r.x = __builtin_amdgcn_update_dpp(0u, first ? b.x : a.x, kWaveRol1, 0xf, 0xf, false);
    r.y = __builtin_amdgcn_update_dpp(0u, first ? b.y : a.y, kWaveRol1, 0xf, 0xf, false);
    r.z = __builtin_amdgcn_update_dpp(0u, first ? b.z : a.z, kWaveRol1, 0xf, 0xf, false);
    r.w = __builtin_amdgcn_update_dpp(0u, first ? b.w : a.w, kWaveRol1, 0xf, 0xf, false);
    return __builtin_bit_cast(V, r);
}

// Block b: column block j = b % ncb, row phase k = b / ncb of the
// K = gridDim.x / ncb phases. Phase k takes rows k, k + K, k + 2K, ... (in
// groups of 64 / ngroups rows, see below), so the waves of one column block
// move down the matrix together and the whole grid sweeps it front to back,
// as the single-value kernel sweeps its array; giving each wave a contiguous
// chunk of rows instead ran 4-8% slower on 1 GiB matrices. A wave covers
// `ngroups` column groups of VEC columns per load: normally ngroups == 64
// (one group per lane), and each row is read with CW loads that cover
// CW * 64 * VEC adjacent columns (CW KiB when VEC == 4), lane l taking
// columns l*VEC + w*64*VEC for w < CW. For narrow matrices (CW == 1 only)
// ngroups divides 64 and the wave's lanes cover 64 / ngroups rows per load
// (lane l: group l % ngroups, row offset l / ngroups); lanes of one group are
// added with shuffles at the end. With VEC == 4, cols and ld are multiples of
// 4 and x is 16-byte aligned. In the last column block a lane whose column
// w lies past the end reads its column-0 vector again instead (so every load
// stays in bounds and no load is predicated) and never stores that result.
// With SHIFT (VEC == 4, any x, cols and ld) a row's four columns of a lane
// start at any position s of an aligned 16-byte vector: the lane loads that
// vector, takes the next one from the lane holding it (lane l + 1; lane 63
// takes lane 0's vector of its next column group), and picks its columns
// from the two. So each block owns cspan columns, one group fewer than its
// lanes cover: the last group of a packed row, or lane 63's last group, is
// a spare that only lends its vector. Every lane of a row group loads, also
// past cols (for its neighbour), with the vector index clamped to the one
// holding the row's last column, so no load reaches past the matrix; the
// first vector can begin before x, but only within the aligned vector
// holding x[0]. Columns past cols, and spare groups, are never stored.
template <class Op, int VEC, int CW, int UNROLL, bool NT, bool PREFETCH, bool SHIFT = false, bool FMAX = false>
__global__ __launch_bounds__(kWave) void cols_partial_kernel(const typename Op::elem_t* __restrict__ x,
                                                             size_t rows, size_t cols, size_t ld,
                                                             size_t ncb, unsigned int ngroups, size_t cspan,
                                                             int order, int xmap,
                                                             typename Op::acc_t* __restrict__ partials,
                                                             typename Op::out_t* __restrict__ out) {
    using acc_t = typename Op::acc_t;
    using V = typename ColVec<VEC, Op>::type;
    const unsigned int lane = threadIdx.x;
    const size_t nphases = gridDim.x / ncb;
    // xmap: the blocks of one XCD (blocks are dealt to the kXcds XCDs in
    // turn, block b to XCD b mod kXcds) take one contiguous range of block
    // indices i = j + k * ncb, XCD x the range from x * (G / kXcds) +
    // min(x, G mod kXcds), so that a line two neighbouring column blocks, or
    // two adjacent rows, share is fetched into one XCD's L2. With nphases a
    // multiple of kXcds each XCD holds every column block of a run of whole
    // phases.
    size_t bi = blockIdx.x;
    if (xmap) {
        const size_t x = blockIdx.x % kXcds, per = gridDim.x / kXcds, extra = gridDim.x % kXcds;
        bi = x * per + (x < extra ? x : extra) + blockIdx.x / kXcds;
    }
    const size_t j = bi % ncb;
    const size_t k = bi / ncb;
    const unsigned int g = lane % ngroups;
    const size_t group = kWave / ngroups;  // rows per load
    const size_t q = lane / ngroups;
    const size_t span = (size_t)ngroups * VEC;  // columns per load
    const size_t cstart = j * (SHIFT ? cspan : span * CW);
    const size_t c0 = cstart + (size_t)g * VEC;
    // The phase's rows r0 + q, r0 + q + rpl, ... below r1: every nphases-th
    // group of rows (orders 0 and 1), or one run of consecutive rows (order
    // 2: phase k takes rows [k * per, (k + 1) * per), per a multiple of the
    // group).
    size_t r0, r1, rpl;
    if (order == 2) {
        const size_t per = (rows + nphases * group - 1) / (nphases * group) * group;
        r0 = k * per;
        r1 = r0 + per < rows ? r0 + per : rows;
        rpl = group;
    } else {
        r0 = k * group;
        r1 = rows;
        rpl = group * nphases;
    }
    acc_t acc[CW][VEC];
#pragma unroll
    for (int w = 0; w < CW; ++w)
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[w][i] = Op::identity();
    // Lanes past the last whole row group of a load stay idle, and so (but
    // for SHIFT) do lanes past the last column.
    if ((SHIFT || c0 < cols) && q < group && r0 < r1) {
        size_t off[CW];  // in V units from the lane's column-0 vector
#pragma unroll
        for (int w = 0; w < CW; ++w) off[w] = (SHIFT || c0 + w * span < cols) ? w * (size_t)ngroups : 0;
        const size_t step = ld / VEC * rpl;  // in V units, between a lane's consecutive rows
        constexpr size_t U = UNROLL;
        // SHIFT: positions are elements from the aligned vector at or before
        // x (xv), a row's columns of this lane at xoff + r * ld + c0.
        const size_t xoff = SHIFT ? ((uintptr_t)x & 15) / sizeof(typename Op::elem_t) : 0;
        const V* __restrict__ xv = reinterpret_cast<const V*>(x - xoff);
        const size_t estep = ld * rpl;  // elements between a lane's consecutive rows
        struct Buf {
            V v[UNROLL][CW];
            unsigned int s[SHIFT ? UNROLL : 1];
        };
        // A lane's row at position e: one vector per column group, clamped
        // to the vector holding the row's last column (a vector past it
        // holds none of the row's columns, so no lane needs it; the clamp
        // keeps every load in the row's own lines).
        auto load_shift = [&](V (&v0)[CW], unsigned int& sh, size_t e) {
            sh = (unsigned int)(e % VEC);
            const size_t alast = (e - c0 + cols - 1) / VEC;
#pragma unroll
            for (int w = 0; w < CW; ++w) {
                const size_t a = e / VEC + off[w];
                v0[w] = load_vec<NT>(xv + (a < alast ? a : alast));
            }
        };
        // Fold a row's groups, each with the vector after it from the next lane.
        auto fold_shift = [&](const V (&v0)[CW], unsigned int sh) {
            if constexpr (SHIFT) {
#pragma unroll
                for (int w = 0; w < CW; ++w)
                    col_fold_shift<Op, FMAX>(acc[w], v0[w], next_lane_vec(v0[w], v0[w + 1 < CW ? w + 1 : w], lane), sh);
            }
        };
        // Fold rows r, r + rpl, ... below rend. Groups of UNROLL rows; with
        // PREFETCH, two register buffers alternate: the next group's loads
        // are issued before the current group is folded, so a wave keeps two
        // groups in flight. The scheduling barrier keeps a group's loads
        // issued back to back (left alone, the compiler sometimes interleaves
        // them with waits for the previous group, halving the loads in
        // flight).
        auto sweep = [&](size_t r, size_t rend) {
            // The cursor: row r's column-0 vector (p), or its position (e).
            const V* __restrict__ p = reinterpret_cast<const V*>(x + (SHIFT ? 0 : r * ld + c0));
            size_t e = xoff + r * ld + c0;
            auto load_group = [&](Buf& b, const V* __restrict__ g, size_t ge) {
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    if constexpr (SHIFT) {
                        load_shift(b.v[u], b.s[u], ge + u * estep);
                    } else {
#pragma unroll
                        for (int w = 0; w < CW; ++w) b.v[u][w] = load_vec<NT>(g + u * step + off[w]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            auto fold_group = [&](const Buf& b) {
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    if constexpr (SHIFT) {
                        fold_shift(b.v[u], b.s[u]);
                    } else {
#pragma unroll
                        for (int w = 0; w < CW; ++w) col_fold<Op, VEC, FMAX>(acc[w], b.v[u][w]);
                    }
                }
            };
            auto advance = [&]() { r += U * rpl, p += U * step, e += U * estep; };
            if (!PREFETCH) {
                for (; r + (U - 1) * rpl < rend; advance()) {
                    Buf v;
                    load_group(v, p, e);
                    fold_group(v);
                }
            } else if (r + (U - 1) * rpl < rend) {
                Buf a, b;
                load_group(a, p, e);
                while (true) {
                    if (r + (2 * U - 1) * rpl >= rend) {
                        fold_group(a);
                        advance();
                        break;
                    }
                    load_group(b, p + U * step, e + U * estep);
                    fold_group(a);
                    advance();
                    if (r + (2 * U - 1) * rpl >= rend) {
                        fold_group(b);
                        advance();
                        break;
                    }
                    load_group(a, p + U * step, e + U * estep);
                    fold_group(b);
                    advance();
                }
            }
            for (; r < rend; r += rpl, p += step, e += estep) {
                if constexpr (SHIFT) {
                    V v0[CW];
                    unsigned int sh;
                    load_shift(v0, sh, e);
                    fold_shift(v0, sh);
                } else {
#pragma unroll
                    for (int w = 0; w < CW; ++w) col_fold<Op, VEC, FMAX>(acc[w], load_vec<NT>(p + off[w]));
                }
            }
        };
        // The wave visits its rows in nvis rounds (round i: rows r0 + i * rpl
        // + q). In order 1, block b starts at round b mod nvis and wraps
        // around to round 0, so that the waves of a launch read rows spread
        // over the matrix rather than one band of it.
        const size_t nvis = (r1 - r0 + rpl - 1) / rpl;  // r0 < r1 here
        const size_t split = r0 + (order == 1 ? (size_t)blockIdx.x % nvis : 0) * rpl;
#pragma unroll 1
        for (int part = 0; part < 2; ++part) {  // rounds from the split on, then those before it
            const size_t rb = part == 0 ? split + q : r0 + q;
            const size_t re = part == 0 ? r1 : (split + q < r1 ? split + q : r1);
            sweep(rb, re);
        }
    }
    // Packed rows (CW == 1): lane g collects lanes g + ngroups, g + 2*ngroups,
    // ... in a fixed order (all lanes take part in the shuffles): a halving
    // tree when ngroups divides 64, else one lane after another.
    if ((kWave % ngroups) == 0) {
        for (unsigned int sh = kWave / 2; sh >= ngroups; sh >>= 1) {
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[0][i] = Op::combine(acc[0][i], __shfl_down(acc[0][i], sh, kWave));
        }
    } else {
        for (size_t m = 1; m < group; ++m) {
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                const acc_t t = __shfl(acc[0][i], (int)(lane + m * ngroups) % kWave, kWave);
                if (q == 0) acc[0][i] = Op::combine(acc[0][i], t);
            }
        }
    }
    if (q == 0) {
#pragma unroll
        for (int w = 0; w < CW; ++w) {
            const size_t c = c0 + w * span;
            if (c >= cols || (SHIFT && c - cstart >= cspan)) continue;
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                if (SHIFT && c + i >= cols) continue;
                if (out != nullptr)
                    out[c + i] = Op::finish(acc[w][i]);
                else
                    partials[k * cols + c + i] = acc[w][i];
            }
        }
    }
}

// Pass 2: one wave per column; its lanes take chunks lane, lane + 64, ...,
// then the DPP wave reduce adds them in a fixed order.
constexpr int kColsCombineBlock = 256;

template <class Op>
__global__ __launch_bounds__(kColsCombineBlock) void cols_combine_kernel(
    const typename Op::acc_t* __restrict__ partials, size_t nchunks, size_t cols,
    typename Op::out_t* __restrict__ out) {
    constexpr int W = kColsCombineBlock / kWave;
    const unsigned int lane = threadIdx.x % kWave;
    const size_t c = (size_t)blockIdx.x * W + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (c >= cols) return;  // wave-uniform
    typename Op::acc_t v = Op::identity();
    for (size_t k = lane; k < nchunks; k += kWave) v = Op::combine(v, partials[k * cols + c]);
    v = wave_reduce<Op>(v);
    if (lane == 0) out[c] = Op::finish(v);
}

// Pass 2 of a launch on a view (see ColsLaunch): the partials of real column
// c are items j * cols + rc for j < nchunks * m (chunk j / m, view column
// (j % m) * cols + rc), rc = (c - rot) mod cols its place in a run of cols
// view columns; then its elements after the view (tail elements rc,
// rc + cols, ...) and before it (head elements c, c + cols, ... < rot). One
// block per real column: items dealt to the threads in rounds of
// 4 * kColsCombineBlock (4 loads in flight per thread, each from a clamped
// index so no load is predicated), then the tail and head elements,
// thread-strided, then the block reduce. The order is fixed, so the result
// is deterministic.
template <class Op>
__global__ __launch_bounds__(kColsCombineBlock) void cols_fold_combine_kernel(
    const typename Op::acc_t* __restrict__ partials, unsigned int items, size_t cols,
    const typename Op::elem_t* __restrict__ tail, size_t tail_elems, unsigned int rot,
    const typename Op::elem_t* __restrict__ head, typename Op::out_t* __restrict__ out) {
    using acc_t = typename Op::acc_t;
    __shared__ acc_t lds[kColsCombineBlock / kWave];
    const size_t c = blockIdx.x;
    const size_t rc = (c + cols - rot % cols) % cols;
    acc_t v = Op::identity();
    for (unsigned int j0 = 0; j0 < items; j0 += 4 * kColsCombineBlock) {
        acc_t t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const unsigned int j = j0 + u * kColsCombineBlock + threadIdx.x;
            t[u] = partials[(size_t)(j < items ? j : items - 1) * cols + rc];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (j0 + u * kColsCombineBlock + threadIdx.x < items) v = Op::combine(v, t[u]);
    }
    for (size_t i = rc + (size_t)threadIdx.x * cols; i < tail_elems; i += (size_t)kColsCombineBlock * cols)
        v = Op::combine(v, Op::lift(tail[i], 0));
    for (size_t f = c + (size_t)threadIdx.x * cols; f < rot; f += (size_t)kColsCombineBlock * cols)
        v = Op::combine(v, Op::lift(head[f], 0));
    v = block_reduce<Op, kColsCombineBlock>(v, lds);
    if (threadIdx.x == 0) out[c] = Op::finish(v);
}

// Pass 2 when there are many columns and few partials each: one thread per
// column adds items j * cols + rc for j < items in order (consecutive threads
// read consecutive partials, so the reads coalesce), 8 loads in flight, then
// its tail and head elements in order (as in cols_fold_combine_kernel).
// Serves views and plain launches alike (m = 1, rot = 0, no tail).
template <class Op>
__global__ __launch_bounds__(kColsCombineBlock) void cols_combine_wide_kernel(
    const typename Op::acc_t* __restrict__ partials, unsigned int items, size_t cols,
    const typename Op::elem_t* __restrict__ tail, size_t tail_elems, unsigned int rot,
    const typename Op::elem_t* __restrict__ head, typename Op::out_t* __restrict__ out) {
    using acc_t = typename Op::acc_t;
    const size_t c0 = (size_t)blockIdx.x * kColsCombineBlock + threadIdx.x;
    if (c0 >= cols) return;
    // Thread c0 takes the partials of run position c0, those of real column
    // c = (c0 + rot) mod cols.
    const size_t c = (c0 + rot) % cols;
    acc_t v = Op::identity();
    for (unsigned int j0 = 0; j0 < items; j0 += 8) {
        acc_t t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const unsigned int j = j0 + u < items ? j0 + u : items - 1;  // uniform
            t[u] = partials[(size_t)j * cols + c0];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (j0 + u < items) v = Op::combine(v, t[u]);
    }
    for (size_t i = c0; i < tail_elems; i += cols) v = Op::combine(v, Op::lift(tail[i], 0));
    for (size_t f = c; f < rot; f += cols) v = Op::combine(v, Op::lift(head[f], 0));
    out[c] = Op::finish(v);
}

bool cols_policy_supported(const ColsPolicy& p) {
    const bool u = p.unroll == 1 || p.unroll == 2 || p.unroll == 4 || p.unroll == 8 || p.unroll == 16;
    const bool w = p.width == 1 || p.width == 2 || p.width == 4;
    return u && w && (p.nontemporal == 0 || p.nontemporal == 1) && (p.prefetch == 0 || p.prefetch == 1) &&
           p.target_waves >= 1 && (p.vec == 0 || p.vec == 1 || p.vec == 4) && p.fold >= 0 && p.fold <= 64 &&
           p.order >= 0 && p.order <= 3 && p.xcd >= 0 && p.xcd <= 2;
}

template <class Op, int VEC, int CW, int UNROLL, bool PF, bool SH>
static hipError_t cols_vwup(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                            typename Op::out_t* out, const ColsLaunch& L, bool nt, hipStream_t stream) {
    auto* partials = static_cast<typename Op::acc_t*>(L.partials);
    const dim3 grid((unsigned int)(L.ncb * L.nchunks));
    typename Op::out_t* direct = (L.nchunks == 1 && L.fold_m <= 1 && L.rot == 0) ? out : nullptr;
    // The hardware max fold is built for the shapes whose launches take it
    // by default (folded views of fewer than 256 real columns: 8 rows in
    // flight, one load per row, prefetch; short-wide matrices: 2 rows in
    // flight, four loads per row); other shapes fold with the compare and
    // select, which gives the same results.
    bool launched = false;
    if constexpr (std::is_same_v<Op, MaxF32> && VEC == 4 && !SH &&
                  ((CW == 1 && UNROLL == 8 && PF) || (CW == 4 && UNROLL == 2))) {
        if (L.col_fmax && nt) {
            hipLaunchKernelGGL((cols_partial_kernel<Op, VEC, CW, UNROLL, true, PF, false, true>), grid, dim3(kWave), 0,
                               stream, x, rows, cols, ld, L.ncb, L.ngroups, L.cspan, L.order, L.xmap, partials,
                               direct);
            launched = true;
        }
    }
    // Shifted loads are built non-temporal only (the default of every shape
    // that takes them), which halves their variants.
    if (!launched) {
        if (nt || SH)
            hipLaunchKernelGGL((cols_partial_kernel<Op, VEC, CW, UNROLL, true, PF, SH>), grid, dim3(kWave), 0, stream,
                               x, rows, cols, ld, L.ncb, L.ngroups, L.cspan, L.order, L.xmap, partials, direct);
        else if constexpr (!SH)
            hipLaunchKernelGGL((cols_partial_kernel<Op, VEC, CW, UNROLL, false, PF, false>), grid, dim3(kWave), 0,
                               stream, x, rows, cols, ld, L.ncb, L.ngroups, L.cspan, L.order, L.xmap, partials,
                               direct);
    }
    hipError_t e = hipGetLastError();
    const size_t W = kColsCombineBlock / kWave;
    if (e != hipSuccess) return e;
    if (direct != nullptr) return e;
    // Items per real column; with at least 64 columns per item, one thread
    // per column (coalesced), else one block or wave per column.
    const size_t items = L.nchunks * (size_t)(L.fold_m > 1 ? L.fold_m : 1);
    const auto* tail = static_cast<const typename Op::elem_t*>(L.tail);
    const auto* head = static_cast<const typename Op::elem_t*>(L.head);
    if (items * 64 <= L.real_cols) {
        const size_t nb = (L.real_cols + kColsCombineBlock - 1) / kColsCombineBlock;
        hipLaunchKernelGGL((cols_combine_wide_kernel<Op>), dim3((unsigned int)nb), dim3(kColsCombineBlock), 0, stream,
                           partials, (unsigned int)items, L.real_cols, tail, L.tail_elems, L.rot, head, out);
        return hipGetLastError();
    }
    if (L.fold_m > 1 || L.rot > 0) {
        hipLaunchKernelGGL((cols_fold_combine_kernel<Op>), dim3((unsigned int)L.real_cols), dim3(kColsCombineBlock),
                           0, stream, partials, (unsigned int)items, L.real_cols, tail, L.tail_elems, L.rot, head,
                           out);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((cols_combine_kernel<Op>), dim3((unsigned int)((cols + W - 1) / W)),
                       dim3(kColsCombineBlock), 0, stream, partials, L.nchunks, cols, out);
    return hipGetLastError();
}

template <class Op, int VEC, int CW, int UNROLL, bool SH>
static hipError_t cols_vwu(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                           typename Op::out_t* out, const ColsLaunch& L, bool nt, bool pf, hipStream_t stream) {
    if (pf) return cols_vwup<Op, VEC, CW, UNROLL, true, SH>(x, rows, cols, ld, out, L, nt, stream);
    return cols_vwup<Op, VEC, CW, UNROLL, false, SH>(x, rows, cols, ld, out, L, nt, stream);
}

template <class Op, int VEC, int CW, bool SH>
static hipError_t cols_vw(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                          typename Op::out_t* out, const ColsLaunch& L, const ColsPolicy& p, hipStream_t stream) {
    const bool nt = p.nontemporal != 0;
    const bool pf = p.prefetch != 0;
    switch (p.unroll) {
        case 1: return cols_vwu<Op, VEC, CW, 1, SH>(x, rows, cols, ld, out, L, nt, pf, stream);
        case 2: return cols_vwu<Op, VEC, CW, 2, SH>(x, rows, cols, ld, out, L, nt, pf, stream);
        case 4: return cols_vwu<Op, VEC, CW, 4, SH>(x, rows, cols, ld, out, L, nt, pf, stream);
        case 8: return cols_vwu<Op, VEC, CW, 8, SH>(x, rows, cols, ld, out, L, nt, pf, stream);
        case 16: return cols_vwu<Op, VEC, CW, 16, SH>(x, rows, cols, ld, out, L, nt, pf, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class Op>
static hipError_t cols_op(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                          typename Op::out_t* out, const ColsLaunch& L, const ColsPolicy& p, hipStream_t stream) {
    if (L.vec != 4) {
        switch (L.width) {
            case 1: return cols_vw<Op, 1, 1, false>(x, rows, cols, ld, out, L, p, stream);
            case 2: return cols_vw<Op, 1, 2, false>(x, rows, cols, ld, out, L, p, stream);
            case 4: return cols_vw<Op, 1, 4, false>(x, rows, cols, ld, out, L, p, stream);
            default: return hipErrorInvalidValue;
        }
    }
    if (L.shift) {
        switch (L.width) {
            case 1: return cols_vw<Op, 4, 1, true>(x, rows, cols, ld, out, L, p, stream);
            case 2: return cols_vw<Op, 4, 2, true>(x, rows, cols, ld, out, L, p, stream);
            case 4: return cols_vw<Op, 4, 4, true>(x, rows, cols, ld, out, L, p, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (L.width) {
        case 1: return cols_vw<Op, 4, 1, false>(x, rows, cols, ld, out, L, p, stream);
        case 2: return cols_vw<Op, 4, 2, false>(x, rows, cols, ld, out, L, p, stream);
        case 4: return cols_vw<Op, 4, 4, false>(x, rows, cols, ld, out, L, p, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_cols_sum_f32(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                               const ColsLaunch& L, const ColsPolicy& p, hipStream_t stream) {
    return cols_op<SumF32>(x, rows, cols, ld, out, L, p, stream);
}

hipError_t launch_cols_max_f32(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                               const ColsLaunch& L, const ColsPolicy& p, hipStream_t stream) {
    return cols_op<MaxF32>(x, rows, cols, ld, out, L, p, stream);
}

}  // namespace libred
