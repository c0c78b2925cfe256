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

template <class Op, int VEC>
__device__ __forceinline__ void col_fold(typename Op::acc_t (&acc)[VEC], typename ColVec<VEC, Op>::type v) {
    if constexpr (VEC == 1) {
        acc[0] = Op::combine(acc[0], Op::lift(v, 0));
    } else {
        acc[0] = Op::combine(acc[0], Op::lift(v.x, 0));
        acc[1] = Op::combine(acc[1], Op::lift(v.y, 0));
        acc[2] = Op::combine(acc[2], Op::lift(v.z, 0));
        acc[3] = Op::combine(acc[3], Op::lift(v.w, 0));
    }
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
template <class Op, int VEC, int CW, int UNROLL, bool NT, bool PREFETCH>
__global__ __launch_bounds__(kWave) void cols_partial_kernel(const typename Op::elem_t* __restrict__ x,
                                                             size_t rows, size_t cols, size_t ld,
                                                             size_t ncb, unsigned int ngroups, int order,
                                                             typename Op::acc_t* __restrict__ partials,
                                                             typename Op::out_t* __restrict__ out) {
    using acc_t = typename Op::acc_t;
    using V = typename ColVec<VEC, Op>::type;
    const unsigned int lane = threadIdx.x;
    const size_t j = blockIdx.x % ncb;
    const size_t k = blockIdx.x / ncb;
    const size_t nphases = gridDim.x / ncb;
    const unsigned int g = lane % ngroups;
    const size_t group = kWave / ngroups;  // rows per load
    const size_t q = lane / ngroups;
    const size_t span = (size_t)ngroups * VEC;  // columns per load
    const size_t c0 = j * span * CW + (size_t)g * VEC;
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
    if (c0 < cols && q < group && r0 < r1) {  // lanes past the last whole row group of a load stay idle
        size_t off[CW];  // in V units from the lane's column-0 vector
#pragma unroll
        for (int w = 0; w < CW; ++w) off[w] = c0 + w * span < cols ? w * (size_t)ngroups : 0;
        const size_t step = ld / VEC * rpl;  // in V units, between a lane's consecutive rows
        constexpr size_t U = UNROLL;
        // Fold rows r, r + rpl, ... below rend. Groups of UNROLL rows; with
        // PREFETCH, two register buffers alternate: the next group's loads
        // are issued before the current group is folded, so a wave keeps two
        // groups in flight. The scheduling barrier keeps a group's loads
        // issued back to back (left alone, the compiler sometimes interleaves
        // them with waits for the previous group, halving the loads in
        // flight).
        auto sweep = [&](size_t r, size_t rend) {
            const V* __restrict__ p = reinterpret_cast<const V*>(x + r * ld + c0);
            auto load_group = [&](V (&v)[UNROLL][CW], const V* __restrict__ g) {
#pragma unroll
                for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                    for (int w = 0; w < CW; ++w) v[u][w] = load_vec<NT>(g + u * step + off[w]);
                __builtin_amdgcn_sched_barrier(0);
            };
            auto fold_group = [&](const V (&v)[UNROLL][CW]) {
#pragma unroll
                for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                    for (int w = 0; w < CW; ++w) col_fold<Op, VEC>(acc[w], v[u][w]);
            };
            if (!PREFETCH) {
                for (; r + (U - 1) * rpl < rend; r += U * rpl, p += U * step) {
                    V v[UNROLL][CW];
                    load_group(v, p);
                    fold_group(v);
                }
            } else if (r + (U - 1) * rpl < rend) {
                V a[UNROLL][CW], b[UNROLL][CW];
                load_group(a, p);
                while (true) {
                    if (r + (2 * U - 1) * rpl >= rend) {
                        fold_group(a);
                        r += U * rpl, p += U * step;
                        break;
                    }
                    load_group(b, p + U * step);
                    fold_group(a);
                    r += U * rpl, p += U * step;
                    if (r + (2 * U - 1) * rpl >= rend) {
                        fold_group(b);
                        r += U * rpl, p += U * step;
                        break;
                    }
                    load_group(a, p + U * step);
                    fold_group(b);
                    r += U * rpl, p += U * step;
                }
            }
            for (; r < rend; r += rpl, p += step) {
#pragma unroll
                for (int w = 0; w < CW; ++w) col_fold<Op, VEC>(acc[w], load_vec<NT>(p + off[w]));
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
            if (c >= cols) continue;
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
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
           p.order >= 0 && p.order <= 3;
}

template <class Op, int VEC, int CW, int UNROLL, bool PF>
static hipError_t cols_vwup(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                            typename Op::out_t* out, const ColsLaunch& L, bool nt, hipStream_t stream) {
    auto* partials = static_cast<typename Op::acc_t*>(L.partials);
    const dim3 grid((unsigned int)(L.ncb * L.nchunks));
    typename Op::out_t* direct = (L.nchunks == 1 && L.fold_m <= 1 && L.rot == 0) ? out : nullptr;
    if (nt)
        hipLaunchKernelGGL((cols_partial_kernel<Op, VEC, CW, UNROLL, true, PF>), grid, dim3(kWave), 0, stream, x,
                           rows, cols, ld, L.ncb, L.ngroups, L.order, partials, direct);
    else
        hipLaunchKernelGGL((cols_partial_kernel<Op, VEC, CW, UNROLL, false, PF>), grid, dim3(kWave), 0, stream, x,
                           rows, cols, ld, L.ncb, L.ngroups, L.order, partials, direct);
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

template <class Op, int VEC, int CW, int UNROLL>
static hipError_t cols_vwu(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                           typename Op::out_t* out, const ColsLaunch& L, bool nt, bool pf, hipStream_t stream) {
    if (pf) return cols_vwup<Op, VEC, CW, UNROLL, true>(x, rows, cols, ld, out, L, nt, stream);
    return cols_vwup<Op, VEC, CW, UNROLL, false>(x, rows, cols, ld, out, L, nt, stream);
}

template <class Op, int VEC, int CW>
static hipError_t cols_vw(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                          typename Op::out_t* out, const ColsLaunch& L, const ColsPolicy& p, hipStream_t stream) {
    const bool nt = p.nontemporal != 0;
    const bool pf = p.prefetch != 0;
    switch (p.unroll) {
        case 1: return cols_vwu<Op, VEC, CW, 1>(x, rows, cols, ld, out, L, nt, pf, stream);
        case 2: return cols_vwu<Op, VEC, CW, 2>(x, rows, cols, ld, out, L, nt, pf, stream);
        case 4: return cols_vwu<Op, VEC, CW, 4>(x, rows, cols, ld, out, L, nt, pf, stream);
        case 8: return cols_vwu<Op, VEC, CW, 8>(x, rows, cols, ld, out, L, nt, pf, stream);
        case 16: return cols_vwu<Op, VEC, CW, 16>(x, rows, cols, ld, out, L, nt, pf, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class Op>
static hipError_t cols_op(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                          typename Op::out_t* out, const ColsLaunch& L, const ColsPolicy& p, hipStream_t stream) {
    if (L.vec != 4) {
        switch (L.width) {
            case 1: return cols_vw<Op, 1, 1>(x, rows, cols, ld, out, L, p, stream);
            case 2: return cols_vw<Op, 1, 2>(x, rows, cols, ld, out, L, p, stream);
            case 4: return cols_vw<Op, 1, 4>(x, rows, cols, ld, out, L, p, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (L.width) {
        case 1: return cols_vw<Op, 4, 1>(x, rows, cols, ld, out, L, p, stream);
        case 2: return cols_vw<Op, 4, 2>(x, rows, cols, ld, out, L, p, stream);
        case 4: return cols_vw<Op, 4, 4>(x, rows, cols, ld, out, L, p, stream);
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
