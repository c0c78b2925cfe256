// cols_reduce.hip -- per-column sum and max of a row-major matrix (rows
// starting ld elements apart): out[c] = reduction over r of x[r*ld + c].
//
// The lesson's reduction folds contiguous data; here each output gathers one
// element from every row. A wave still reads contiguous memory: lane l owns
// VEC adjacent columns (one 16-byte load when VEC == 4), so a wave covers
// 64*VEC columns of a row per load (or several short rows at once when the
// matrix is narrow), and walks down its rows with UNROLL loads in flight. For
// parallelism when there are few columns, the rows are cut into `nchunks`
// chunks; pass 1 stores one partial per (chunk, column), and pass 2 adds each
// column's partials with one wave per column in a fixed order
// (deterministic). With a single chunk pass 1 stores the result directly.
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

// Block b: column block j = b % ncb, row chunk k = b / ncb. A wave covers
// `ngroups` column groups of VEC columns per load: normally ngroups == 64
// (one group per lane, 64*VEC columns per block); for narrow matrices
// ngroups divides 64 and the wave's lanes cover 64 / ngroups rows per load
// (lane l: group l % ngroups, row offset l / ngroups), and lanes of one group
// are added with shuffles at the end. With VEC == 4, cols and ld are
// multiples of 4 and x is 16-byte aligned.
template <class Op, int VEC, int UNROLL, bool NT>
__global__ __launch_bounds__(kWave) void cols_partial_kernel(const typename Op::elem_t* __restrict__ x,
                                                             size_t rows, size_t cols, size_t ld,
                                                             size_t rchunk, size_t ncb, unsigned int ngroups,
                                                             typename Op::acc_t* __restrict__ partials,
                                                             typename Op::out_t* __restrict__ out) {
    using acc_t = typename Op::acc_t;
    using V = typename ColVec<VEC, Op>::type;
    const unsigned int lane = threadIdx.x;
    const size_t j = blockIdx.x % ncb;
    const size_t k = blockIdx.x / ncb;
    const unsigned int g = lane % ngroups;
    const size_t rpl = kWave / ngroups;  // rows per load
    const size_t q = lane / ngroups;
    const size_t c0 = (j * ngroups + g) * VEC;
    const size_t r0 = k * rchunk;
    const size_t r1 = r0 + rchunk < rows ? r0 + rchunk : rows;
    acc_t acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = Op::identity();
    if (c0 < cols) {
        const size_t step = ld / VEC * rpl;  // in V units, between a lane's rows
        size_t r = r0 + q;
        const V* __restrict__ p = reinterpret_cast<const V*>(x + r * ld + c0);
        for (; r + (UNROLL - 1) * rpl < r1; r += UNROLL * rpl, p += UNROLL * step) {
            V v[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) v[u] = load_vec<NT>(p + u * step);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) col_fold<Op, VEC>(acc, v[u]);
        }
        for (; r < r1; r += rpl, p += step) col_fold<Op, VEC>(acc, load_vec<NT>(p));
    }
    // Packed rows: lane g collects lanes g + ngroups, g + 2*ngroups, ... in a
    // fixed order (all lanes take part in the shuffles).
    for (unsigned int off = kWave / 2; off >= ngroups; off >>= 1) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] = Op::combine(acc[i], __shfl_down(acc[i], off, kWave));
    }
    if (q == 0 && c0 < cols) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            if (out != nullptr)
                out[c0 + i] = Op::finish(acc[i]);
            else
                partials[k * cols + c0 + i] = acc[i];
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

bool cols_policy_supported(const ColsPolicy& p) {
    const bool u = p.unroll == 1 || p.unroll == 2 || p.unroll == 4 || p.unroll == 8 || p.unroll == 16;
    return u && (p.nontemporal == 0 || p.nontemporal == 1) && p.target_waves >= 1 &&
           (p.vec == 0 || p.vec == 1 || p.vec == 4);
}

template <class Op, int VEC, int UNROLL>
static hipError_t cols_vu(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                          typename Op::out_t* out, const ColsLaunch& L, bool nt, hipStream_t stream) {
    auto* partials = static_cast<typename Op::acc_t*>(L.partials);
    const size_t rchunk = (rows + L.nchunks - 1) / L.nchunks;
    const dim3 grid((unsigned int)(L.ncb * L.nchunks));
    typename Op::out_t* direct = L.nchunks == 1 ? out : nullptr;
    if (nt)
        hipLaunchKernelGGL((cols_partial_kernel<Op, VEC, UNROLL, true>), grid, dim3(kWave), 0, stream, x, rows,
                           cols, ld, rchunk, L.ncb, L.ngroups, partials, direct);
    else
        hipLaunchKernelGGL((cols_partial_kernel<Op, VEC, UNROLL, false>), grid, dim3(kWave), 0, stream, x, rows,
                           cols, ld, rchunk, L.ncb, L.ngroups, partials, direct);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || L.nchunks == 1) return e;
    const size_t W = kColsCombineBlock / kWave;
    hipLaunchKernelGGL((cols_combine_kernel<Op>), dim3((unsigned int)((cols + W - 1) / W)),
                       dim3(kColsCombineBlock), 0, stream, partials, L.nchunks, cols, out);
    return hipGetLastError();
}

template <class Op, int VEC>
static hipError_t cols_v(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                         typename Op::out_t* out, const ColsLaunch& L, const ColsPolicy& p, hipStream_t stream) {
    const bool nt = p.nontemporal != 0;
    switch (p.unroll) {
        case 1: return cols_vu<Op, VEC, 1>(x, rows, cols, ld, out, L, nt, stream);
        case 2: return cols_vu<Op, VEC, 2>(x, rows, cols, ld, out, L, nt, stream);
        case 4: return cols_vu<Op, VEC, 4>(x, rows, cols, ld, out, L, nt, stream);
        case 8: return cols_vu<Op, VEC, 8>(x, rows, cols, ld, out, L, nt, stream);
        case 16: return cols_vu<Op, VEC, 16>(x, rows, cols, ld, out, L, nt, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class Op>
static hipError_t cols_op(const typename Op::elem_t* x, size_t rows, size_t cols, size_t ld,
                          typename Op::out_t* out, const ColsLaunch& L, const ColsPolicy& p, hipStream_t stream) {
    if (L.vec == 4) return cols_v<Op, 4>(x, rows, cols, ld, out, L, p, stream);
    return cols_v<Op, 1>(x, rows, cols, ld, out, L, p, stream);
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
