// rows_sum.hip -- the per-row sum: the row kernels of rows_reduce.hpp (and
// the register kernel of rows_narrow.hip) for the float32 sum, accumulated
// in float64 and rounded once per row; also the check of a row policy.
#include "rows_reduce.hpp"

namespace libred {

bool rows_policy_supported(const RowsPolicy& p) {
    const bool b = p.block == 64 || p.block == 128 || p.block == 256 || p.block == 512;
    const bool u = p.unroll == 1 || p.unroll == 2 || p.unroll == 4 || p.unroll == 8 || p.unroll == 16;
    return b && u && (p.nontemporal == 0 || p.nontemporal == 1) && p.max_blocks >= 1 && p.split >= 0 &&
           p.split <= 2 && (p.prefetch == 0 || p.prefetch == 1) && p.cover >= 0 && p.cover <= 2 &&
           p.short_rows >= 0 && p.short_rows <= 17 && p.defer >= 0 && p.defer <= 2 && p.lines >= 0 &&
           p.lines <= 2 && p.xcd >= 0 && p.xcd <= 4096 &&
           p.max_fold >= 0 && p.max_fold <= 2;
}

hipError_t launch_rows_sum_f32(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                               const RowsLaunch& L, const RowsPolicy& p, hipStream_t stream) {
    if (L.narrow)
        return launch_rows_narrow(0, x, rows, cols, out, L.grid, p.nontemporal != 0, L.narrow == 2, stream);
    return rows_op<SumF32>(x, rows, cols, ld, out, L, p, stream);
}

}  // namespace libred
