// rows_max.hip -- the per-row maximum: the row kernels of rows_reduce.hpp
// (and the register kernel of rows_narrow.hip) for the float32 max under the
// strictly-greater rule.
#include "rows_reduce.hpp"

namespace libred {

hipError_t launch_rows_max_f32(const float* x, size_t rows, size_t cols, size_t ld, float* out,
                               const RowsLaunch& L, const RowsPolicy& p, hipStream_t stream) {
    if (L.narrow)
        return launch_rows_narrow(1, x, rows, cols, out, L.grid, p.nontemporal != 0, L.narrow == 2, stream);
    return rows_op<MaxF32>(x, rows, cols, ld, out, L, p, stream);
}

}  // namespace libred
