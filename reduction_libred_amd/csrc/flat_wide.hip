// flat_wide.hip -- sums of bfloat16 and IEEE half inputs (eight per 16-byte
// load, widened exactly, accumulated in float64, rounded once to float32) and
// of float64 inputs (two per load).
#include "flat_reduce.hpp"
#include "ops_ext.hpp"

namespace libred {

hipError_t launch_sum_bf16(const uint16_t* x, size_t n, float* out, int grid, const FlatPolicy& p,
                           const Workspace& ws, hipStream_t stream) {
    return launch_op<SumBF16>(x, n, out, grid, p, ws, stream);
}

hipError_t launch_sum_f16(const uint16_t* x, size_t n, float* out, int grid, const FlatPolicy& p,
                          const Workspace& ws, hipStream_t stream) {
    return launch_op<SumF16>(x, n, out, grid, p, ws, stream);
}

hipError_t launch_sum_f64(const double* x, size_t n, double* out, int grid, const FlatPolicy& p,
                          const Workspace& ws, hipStream_t stream) {
    return launch_op<SumF64>(x, n, out, grid, p, ws, stream);
}

}  // namespace libred
