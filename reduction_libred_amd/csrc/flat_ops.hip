// flat_ops.hip -- the int32 -> int64 sum, the float32 max and min.
#include "flat_reduce.hpp"
#include "ops_ext.hpp"

namespace libred {

hipError_t launch_sum_i32_i64(const int32_t* x, size_t n, int64_t* out, int grid,
                              const FlatPolicy& p, const Workspace& ws, hipStream_t stream) {
    return launch_op<SumI32>(x, n, out, grid, p, ws, stream);
}

hipError_t launch_max_f32(const float* x, size_t n, float* out, int grid, const FlatPolicy& p,
                          const Workspace& ws, hipStream_t stream) {
    return launch_op<MaxF32>(x, n, out, grid, p, ws, stream);
}

hipError_t launch_min_f32(const float* x, size_t n, float* out, int grid, const FlatPolicy& p,
                          const Workspace& ws, hipStream_t stream) {
    return launch_op<MinF32>(x, n, out, grid, p, ws, stream);
}

}  // namespace libred
