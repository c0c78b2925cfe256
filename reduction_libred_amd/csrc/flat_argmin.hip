// flat_argmin.hip -- index of the min (lowest index of equal minima; NaN
// never wins).
#include "flat_reduce.hpp"
#include "ops_ext.hpp"

namespace libred {

hipError_t launch_argmin_f32(const float* x, size_t n, int64_t* out, int grid, const FlatPolicy& p,
                             const Workspace& ws, hipStream_t stream) {
    return launch_op<ArgMinF32>(x, n, out, grid, p, ws, stream);
}

}  // namespace libred
