// flat_argmax.hip -- index of the max (lowest index of equal maxima; NaN
// never wins).
#include "flat_reduce.hpp"
#include "ops_ext.hpp"

namespace libred {

hipError_t launch_argmax_f32(const float* x, size_t n, int64_t* out, int grid, const FlatPolicy& p,
                             const Workspace& ws, hipStream_t stream) {
    return launch_op<ArgMaxF32>(x, n, out, grid, p, ws, stream);
}

}  // namespace libred
