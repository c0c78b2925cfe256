// flat_fused.hip -- the one-pass sum / max / sum-of-magnitudes, and the xor
// read probe.
#include "flat_reduce.hpp"
#include "ops_ext.hpp"

namespace libred {

hipError_t launch_sum_max_f32(const float* x, size_t n, float* out3, int grid, const FlatPolicy& p,
                              const Workspace& ws, hipStream_t stream) {
    return launch_op<SumMaxAbsF32>(x, n, reinterpret_cast<SumMaxAbsOut*>(out3), grid, p, ws, stream);
}

hipError_t launch_xor_u32(const uint32_t* x, size_t n, uint32_t* out, int grid, const FlatPolicy& p,
                          const Workspace& ws, hipStream_t stream) {
    return launch_op<XorU32>(x, n, out, grid, p, ws, stream);
}

}  // namespace libred
