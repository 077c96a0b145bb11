// Backward with recomputation (bf16): placeholder until the kernels land.
#include "common.hpp"
#include "launch.hpp"

namespace fattn {
hipError_t launch_bwd_bf16(const BwdArgs&) { return hipErrorNotSupported; }
}  // namespace fattn
