// Backward pass (placeholder until the recompute kernels land).
#include "attn_launch.h"
namespace attn {
hipError_t launch_bwd(const BwdArgs&) { return hipErrorNotSupported; }
}  // namespace attn
