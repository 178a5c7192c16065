// Backward pass (placeholder until the kernels land).
#include "fa_common.h"
#include "fa_launch.h"

namespace fa355 {
hipError_t launch_bwd(const BwdArgs&) { return hipErrorNotSupported; }
}  // namespace fa355
