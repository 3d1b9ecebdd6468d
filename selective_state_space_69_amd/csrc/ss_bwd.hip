// Backward selective scan (placeholder until the recompute kernels land).
#include "ss_device.hpp"

namespace ss {
int launch_bwd(const ss_desc_t&, const BwdPlan&, const BwdArgs&, void*) {
  return int(hipErrorNotSupported);
}
}  // namespace ss
