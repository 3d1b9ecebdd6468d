// Instantiation of the 64-channel forward kernels for f32 input, f32 output
// (one translation unit per element-type pair, so the build compiles them in
// parallel).
#include "ss_fwd_kernels.hpp"

namespace ss {

hipError_t fwd_dispatch_f32_f32(const FwdParams& p, int disc, int nsplit, bool has_z, bool softplus,
                       bool summary, int64_t nblocks, hipStream_t st) {
  return dispatch_disc<float, float>(p, disc, nsplit, has_z, softplus, summary, nblocks, st);
}

}  // namespace ss
