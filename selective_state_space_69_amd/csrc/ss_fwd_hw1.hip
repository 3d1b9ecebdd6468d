// Forward selective scan for gfx950, 16-channel workgroups: one state per
// lane, sixteen owner slots and 16-step blocks (the layout and the arithmetic
// are in ss_fwd_hw.hpp).  For problems too narrow for two states per lane to
// give the SIMDs several waves: at B = 8, D = 1536 it makes 768 workgroups,
// three per compute unit and three waves per SIMD, in one pass over time.
#include "ss_fwd_hw.hpp"

namespace ss {
namespace {

template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY, bool REV>
// three waves per SIMD: three workgroups per compute unit (43 KB of LDS each)
__global__ __launch_bounds__(kWave * HwLayout<1>::kWaves, 3) void fwd_hw1_kernel(FwdParams p) {
  fwd_hw_body<1, In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, REV>(p);
}

template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY>
hipError_t launch_one(const FwdParams& p, int64_t nblocks, hipStream_t st) {
  if (p.rev)
    hipLaunchKernelGGL((fwd_hw1_kernel<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, true>),
                       dim3(unsigned(nblocks)), dim3(kWave * HwLayout<1>::kWaves), 0, st, p);
  else
    hipLaunchKernelGGL((fwd_hw1_kernel<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, false>),
                       dim3(unsigned(nblocks)), dim3(kWave * HwLayout<1>::kWaves), 0, st, p);
  return hipGetLastError();
}

#include "ss_fwd_hw_dispatch.inc"

}  // namespace

hipError_t launch_fwd_hw1(const ss_desc_t& d, const FwdParams& p, bool summary, int64_t nblocks,
                          hipStream_t st) {
  return dispatch_types(d, p, summary, nblocks, st);
}

}  // namespace ss
