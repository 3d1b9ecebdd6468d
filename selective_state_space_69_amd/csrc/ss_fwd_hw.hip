// Forward selective scan for gfx950, 32-channel workgroups: two states per
// lane, eight owner slots and 8-step blocks (the layout and the arithmetic are
// in ss_fwd_hw.hpp).  On the Mamba-2.8B shape (B = 8, D = 5120) it makes 1280
// workgroups: five per compute unit, five waves per SIMD.
#include "ss_fwd_hw.hpp"

namespace ss {
namespace {

template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY, bool REV>
// five waves per SIMD: five workgroups per compute unit
__global__ __launch_bounds__(kWave * HwLayout<2>::kWaves, 5) void fwd_hw_kernel(FwdParams p) {
  fwd_hw_body<2, In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, REV>(p);
}

template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY>
hipError_t launch_one(const FwdParams& p, int64_t nblocks, hipStream_t st) {
  if (p.rev)
    hipLaunchKernelGGL((fwd_hw_kernel<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, true>),
                       dim3(unsigned(nblocks)), dim3(kWave * HwLayout<2>::kWaves), 0, st, p);
  else
    hipLaunchKernelGGL((fwd_hw_kernel<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, false>),
                       dim3(unsigned(nblocks)), dim3(kWave * HwLayout<2>::kWaves), 0, st, p);
  return hipGetLastError();
}

#include "ss_fwd_hw_dispatch.inc"

}  // namespace

hipError_t launch_fwd_hw(const ss_desc_t& d, const FwdParams& p, bool summary, int64_t nblocks,
                         hipStream_t st) {
  return dispatch_types(d, p, summary, nblocks, st);
}

}  // namespace ss
