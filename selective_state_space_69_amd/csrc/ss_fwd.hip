// Forward selective scan, host side: the launch plan (row packing, chunk
// summaries and carries, output pass) around the 64-channel kernels
// (ss_fwd_kernels.hpp, instantiated in ss_fwd_<in>_<out>.hip) and the
// kernels with the states over the lanes (ss_fwd_hw.hpp: 32 channels in
// ss_fwd_hw.hip, 16 in ss_fwd_hw1.hip).
#include "ss_fwd_common.hpp"

namespace ss {
namespace {

// B and C rows padded to 16 entries per (b, t) (zero past N), in the input type:
// the layout the scan kernels read.  Needed when N < 16, and when the rows sit
// S > N elements apart (column ranges of a wider projection output).
template <typename In>
__global__ __launch_bounds__(256) void pack_rows_kernel(const In* __restrict__ Bm,
                                                        const In* __restrict__ Cm,
                                                        In* __restrict__ Bp, In* __restrict__ Cp,
                                                        int64_t rows, int N, int64_t S) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= rows * kMaxState) return;
  const int64_t r = gid / kMaxState;
  const int n = int(gid % kMaxState);
  Bp[gid] = n < N ? Bm[r * S + n] : In(0);
  Cp[gid] = n < N ? Cm[r * S + n] : In(0);
}

hipError_t dispatch(const ss_desc_t& d, const FwdParams& p, int nsplit, bool summary,
                    int64_t nblocks, hipStream_t st) {
  const bool has_z = p.z != nullptr, sp = d.delta_softplus != 0;
  if (d.in_dtype == SS_BF16) {
    if (summary || d.out_dtype == SS_F32)
      return fwd_dispatch_bf16_f32(p, d.disc, nsplit, has_z, sp, summary, nblocks, st);
    return fwd_dispatch_bf16_bf16(p, d.disc, nsplit, has_z, sp, false, nblocks, st);
  }
  if (summary || d.out_dtype == SS_F32)
    return fwd_dispatch_f32_f32(p, d.disc, nsplit, has_z, sp, summary, nblocks, st);
  return fwd_dispatch_f32_bf16(p, d.disc, nsplit, has_z, sp, false, nblocks, st);
}

}  // namespace

namespace {

FwdParams make_params(const ss_desc_t& d, const TimePlan& tp, const FwdArgs& a) {
  FwdParams p{};
  p.u = a.u; p.delta = a.delta; p.A = a.A;
  p.Dskip = a.Dskip; p.bias = a.bias; p.z = a.z; p.h0 = a.h0;
  p.y = a.y; p.h_last = a.h_last; p.hend = a.hend; p.dsum = a.dsum;
  p.Brow = a.Brow; p.Crow = a.Crow;
  p.L = d.seqlen; p.D = d.dim; p.N = int32_t(d.dstate);
  p.chunk_len = tp.chunk_len;
  p.nchunks = int32_t(tp.nchunks);
  p.rev = a.rev ? 1 : 0;
  p.acc = a.acc ? 1 : 0;
  const int64_t width = tp.nsplit == kHalfWaveSplit   ? 32
                        : tp.nsplit == kOneStateSplit ? 16
                                                      : kWave;   // channels per workgroup
  p.ndblk = int32_t((d.dim + width - 1) / width);
  return p;
}

}  // namespace

int launch_pack_rows(const ss_desc_t& d, const void* Bm, const void* Cm, void* Brow, void* Crow,
                     void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t rows = d.batch * d.seqlen;
  const unsigned nb = unsigned((rows * kMaxState + 255) / 256);
  const int64_t S = d.bc_stride != 0 ? d.bc_stride : d.dstate;
  if (d.in_dtype == SS_BF16)
    hipLaunchKernelGGL(pack_rows_kernel<uint16_t>, dim3(nb), dim3(256), 0, st,
                       static_cast<const uint16_t*>(Bm), static_cast<const uint16_t*>(Cm),
                       static_cast<uint16_t*>(Brow), static_cast<uint16_t*>(Crow), rows,
                       int(d.dstate), S);
  else
    hipLaunchKernelGGL(pack_rows_kernel<float>, dim3(nb), dim3(256), 0, st,
                       static_cast<const float*>(Bm), static_cast<const float*>(Cm),
                       static_cast<float*>(Brow), static_cast<float*>(Crow), rows, int(d.dstate),
                       S);
  return int(hipGetLastError());
}

int launch_fwd_carries(const ss_desc_t& d, const TimePlan& tp, const FwdArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  FwdParams p = make_params(d, tp, a);
  const int64_t cols = d.batch * p.ndblk;
  p.grid_chunks = p.nchunks - 1;   // the last chunk's summary is never needed
  hipError_t e = tp.nsplit == kHalfWaveSplit   ? launch_fwd_hw(d, p, true, cols * p.grid_chunks, st)
                 : tp.nsplit == kOneStateSplit ? launch_fwd_hw1(d, p, true, cols * p.grid_chunks, st)
                                               : dispatch(d, p, tp.nsplit, true, cols * p.grid_chunks, st);
  if (e != hipSuccess) return int(e);
  return launch_chunk_carry(a.hend, a.dsum, a.A, a.h0, d.batch, d.dim, int(d.dstate), p.nchunks,
                            false, stream);
}

int launch_fwd(const ss_desc_t& d, const FwdPlan& plan, const FwdArgs& args, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  FwdArgs a = args;
  if (plan.packed_rows) {
    const int e = launch_pack_rows(d, a.Bm, a.Cm, a.Brow, a.Crow, stream);
    if (e != 0) return e;
  } else {
    a.Brow = const_cast<void*>(a.Bm);
    a.Crow = const_cast<void*>(a.Cm);
  }
  if (plan.tp.nchunks > 1) {
    const int e = launch_fwd_carries(d, plan.tp, a, stream);
    if (e != 0) return e;
  }
  FwdParams p = make_params(d, plan.tp, a);
  p.grid_chunks = p.nchunks;
  const int64_t cols = d.batch * p.ndblk;
  if (plan.tp.nsplit == kHalfWaveSplit) return int(launch_fwd_hw(d, p, false, cols * p.grid_chunks, st));
  if (plan.tp.nsplit == kOneStateSplit) return int(launch_fwd_hw1(d, p, false, cols * p.grid_chunks, st));
  return int(dispatch(d, p, plan.tp.nsplit, false, cols * p.grid_chunks, st));
}

}  // namespace ss

