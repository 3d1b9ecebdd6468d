// Single-token recurrent step (inference mode: "A Visual Guide to Mamba"
// summary, recurrent representation; the state is O(1) per token).  Four lanes
// per (b, d), each with four states n = 4q .. 4q+3: read h[b, d, n], apply one
// step of the same discretised recurrence as the forward scan, write h back;
// the four partial sums of C h meet through two quad butterflies and the first
// lane of the quad writes y.  Bound by the state traffic, 2 * 4 * N bytes per
// (b, d): with N = 16 every access is a 16-byte vector and a quad reads or
// writes 64 contiguous bytes.
#include "ss_device.hpp"

namespace ss {
namespace {

struct StepParams {
  float* h;
  const void* u;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  const float* bias;
  const void* z;
  void* y;
  int64_t B, D;
  int64_t S;   // elements from one batch row of Bm, Cm to the next
  int32_t N, disc, softplus;
};

constexpr int kQuad = 4;   // lanes per (b, d)

template <typename In, typename Out, bool N16>
__global__ __launch_bounds__(256) void step_kernel(StepParams p) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t ch = gid / kQuad;            // (b, d)
  const int q = int(gid % kQuad);
  const bool live = ch < p.B * p.D;
  const int64_t chc = live ? ch : p.B * p.D - 1;   // idle lanes still join the butterflies
  const int64_t b = chc / p.D, d = chc % p.D;
  const int N = p.N;
  const In* u = static_cast<const In*>(p.u);
  const In* dl_in = static_cast<const In*>(p.delta);

  const float uf = to_f32(u[chc]);
  const float x2 = (to_f32(dl_in[chc]) + (p.bias ? p.bias[d] : 0.0f)) * kLog2e;
  const float dl = p.softplus ? softplus_log2(x2) : x2;   // dt * log2(e)
  const float dt = dl * kLn2;

  float hv[4], Av[4], Bv[4], Cv[4];
  const int n0 = q * 4;
  float* h = p.h + chc * N + n0;
  const float* Ap = p.A + d * N + n0;
  const In* Bp = static_cast<const In*>(p.Bm) + b * p.S + n0;
  const In* Cp = static_cast<const In*>(p.Cm) + b * p.S + n0;
  if constexpr (N16) {
    const float4 h4 = *reinterpret_cast<const float4*>(h), a4 = *reinterpret_cast<const float4*>(Ap);
    const float4 b4 = unpack4(load_raw4(Bp)), c4 = unpack4(load_raw4(Cp));
    hv[0] = h4.x; hv[1] = h4.y; hv[2] = h4.z; hv[3] = h4.w;
    Av[0] = a4.x; Av[1] = a4.y; Av[2] = a4.z; Av[3] = a4.w;
    Bv[0] = b4.x; Bv[1] = b4.y; Bv[2] = b4.z; Bv[3] = b4.w;
    Cv[0] = c4.x; Cv[1] = c4.y; Cv[2] = c4.z; Cv[3] = c4.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = n0 + j < N;
      hv[j] = in ? h[j] : 0.0f;
      Av[j] = in ? Ap[j] : -1.0f;
      Bv[j] = in ? to_f32(Bp[j]) : 0.0f;
      Cv[j] = in ? to_f32(Cp[j]) : 0.0f;
    }
  }
  // the precise decay (the step is bound by the state's traffic, so its few
  // extra operations are free): h <- h + (E h + coef B u), E = A_bar - 1, so a
  // long decode loop does not compound the rounding of A_bar near 1
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = Av[j];
    float coef;
    const float e = precise_decay<true>(dl, a, a == 0.0f ? 0.0f : 1.0f / a, coef);
    if (p.disc == SS_EULER) coef = dt;
    hv[j] += __builtin_fmaf(e, hv[j], coef * (Bv[j] * uf));
    acc = __builtin_fmaf(Cv[j], hv[j], acc);
  }
  // sum over the quad (lanes 4k .. 4k+3 hold one (b, d))
  acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0xb1, 0xf, 0xf, false));
  acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0x4e, 0xf, 0xf, false));
  if (!live) return;
  if constexpr (N16) {
    *reinterpret_cast<float4*>(h) = make_float4(hv[0], hv[1], hv[2], hv[3]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (n0 + j < N) h[j] = hv[j];
  }
  if (q != 0) return;
  float yv = __builtin_fmaf(p.Dskip ? p.Dskip[d] : 0.0f, uf, acc);
  if (p.z) yv *= silu(to_f32(static_cast<const In*>(p.z)[chc]));
  store_out<Out>(static_cast<Out*>(p.y) + chc, yv);
}

}  // namespace

// 16-byte vector loads only for dense 16-state rows (16-byte aligned by the
// entry point's checks); rows with a stride are read element by element.
template <typename In, typename Out>
void launch_typed(const StepParams& p, bool vec, dim3 grid, dim3 block, hipStream_t st) {
  if (vec) hipLaunchKernelGGL((step_kernel<In, Out, true>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((step_kernel<In, Out, false>), grid, block, 0, st, p);
}

int launch_step(const ss_desc_t& d, const StepArgs& a, void* stream) {
  StepParams p{a.h, a.u, a.delta, a.A, a.Bm, a.Cm, a.Dskip, a.bias, a.z, a.y,
               d.batch, d.dim, d.bc_stride != 0 ? d.bc_stride : d.dstate,
               int32_t(d.dstate), d.disc, d.delta_softplus};
  const int64_t total = d.batch * d.dim * kQuad;
  const dim3 grid(unsigned((total + 255) / 256)), block(256);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool vec = d.dstate == kMaxState && d.bc_stride == 0;
  if (d.in_dtype == SS_BF16) {
    if (d.out_dtype == SS_F32) launch_typed<uint16_t, float>(p, vec, grid, block, st);
    else launch_typed<uint16_t, uint16_t>(p, vec, grid, block, st);
  } else {
    if (d.out_dtype == SS_F32) launch_typed<float, float>(p, vec, grid, block, st);
    else launch_typed<float, uint16_t>(p, vec, grid, block, st);
  }
  return int(hipGetLastError());
}

}  // namespace ss
