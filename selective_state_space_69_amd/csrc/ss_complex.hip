// Forward selective scan with complex diagonal A (gfx950, wave64).
//
// The pages name a complex diagonal initialisation of A (S4D-Lin) beside the
// real one ("A Survey of Mamba" summary, HiPPO-based memory initialisation) and
// compare complex with real decay ("Mamba: S4 epic upgrade", ablation on A).
// Per channel (b, d) and complex state n, with the real scan's step size:
//     abar  = exp(dt a)                          a = A[d, n] complex
//     bcoef = (abar - 1) / a   (exact ZOH, a series near dt a = 0; dt in Euler mode)
//     h_n   = abar h_n + bcoef B_n u             B_n, C_n complex (per b, t)
//     y     = 2 Re(sum_n C_n h_n) + D u          each state stands for itself and
//                                                its conjugate
//     out   = y * silu(z)
//
// Layout: a workgroup of 4 waves covers 32 channels; a wave covers 8 channels
// with 8 lanes each, and lane q of a channel holds the complex states 2q and
// 2q + 1 (N <= 16).  Time runs in blocks of 8 steps, and lane q also owns step
// q of every block: it alone loads that step's u, delta and z, computes its
// softplus and gate, publishes (dt, u) through LDS for the other lanes, and
// stores its y.  The 8 per-step partial sums of C h a lane builds in a block
// are reduce-scattered over the channel's 8 lanes (DPP half-row mirror, then
// quad swaps), so lane q ends with the sum for its own step.  Each state and
// step needs one v_exp_f32 (the modulus) and one v_sin_f32 / v_cos_f32 pair
// (the phase, in revolutions, reduced to [0, 1) first).  B and C rows of a
// block are staged in LDS as fp32 (re, im) pairs; the inputs of the next block
// are fetched while the current one runs.  No time chunks: one workgroup walks
// the whole sequence of its channels.  On the Mamba-2.8B width (B = 8,
// D = 5120) the grid is 1280 workgroups: five per compute unit, five waves per
// SIMD.
#include <type_traits>

#include "ss_device.hpp"

namespace ss {
namespace {

constexpr int kCBlk = 8;                 // steps per block
constexpr int kSPL = 2;                  // complex states per lane
constexpr int kLPC = 8;                  // lanes per channel (= steps per block)
constexpr int kChPerWave = kWave / kLPC;
constexpr int kCWaves = 4;
constexpr int kChPerGroup = kChPerWave * kCWaves;
constexpr int kMaxC = kSPL * kLPC;       // 16 complex states
constexpr float kInv2Pi = 0.15915494309189535f;
static_assert(kLPC == kCBlk, "lane q of a channel owns step q of a block");

struct CParams {
  const void* u;
  const void* delta;
  const float* A;       // (D, N, 2)
  const void* Bm;       // (B, L, N, 2)
  const void* Cm;       // (B, L, N, 2)
  const float* Dskip;
  const float* bias;
  const void* z;
  const float* h0;      // (B, D, N, 2)
  void* y;
  float* h_last;        // (B, D, N, 2)
  int64_t L, D;
  int32_t N, ndblk;
};

// x from the lane DPP control CTRL selects (every control used here has a
// source in range for every lane)
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
// one stage of a reduce-scatter: the lane keeps the half of its values its
// id bit selects (upper: hi) and adds the partner's copy of that half
template <int CTRL>
__device__ __forceinline__ float dpp_pair(float lo, float hi, bool upper) {
  return (upper ? hi : lo) + dpp<CTRL>(upper ? lo : hi);
}
constexpr int kDppHalfMirror = 0x141;   // lane l <-> 7 - l inside each group of 8
constexpr int kDppQuadXor2 = 0x4e;      // quad_perm [2, 3, 0, 1]
constexpr int kDppQuadXor1 = 0xb1;      // quad_perm [1, 0, 3, 2]

// 8 values per lane -> lane q of each group of 8 holds the group's sum of
// value q.  Stage partners: l <-> 7 - l (keep by bit 2), then l ^ 2, l ^ 1.
__device__ __forceinline__ float reduce_scatter8(const float (&v)[8], int q) {
  float c[4], e[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = dpp_pair<kDppHalfMirror>(v[i], v[i + 4], (q & 4) != 0);
#pragma unroll
  for (int i = 0; i < 2; ++i) e[i] = dpp_pair<kDppQuadXor2>(c[i], c[i + 2], (q & 2) != 0);
  return dpp_pair<kDppQuadXor1>(e[0], e[1], (q & 1) != 0);
}

template <typename In>
struct Pair;
template <>
struct Pair<float> {
  using raw = uint2;
  static __device__ __forceinline__ raw load(const float* p) {
    return *reinterpret_cast<const uint2*>(p);
  }
  static __device__ __forceinline__ float2 f32(raw r) {
    return make_float2(__uint_as_float(r.x), __uint_as_float(r.y));
  }
};
template <>
struct Pair<uint16_t> {
  using raw = uint32_t;
  static __device__ __forceinline__ raw load(const uint16_t* p) {
    return *reinterpret_cast<const uint32_t*>(p);
  }
  static __device__ __forceinline__ float2 f32(raw r) {
    return make_float2(__uint_as_float(r << 16), __uint_as_float(r & 0xffff0000u));
  }
};

template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS>
// five waves per SIMD (five workgroups per CU at the 2.8B width): at most 96 VGPRs
__global__ __launch_bounds__(kWave * kCWaves, 5) void fwd_complex_kernel(CParams p) {
  const int tid = int(threadIdx.x);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int q = lane % kLPC, cl = lane / kLPC;
  const int chan = wave * kChPerWave + cl;                 // channel within the group
  const int dblk = int(blockIdx.x % unsigned(p.ndblk));
  const int64_t b = int64_t(blockIdx.x / unsigned(p.ndblk));
  const int64_t d = int64_t(dblk) * kChPerGroup + chan;
  const bool active = d < p.D;
  const int64_t dc = active ? d : p.D - 1;
  const int N = p.N;
  const int64_t L = p.L, D = p.D;

  // per-state constants: modulus rate, phase rate (revolutions per dt log2 e),
  // a itself and 1 / a (0 when a == 0)
  float ar[kSPL], aw[kSPL], ai[kSPL], iar[kSPL], iai[kSPL], hr[kSPL], hi[kSPL];
  bool weak = false;
#pragma unroll
  for (int j = 0; j < kSPL; ++j) {
    const int n = kSPL * q + j;
    float re = -1.0f, im = 0.0f;   // unused states: inert (their B and C rows are 0)
    if (n < N) {
      re = p.A[(dc * N + n) * 2];
      im = p.A[(dc * N + n) * 2 + 1];
    }
    ar[j] = re;
    ai[j] = im;
    aw[j] = im * (kLn2 * kInv2Pi);
    const float m2 = re * re + im * im;
    weak |= m2 < kWeakA * kWeakA;
    iar[j] = m2 == 0.0f ? 0.0f : re / m2;
    iai[j] = m2 == 0.0f ? 0.0f : -im / m2;
    hr[j] = 0.0f;
    hi[j] = 0.0f;
    if (p.h0 && n < N) {
      hr[j] = p.h0[((b * D + dc) * N + n) * 2];
      hi[j] = p.h0[((b * D + dc) * N + n) * 2 + 1];
    }
  }
  // exact ZOH: the guarded coefficient where some state of the wave has |a| < kWeakA
  const bool guard = __any(weak);
  const float Dd = p.Dskip ? p.Dskip[dc] : 0.0f;
  const float bias2 = (p.bias ? p.bias[dc] : 0.0f) * kLog2e;

  // B and C rows of a block: [buffer][step][B | C][state] as (re, im); the
  // owned steps' (dt log2 e, u): [buffer][step][channel]
  __shared__ __align__(16) float2 rows[2][kCBlk][2][kMaxC];
  __shared__ __align__(16) float2 act[2][kCBlk][kChPerGroup];
  // staging thread: step sk, matrix sw (0 = B, 1 = C), state sn
  const int sk = tid / (2 * kMaxC), sw = (tid / kMaxC) % 2, sn = tid % kMaxC;
  const In* rbase = static_cast<const In*>(sw ? p.Cm : p.Bm);
  const In* ub = static_cast<const In*>(p.u) + b * L * D + dc;
  const In* db = static_cast<const In*>(p.delta) + b * L * D + dc;
  const In* zb = HAS_Z ? static_cast<const In*>(p.z) + b * L * D + dc : nullptr;
  Out* yb = static_cast<Out*>(p.y) + b * L * D + dc;

  typename Pair<In>::raw rw[2];
  In ur[2], dr[2], zr[2];        // the owned step's inputs, by block parity
  float u_own[2], g_own[2];      // its u and gate
  // fetch block t0 into register set S (steps past the end read step L - 1;
  // their step size and input are forced to 0 below)
  auto fetch = [&](auto S_, int64_t t0) {
    constexpr int S = decltype(S_)::value;
    const int64_t t = t0 + q < L ? t0 + q : L - 1;
    ur[S] = ub[t * D];
    dr[S] = db[t * D];
    if (HAS_Z) zr[S] = zb[t * D];
    const int64_t tr = t0 + sk < L ? t0 + sk : L - 1;
    rw[S] = Pair<In>::load(rbase + ((b * L + tr) * N + (sn < N ? sn : 0)) * 2);
  };
  // the block's rows and this lane's owned-step values into buffer S
  auto stage = [&](auto S_, int64_t t0) {
    constexpr int S = decltype(S_)::value;
    float2 v = Pair<In>::f32(rw[S]);
    if (sn >= N || t0 + sk >= L) v = make_float2(0.0f, 0.0f);
    rows[S][sk][sw][sn] = v;
    const bool valid = t0 + q < L;
    const float x2 = __builtin_fmaf(to_f32(dr[S]), kLog2e, bias2);
    const float dl = valid ? (SOFTPLUS ? softplus_log2(x2) : x2) : 0.0f;   // dt log2 e
    u_own[S] = valid ? to_f32(ur[S]) : 0.0f;
    g_own[S] = HAS_Z ? silu(to_f32(zr[S])) : 1.0f;
    act[S][q][chan] = make_float2(dl, u_own[S]);
  };

  // G: the wave holds a slowly decaying state (guarded coefficient); a
  // template parameter so that the fast loop has no branch inside
  auto block = [&](auto S_, auto G_, int64_t t0) {
    constexpr int S = decltype(S_)::value;
    constexpr bool G = decltype(G_)::value;
    if (t0 + kCBlk < L) fetch(std::integral_constant<int, S ^ 1>{}, t0 + kCBlk);
    float part[kCBlk];                                     // Re sum_n C h, per step
#pragma unroll
    for (int k = 0; k < kCBlk; ++k) {
      const float2 du = act[S][k][chan];
      const float dl = du.x, uk = du.y;
      const float dt = dl * kLn2;
      const float4 bq = *reinterpret_cast<const float4*>(&rows[S][k][0][kSPL * q]);
      const float4 cq = *reinterpret_cast<const float4*>(&rows[S][k][1][kSPL * q]);
      const float Br[kSPL] = {bq.x, bq.z}, Bi[kSPL] = {bq.y, bq.w};
      const float Cr[kSPL] = {cq.x, cq.z}, Ci[kSPL] = {cq.y, cq.w};
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < kSPL; ++j) {
        const float e = hw_exp2(dl * ar[j]);                          // |abar|
        const float ph = __builtin_amdgcn_fractf(dl * aw[j]);         // arg abar / 2 pi
        const float abr = e * __builtin_amdgcn_cosf(ph);
        const float abi = e * __builtin_amdgcn_sinf(ph);
        float cr = dt, ci = 0.0f;                                     // Euler
        if (DISC == SS_ZOH) {
          const float mr = abr - 1.0f;                                // (abar - 1) / a
          cr = mr * iar[j] - abi * iai[j];
          ci = __builtin_fmaf(mr, iai[j], abi * iar[j]);
          if (G) {
            // a slowly decaying state in the wave: near x = dt a = 0 the
            // quotient cancels, so take dt (1 + x/2 + x^2/6 + x^3/24) there
            const float xr = dt * ar[j], xi = dt * ai[j];
            float pr = __builtin_fmaf(xr, 1.0f / 24.0f, 1.0f / 6.0f), pi = xi * (1.0f / 24.0f);
            float tr = __builtin_fmaf(pr, xr, __builtin_fmaf(-pi, xi, 0.5f));
            pi = __builtin_fmaf(pr, xi, pi * xr);
            pr = tr;
            tr = __builtin_fmaf(pr, xr, __builtin_fmaf(-pi, xi, 1.0f));
            pi = __builtin_fmaf(pr, xi, pi * xr);
            const bool ser =
                __builtin_unpredictable(__builtin_fmaf(xr, xr, xi * xi) < kZohSeries * kZohSeries);
            cr = ser ? dt * tr : cr;
            ci = ser ? dt * pi : ci;
          }
        }
        const float bur = Br[j] * uk, bui = Bi[j] * uk;
        const float qr = cr * bur - ci * bui, qi = __builtin_fmaf(cr, bui, ci * bur);
        const float nr = __builtin_fmaf(abr, hr[j], __builtin_fmaf(-abi, hi[j], qr));
        const float ni = __builtin_fmaf(abr, hi[j], __builtin_fmaf(abi, hr[j], qi));
        hr[j] = nr;
        hi[j] = ni;
        acc = __builtin_fmaf(Cr[j], nr, __builtin_fmaf(-Ci[j], ni, acc));
      }
      part[k] = acc;
    }
    // y of the owned step: the channel's sum for step q, skip, gate
    const float sum = reduce_scatter8(part, q);
    float yv = __builtin_fmaf(2.0f, sum, Dd * u_own[S]);
    if (HAS_Z) yv *= g_own[S];
    if (t0 + q < L && active) store_out<Out>(yb + (t0 + q) * D, yv);
    // the next block's rows and owned-step values into the other buffers (last
    // read by the previous block, which every wave finished before the
    // barrier that ended it)
    if (t0 + kCBlk < L) stage(std::integral_constant<int, S ^ 1>{}, t0 + kCBlk);
    __syncthreads();
  };

  fetch(std::integral_constant<int, 0>{}, 0);
  stage(std::integral_constant<int, 0>{}, 0);
  __syncthreads();
  auto walk = [&](auto G_) {
    for (int64_t t0 = 0; t0 < L; t0 += 2 * kCBlk) {
      block(std::integral_constant<int, 0>{}, G_, t0);
      if (t0 + kCBlk < L) block(std::integral_constant<int, 1>{}, G_, t0 + kCBlk);
    }
  };
  if (DISC == SS_ZOH && guard) walk(std::true_type{});
  else walk(std::false_type{});
  if (p.h_last && active) {
#pragma unroll
    for (int j = 0; j < kSPL; ++j) {
      const int n = kSPL * q + j;
      if (n < N) {
        p.h_last[((b * D + d) * N + n) * 2] = hr[j];
        p.h_last[((b * D + d) * N + n) * 2 + 1] = hi[j];
      }
    }
  }
}

template <typename In, typename Out, int DISC>
hipError_t dispatch_flags(const CParams& p, bool has_z, bool sp, dim3 grid, hipStream_t st) {
  const dim3 block(kWave * kCWaves);
  if (has_z) {
    if (sp) hipLaunchKernelGGL((fwd_complex_kernel<In, Out, DISC, true, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((fwd_complex_kernel<In, Out, DISC, true, false>), grid, block, 0, st, p);
  } else {
    if (sp) hipLaunchKernelGGL((fwd_complex_kernel<In, Out, DISC, false, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((fwd_complex_kernel<In, Out, DISC, false, false>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

template <typename In, typename Out>
hipError_t dispatch_disc(const CParams& p, int disc, bool has_z, bool sp, dim3 grid,
                         hipStream_t st) {
  return disc == SS_ZOH ? dispatch_flags<In, Out, SS_ZOH>(p, has_z, sp, grid, st)
                        : dispatch_flags<In, Out, SS_EULER>(p, has_z, sp, grid, st);
}

// One recurrent step with complex A (decoding): h (B, D, N, 2) in place, y (B, D).
// kLPC lanes per (b, d), lane q holding states n = kSPL q + j as in the scan,
// with the same per-state arithmetic (modulus and phase of A_bar, the ZOH
// coefficient with its series near dt a = 0), so a step continues a scan.  The
// lanes' partial sums of Re C h meet by butterflies in a fixed order.
template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS>
__global__ __launch_bounds__(256) void step_complex_kernel(StepArgs a, int64_t BD, int64_t D, int N) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int q = int(gid % kLPC);
  const int64_t ch = gid / kLPC;
  const bool live = ch < BD;
  const int64_t chc = live ? ch : BD - 1;                 // idle lanes still join the butterflies
  const int64_t b = chc / D, d = chc % D;
  const float x2 = __builtin_fmaf(to_f32(static_cast<const In*>(a.delta)[chc]), kLog2e,
                                  (a.bias ? a.bias[d] : 0.0f) * kLog2e);
  const float dl = SOFTPLUS ? softplus_log2(x2) : x2;     // dt log2 e
  const float dt = dl * kLn2;
  const float uk = to_f32(static_cast<const In*>(a.u)[chc]);
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < kSPL; ++j) {
    const int n = kSPL * q + j;
    if (n >= N) continue;
    const float ar = a.A[(d * N + n) * 2], ai = a.A[(d * N + n) * 2 + 1];
    const float m2 = ar * ar + ai * ai;
    const float iar = m2 == 0.0f ? 0.0f : ar / m2, iai = m2 == 0.0f ? 0.0f : -ai / m2;
    const float e = hw_exp2(dl * ar);
    const float ph = __builtin_amdgcn_fractf(dl * (ai * (kLn2 * kInv2Pi)));
    const float abr = e * __builtin_amdgcn_cosf(ph), abi = e * __builtin_amdgcn_sinf(ph);
    float cr = dt, ci = 0.0f;                                     // Euler
    if (DISC == SS_ZOH) {
      const float mr = abr - 1.0f;
      cr = mr * iar - abi * iai;
      ci = __builtin_fmaf(mr, iai, abi * iar);
      const float xr = dt * ar, xi = dt * ai;
      float pr = __builtin_fmaf(xr, 1.0f / 24.0f, 1.0f / 6.0f), pi = xi * (1.0f / 24.0f);
      float tr = __builtin_fmaf(pr, xr, __builtin_fmaf(-pi, xi, 0.5f));
      pi = __builtin_fmaf(pr, xi, pi * xr);
      pr = tr;
      tr = __builtin_fmaf(pr, xr, __builtin_fmaf(-pi, xi, 1.0f));
      pi = __builtin_fmaf(pr, xi, pi * xr);
      const bool ser =
          __builtin_unpredictable(__builtin_fmaf(xr, xr, xi * xi) < kZohSeries * kZohSeries);
      cr = ser ? dt * tr : cr;
      ci = ser ? dt * pi : ci;
    }
    const typename Pair<In>::raw rb = Pair<In>::load(static_cast<const In*>(a.Bm) + (b * N + n) * 2);
    const typename Pair<In>::raw rc = Pair<In>::load(static_cast<const In*>(a.Cm) + (b * N + n) * 2);
    const float2 Bv = Pair<In>::f32(rb), Cv = Pair<In>::f32(rc);
    const float bur = Bv.x * uk, bui = Bv.y * uk;
    const float qr = cr * bur - ci * bui, qi = __builtin_fmaf(cr, bui, ci * bur);
    float* hp = a.h + (chc * N + n) * 2;
    const float hr = hp[0], hi = hp[1];
    const float nr = __builtin_fmaf(abr, hr, __builtin_fmaf(-abi, hi, qr));
    const float ni = __builtin_fmaf(abr, hi, __builtin_fmaf(abi, hr, qi));
    if (live) {
      hp[0] = nr;
      hp[1] = ni;
    }
    acc = __builtin_fmaf(Cv.x, nr, __builtin_fmaf(-Cv.y, ni, acc));
  }
#pragma unroll
  for (int m = 1; m < kLPC; m *= 2) acc += __shfl_xor(acc, m);
  if (q == 0 && live) {
    float y = __builtin_fmaf(a.Dskip ? a.Dskip[d] : 0.0f, uk, 2.0f * acc);   // conjugate pairs
    if (HAS_Z) y *= silu(to_f32(static_cast<const In*>(a.z)[chc]));
    store_out<Out>(static_cast<Out*>(a.y) + chc, y);
  }
}

template <typename In, typename Out, int DISC>
hipError_t step_flags(const StepArgs& s, int64_t BD, int64_t D, int N, bool has_z, bool sp,
                      hipStream_t st) {
  const dim3 grid(unsigned((BD * kLPC + 255) / 256)), block(256);
  if (has_z) {
    if (sp) hipLaunchKernelGGL((step_complex_kernel<In, Out, DISC, true, true>), grid, block, 0, st, s, BD, D, N);
    else hipLaunchKernelGGL((step_complex_kernel<In, Out, DISC, true, false>), grid, block, 0, st, s, BD, D, N);
  } else {
    if (sp) hipLaunchKernelGGL((step_complex_kernel<In, Out, DISC, false, true>), grid, block, 0, st, s, BD, D, N);
    else hipLaunchKernelGGL((step_complex_kernel<In, Out, DISC, false, false>), grid, block, 0, st, s, BD, D, N);
  }
  return hipGetLastError();
}

template <typename In, typename Out>
hipError_t step_disc(const StepArgs& s, const ss_desc_t& d, hipStream_t st) {
  const int64_t BD = d.batch * d.dim;
  const bool has_z = s.z != nullptr, sp = d.delta_softplus != 0;
  return d.disc == SS_ZOH ? step_flags<In, Out, SS_ZOH>(s, BD, d.dim, int(d.dstate), has_z, sp, st)
                          : step_flags<In, Out, SS_EULER>(s, BD, d.dim, int(d.dstate), has_z, sp, st);
}

}  // namespace

int launch_step_complex(const ss_desc_t& d, const StepArgs& s, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (d.in_dtype == SS_BF16)
    e = d.out_dtype == SS_F32 ? step_disc<uint16_t, float>(s, d, st) : step_disc<uint16_t, uint16_t>(s, d, st);
  else
    e = d.out_dtype == SS_F32 ? step_disc<float, float>(s, d, st) : step_disc<float, uint16_t>(s, d, st);
  return int(e);
}

int launch_fwd_complex(const ss_desc_t& d, const void* u, const void* delta, const float* A,
                       const void* Bm, const void* Cm, const float* Dskip, const float* bias,
                       const void* z, const float* h0, void* y, float* h_last, void* stream) {
  CParams p{u, delta, A, Bm, Cm, Dskip, bias, z, h0, y, h_last, d.seqlen, d.dim,
            int32_t(d.dstate), int32_t((d.dim + kChPerGroup - 1) / kChPerGroup)};
  const dim3 grid(unsigned(d.batch * p.ndblk));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool has_z = z != nullptr, sp = d.delta_softplus != 0;
  hipError_t e;
  if (d.in_dtype == SS_BF16)
    e = d.out_dtype == SS_F32 ? dispatch_disc<uint16_t, float>(p, d.disc, has_z, sp, grid, st)
                              : dispatch_disc<uint16_t, uint16_t>(p, d.disc, has_z, sp, grid, st);
  else
    e = d.out_dtype == SS_F32 ? dispatch_disc<float, float>(p, d.disc, has_z, sp, grid, st)
                              : dispatch_disc<float, uint16_t>(p, d.disc, has_z, sp, grid, st);
  return int(e);
}

}  // namespace ss
