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
// quad swaps), so lane q ends with the sum for its own step.
//
// Two forms of the step.  The fast one forms abar from one v_exp_f32 (the
// modulus) and one v_sin_f32 / v_cos_f32 pair (the phase, in revolutions).
// Those hardware results are off by up to ~1.3e-7, and v_cos_f32 is biased
// low by ~5e-8 near a zero phase; a state remembered for M steps at a nearly
// constant step size compounds that bias to ~M * 5e-8 of its modulus, which
// outgrows the fp32 bound once M reaches a few thousand steps.  The precise
// form carries E = abar - 1 = e^x (cos th + i sin th) - 1 instead,
// h <- h + (E h + bcoef B u), with e^x - 1 to full relative accuracy and sin,
// cos and cos - 1 from polynomials (sincos_rev), and takes the ZOH coefficient
// as E / a.  fp32 inputs always take it; bf16 waves take it when some state
// decays slowly (|Re a| < kWeakA), the others keep the fast form, whose error
// stays inside the bf16 bound.  B and C rows of a
// block are staged in LDS as fp32 (re, im) pairs; the inputs of the next block
// are fetched while the current one runs.  On the Mamba-2.8B width (B = 8,
// D = 5120) the grid is 1280 workgroups: five per compute unit, five waves per
// SIMD, each walking the whole sequence of its channels.
//
// Long, narrow problems are cut into time chunks, as the real scan is: a
// summary pass runs each chunk but the last from a zero state and keeps its end
// state and its sum of step sizes; an in-order walk (one lane per (b, n, d))
// turns those into each chunk's start state with the chunk maps
// h -> abar_c h + s_c, abar_c = exp(a sum dt) ("A Visual Guide to Mamba"
// summary, The Scan Operation: segments combined associatively); the output
// pass then runs every chunk from its true start.  The step sums are kept in
// fp64: a chunk's rotation angle Im(a) sum dt reaches hundreds of radians, and
// an fp32 sum (relative error ~1e-6 over thousands of steps) would put ~1e-2 rad
// of phase error into the carried state.
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
constexpr double kLn2Over2Pi = 0.69314718055994531 / 6.283185307179586;   // revolutions per log2 e
constexpr double kLog2eD = 1.4426950408889634;
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
  // (B, nc, N, D) complex: chunk c's zero-start end state from the summary pass
  // (c <= nc - 2), then the start state of chunk c (c >= 1)
  float2* hend;
  double* dsum;         // (B, nc, D): sum over chunk c of dt log2 e (c <= nc - 2)
  int64_t L, D;
  int64_t chunk_len;
  int32_t N, ndblk, nchunks, grid_chunks;
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

// sin(2 pi ph), cos(2 pi ph) and cos(2 pi ph) - 1 for a phase ph in
// revolutions (|ph| < 2^22), each to about 2 ulp (cos - 1 relative to itself):
// ph = k / 2 + r with k = rint(2 ph) and |r| <= 1/4 (exact in fp32), Taylor
// polynomials of sin t (through t^13) and cos t - 1 (through t^12) at
// t = 2 pi r, |t| <= pi / 2 (truncation below 7e-10 and 7e-9 relative), then
// a sign flip for odd k.  2 pi enters as a two-term split, so t is rounded
// once.
__device__ __forceinline__ void sincos_rev(float ph, float& s, float& c, float& cm1) {
  constexpr float kTwoPiHi = 6.28318548202514648f;        // fp32(2 pi)
  constexpr float kTwoPiLo = -1.7484555314695172e-07f;    // 2 pi - kTwoPiHi
  const float k = __builtin_rintf(2.0f * ph);
  const float r = __builtin_fmaf(k, -0.5f, ph);
  const float t = __builtin_fmaf(r, kTwoPiHi, r * kTwoPiLo);
  const float t2 = t * t;
  float ps = 1.0f / 6227020800.0f;                        // 1 / 13!
  ps = __builtin_fmaf(ps, t2, -1.0f / 39916800.0f);
  ps = __builtin_fmaf(ps, t2, 1.0f / 362880.0f);
  ps = __builtin_fmaf(ps, t2, -1.0f / 5040.0f);
  ps = __builtin_fmaf(ps, t2, 1.0f / 120.0f);
  ps = __builtin_fmaf(ps, t2, -1.0f / 6.0f);
  ps = __builtin_fmaf(ps, t2, 1.0f);
  float pc = 1.0f / 479001600.0f;                         // 1 / 12!
  pc = __builtin_fmaf(pc, t2, -1.0f / 3628800.0f);
  pc = __builtin_fmaf(pc, t2, 1.0f / 40320.0f);
  pc = __builtin_fmaf(pc, t2, -1.0f / 720.0f);
  pc = __builtin_fmaf(pc, t2, 1.0f / 24.0f);
  pc = __builtin_fmaf(pc, t2, -0.5f);
  const float st = t * ps, cmt = t2 * pc;                 // sin t, cos t - 1
  const bool odd = __builtin_amdgcn_fractf(0.5f * k) != 0.0f;
  s = odd ? -st : st;
  c = odd ? -1.0f - cmt : 1.0f + cmt;
  cm1 = odd ? -2.0f - cmt : cmt;
}

// dt log2 e = softplus(delta + bias) log2 e (or (delta + bias) log2 e), with the
// argument x2 = (delta + bias) log2 e carried as two terms.  Rounded to fp32
// once, x2 (|x2| ~ 9 at dt ~ 1e-3, ulp ~ 1e-6) would put up to ~3e-7 of
// relative error into dt, and the bias's share of that error repeats every
// step; a complex state turns through Im(a) / |Re(a)| radians over its memory
// (~75 for the S4D-Lin A), which multiplies a repeated error in dt.  Here
// b2h + b2l = bias log2 e (formed in fp64), delta log2 e keeps its exact
// product error, the two high parts meet in a TwoSum, and 2^-|x2| takes the
// low part to first order (it is below 2^-20 of x2).  The rest is
// softplus_log2's Fast2Sum form of log2(1 + e).
__device__ __forceinline__ float step_log2(float delta, float b2h, float b2l, bool softplus) {
  constexpr float kL2eHi = 1.44269502162933349609375f;    // fp32(log2 e)
  constexpr float kL2eLo = 1.925963033500011e-08f;         // log2 e - kL2eHi
  const float ph = delta * kL2eHi;
  const float pl = __builtin_fmaf(delta, kL2eHi, -ph) + delta * kL2eLo;
  const float sh = ph + b2h;                               // TwoSum: sh + sl = ph + b2h
  const float bv = sh - ph;
  const float sl = (ph - (sh - bv)) + (b2h - bv);
  const float lo = sl + (pl + b2l);
  if (!softplus) return sh + lo;
  const bool pos = sh > 0.0f;
  const float e0 = hw_exp2(-__builtin_fabsf(sh));
  const float e = __builtin_fmaf(e0, (pos ? -lo : lo) * kLn2, e0);   // 2^-|sh + lo|
  const float u1 = 1.0f + e;
  const float r = e - (u1 - 1.0f);                         // exact rounding error of u1
  const float k = __builtin_fmaf(-u1, kLog2e, 2.0f * kLog2e);
  return __builtin_fmaxf(sh, 0.0f) + ((pos ? lo : 0.0f) + __builtin_fmaf(r, k, hw_log2(u1)));
}

// E = abar - 1 for abar = e^x (cos th + i sin th): y2 = x log2 e, ph = th / 2 pi
__device__ __forceinline__ void cexpm1(float y2, float ph, float& er, float& ei) {
  const float em1 = precise_expm1(y2);
  float sn, cs, cm1;
  sincos_rev(ph, sn, cs, cm1);
  er = __builtin_fmaf(em1, cs, cm1);       // (e^x - 1) cos th + (cos th - 1)
  ei = __builtin_fmaf(em1, sn, sn);        // e^x sin th
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

// SUMMARY: run chunk `chunk` from a zero state and keep its end state and step
// sum (no output); otherwise run it from its start state and store y.
template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY>
// five waves per SIMD (five workgroups per CU at the 2.8B width): at most 96
// VGPRs; the summary pass, which also keeps an fp64 step sum, four (128 VGPRs)
__global__ __launch_bounds__(kWave * kCWaves, SUMMARY ? 4 : 5) void fwd_complex_kernel(CParams p) {
  const int tid = int(threadIdx.x);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int q = lane % kLPC, cl = lane / kLPC;
  const int chan = wave * kChPerWave + cl;                 // channel within the group
  const int dblk = int(blockIdx.x % unsigned(p.ndblk));
  const int64_t rest = int64_t(blockIdx.x / unsigned(p.ndblk));
  const int chunk = int(rest % p.grid_chunks);
  const int64_t b = rest / p.grid_chunks;
  const int64_t d = int64_t(dblk) * kChPerGroup + chan;
  const bool active = d < p.D;
  const int64_t dc = active ? d : p.D - 1;
  const int N = p.N;
  const int64_t L = p.L, D = p.D;
  // this workgroup's steps [tb, te); "L" below bounds the loads and stores
  const int64_t tb = int64_t(chunk) * p.chunk_len;
  const int64_t te = tb + p.chunk_len < L ? tb + p.chunk_len : L;

  // per-state constants: modulus rate, phase rate (revolutions per dt log2 e,
  // formed in fp64 and kept as aw + awl, so that the rate carries no rounding
  // that would repeat every step), 1 / a (0 when a == 0) and z0 = [a == 0]
  // (the ZOH coefficient is then dt)
  float ar[kSPL], aw[kSPL], awl[kSPL], iar[kSPL], iai[kSPL], z0[kSPL], hr[kSPL], hi[kSPL];
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
    const double awd = double(im) * kLn2Over2Pi;
    aw[j] = float(awd);
    awl[j] = float(awd - double(aw[j]));
    const float m2 = re * re + im * im;
    weak |= !(__builtin_fabsf(re) >= kWeakA);
    iar[j] = m2 == 0.0f ? 0.0f : re / m2;
    iai[j] = m2 == 0.0f ? 0.0f : -im / m2;
    z0[j] = m2 == 0.0f ? 1.0f : 0.0f;
    hr[j] = 0.0f;
    hi[j] = 0.0f;
    if (!SUMMARY && n < N) {
      if (chunk == 0 && p.h0) {
        hr[j] = p.h0[((b * D + dc) * N + n) * 2];
        hi[j] = p.h0[((b * D + dc) * N + n) * 2 + 1];
      } else if (chunk > 0) {
        const float2 hs = p.hend[((b * p.nchunks + chunk) * N + n) * D + dc];
        hr[j] = hs.x;
        hi[j] = hs.y;
      }
    }
  }
  double dsum = 0.0;
  // the precise step for fp32 inputs and for waves holding a slowly decaying state
  bool precise;
  if constexpr (std::is_same<In, float>::value) precise = true;
  else precise = __any(weak);
  const float Dd = p.Dskip ? p.Dskip[dc] : 0.0f;
  const double b2 = double(p.bias ? p.bias[dc] : 0.0f) * kLog2eD;   // bias log2 e, two terms
  const float b2h = float(b2), b2l = float(b2 - double(b2h));

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
    const int64_t t = t0 + q < te ? t0 + q : te - 1;
    ur[S] = ub[t * D];
    dr[S] = db[t * D];
    if (HAS_Z && !SUMMARY) zr[S] = zb[t * D];
    const int64_t tr = t0 + sk < te ? t0 + sk : te - 1;
    rw[S] = Pair<In>::load(rbase + ((b * L + tr) * N + (sn < N ? sn : 0)) * 2);
  };
  // the block's rows and this lane's owned-step values into buffer S
  // P: the precise step, which also takes the step size from the two-term
  // argument (the fast step's error budget does not need it)
  auto stage = [&](auto S_, auto P_, int64_t t0) {
    constexpr int S = decltype(S_)::value;
    constexpr bool P = decltype(P_)::value;
    float2 v = Pair<In>::f32(rw[S]);
    if (sn >= N || t0 + sk >= te) v = make_float2(0.0f, 0.0f);
    rows[S][sk][sw][sn] = v;
    const bool valid = t0 + q < te;
    float dl;                                                         // dt log2 e
    if (P) {
      dl = step_log2(to_f32(dr[S]), b2h, b2l, SOFTPLUS);
    } else {
      const float x2 = __builtin_fmaf(to_f32(dr[S]), kLog2e, b2h);
      dl = SOFTPLUS ? softplus_log2(x2) : x2;
    }
    dl = valid ? dl : 0.0f;
    u_own[S] = valid ? to_f32(ur[S]) : 0.0f;
    g_own[S] = HAS_Z && !SUMMARY ? silu(to_f32(zr[S])) : 1.0f;
    act[S][q][chan] = make_float2(dl, u_own[S]);
  };

  // P: the precise step (a template parameter, so that neither loop branches)
  auto block = [&](auto S_, auto P_, int64_t t0) {
    constexpr int S = decltype(S_)::value;
    constexpr bool P = decltype(P_)::value;
    if (t0 + kCBlk < te) fetch(std::integral_constant<int, S ^ 1>{}, t0 + kCBlk);
    float part[kCBlk];                                     // Re sum_n C h, per step
    float bsum = 0.0f;                                     // the block's step sum
#pragma unroll
    for (int k = 0; k < kCBlk; ++k) {
      const float2 du = act[S][k][chan];
      const float dl = du.x, uk = du.y;
      if (SUMMARY) bsum += dl;
      const float dt = dl * kLn2;
      const float4 bq = *reinterpret_cast<const float4*>(&rows[S][k][0][kSPL * q]);
      const float4 cq = *reinterpret_cast<const float4*>(&rows[S][k][1][kSPL * q]);
      const float Br[kSPL] = {bq.x, bq.z}, Bi[kSPL] = {bq.y, bq.w};
      const float Cr[kSPL] = {cq.x, cq.z}, Ci[kSPL] = {cq.y, cq.w};
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < kSPL; ++j) {
        const float bur = Br[j] * uk, bui = Bi[j] * uk;
        float nr, ni;
        if (P) {
          float er, ei;                                               // abar - 1
          cexpm1(dl * ar[j], __builtin_fmaf(dl, aw[j], dl * awl[j]), er, ei);
          float cr = dt, ci = 0.0f;                                   // Euler
          if (DISC == SS_ZOH) {                                       // E / a (dt if a == 0)
            cr = __builtin_fmaf(er, iar[j], __builtin_fmaf(-ei, iai[j], dt * z0[j]));
            ci = __builtin_fmaf(er, iai[j], ei * iar[j]);
          }
          const float qr = cr * bur - ci * bui, qi = __builtin_fmaf(cr, bui, ci * bur);
          nr = hr[j] + __builtin_fmaf(er, hr[j], __builtin_fmaf(-ei, hi[j], qr));
          ni = hi[j] + __builtin_fmaf(er, hi[j], __builtin_fmaf(ei, hr[j], qi));
        } else {
          const float e = hw_exp2(dl * ar[j]);                        // |abar|
          const float ph = __builtin_amdgcn_fractf(dl * aw[j]);       // arg abar / 2 pi
          const float abr = e * __builtin_amdgcn_cosf(ph);
          const float abi = e * __builtin_amdgcn_sinf(ph);
          float cr = dt, ci = 0.0f;                                   // Euler
          if (DISC == SS_ZOH) {
            const float mr = abr - 1.0f;                              // (abar - 1) / a
            cr = mr * iar[j] - abi * iai[j];
            ci = __builtin_fmaf(mr, iai[j], abi * iar[j]);
          }
          const float qr = cr * bur - ci * bui, qi = __builtin_fmaf(cr, bui, ci * bur);
          nr = __builtin_fmaf(abr, hr[j], __builtin_fmaf(-abi, hi[j], qr));
          ni = __builtin_fmaf(abr, hi[j], __builtin_fmaf(abi, hr[j], qi));
        }
        hr[j] = nr;
        hi[j] = ni;
        if (!SUMMARY) acc = __builtin_fmaf(Cr[j], nr, __builtin_fmaf(-Ci[j], ni, acc));
      }
      part[k] = acc;
    }
    if (SUMMARY) dsum += double(bsum);   // 8 fp32 terms per block, fp64 across blocks
    if (!SUMMARY) {
      // y of the owned step: the channel's sum for step q, skip, gate
      const float sum = reduce_scatter8(part, q);
      float yv = __builtin_fmaf(2.0f, sum, Dd * u_own[S]);
      if (HAS_Z) yv *= g_own[S];
      if (t0 + q < te && active) store_out<Out>(yb + (t0 + q) * D, yv);
    }
    // the next block's rows and owned-step values into the other buffers (last
    // read by the previous block, which every wave finished before the
    // barrier that ended it)
    if (t0 + kCBlk < te) stage(std::integral_constant<int, S ^ 1>{}, P_, t0 + kCBlk);
    __syncthreads();
  };

  auto walk = [&](auto P_) {
    fetch(std::integral_constant<int, 0>{}, tb);
    stage(std::integral_constant<int, 0>{}, P_, tb);
    __syncthreads();
    for (int64_t t0 = tb; t0 < te; t0 += 2 * kCBlk) {
      block(std::integral_constant<int, 0>{}, P_, t0);
      if (t0 + kCBlk < te) block(std::integral_constant<int, 1>{}, P_, t0 + kCBlk);
    }
  };
  if (precise) walk(std::true_type{});
  else walk(std::false_type{});
  if (SUMMARY) {
    if (active) {
#pragma unroll
      for (int j = 0; j < kSPL; ++j) {
        const int n = kSPL * q + j;
        if (n < N) p.hend[((b * p.nchunks + chunk) * N + n) * D + d] = make_float2(hr[j], hi[j]);
      }
      if (q == 0) p.dsum[(b * p.nchunks + chunk) * D + d] = dsum;
    }
    return;
  }
  if (p.h_last && active && te == L) {
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
hipError_t dispatch_flags(const CParams& p, bool has_z, bool sp, bool summary, dim3 grid,
                          hipStream_t st) {
  const dim3 block(kWave * kCWaves);
  if (summary) {
    // no output, no gate: one instantiation per input type (the fp32-output one)
    if constexpr (std::is_same<Out, float>::value) {
      if (sp) hipLaunchKernelGGL((fwd_complex_kernel<In, Out, DISC, false, true, true>), grid, block, 0, st, p);
      else hipLaunchKernelGGL((fwd_complex_kernel<In, Out, DISC, false, false, true>), grid, block, 0, st, p);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (has_z) {
    if (sp) hipLaunchKernelGGL((fwd_complex_kernel<In, Out, DISC, true, true, false>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((fwd_complex_kernel<In, Out, DISC, true, false, false>), grid, block, 0, st, p);
  } else {
    if (sp) hipLaunchKernelGGL((fwd_complex_kernel<In, Out, DISC, false, true, false>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((fwd_complex_kernel<In, Out, DISC, false, false, false>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

template <typename In, typename Out>
hipError_t dispatch_disc(const CParams& p, int disc, bool has_z, bool sp, bool summary, dim3 grid,
                         hipStream_t st) {
  return disc == SS_ZOH ? dispatch_flags<In, Out, SS_ZOH>(p, has_z, sp, summary, grid, st)
                        : dispatch_flags<In, Out, SS_EULER>(p, has_z, sp, summary, grid, st);
}

hipError_t dispatch_types(const ss_desc_t& d, const CParams& p, bool summary, dim3 grid,
                          hipStream_t st) {
  const bool has_z = p.z != nullptr, sp = d.delta_softplus != 0;
  if (d.in_dtype == SS_BF16)
    return d.out_dtype == SS_F32 || summary
               ? dispatch_disc<uint16_t, float>(p, d.disc, has_z, sp, summary, grid, st)
               : dispatch_disc<uint16_t, uint16_t>(p, d.disc, has_z, sp, false, grid, st);
  return d.out_dtype == SS_F32 || summary
             ? dispatch_disc<float, float>(p, d.disc, has_z, sp, summary, grid, st)
             : dispatch_disc<float, uint16_t>(p, d.disc, has_z, sp, false, grid, st);
}

// Chunk carries of the complex scan: one lane per (b, n, d) walks the chunks
// in order.  Slot c of hend holds chunk c's zero-start end state s_c
// (c <= nc - 2); afterwards slot c (c >= 1) holds chunk c's start state.  The
// chunk map is h -> abar_c h + s_c with abar_c = exp(a sum dt), applied in the
// precise form h + (E_c h + s_c), E_c = abar_c - 1; its phase Im(a) sum dt is
// reduced to [-1/2, 1/2] revolutions in fp64 (the sum is fp64 too).
__global__ __launch_bounds__(256) void complex_walk_kernel(float2* __restrict__ hend,
                                                           const double* __restrict__ dsum,
                                                           const float* __restrict__ A,
                                                           const float* __restrict__ h0,
                                                           int64_t B, int64_t D, int N, int nc) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= B * N * D) return;
  const int64_t d = gid % D;
  const int n = int((gid / D) % N);
  const int64_t b = gid / (D * N);
  const float ar = A[(d * N + n) * 2];
  const double aw = double(A[(d * N + n) * 2 + 1]) * kLn2Over2Pi;
  float hr = h0 ? h0[((b * D + d) * N + n) * 2] : 0.0f;
  float hi = h0 ? h0[((b * D + d) * N + n) * 2 + 1] : 0.0f;
  float2* st = hend + (b * nc) * int64_t(N) * D + int64_t(n) * D + d;
  const int64_t sstride = int64_t(N) * D;
  const double* ds = dsum + (b * nc) * D + d;
  for (int c = 0; c < nc - 1; ++c) {
    const float2 sc = st[c * sstride];
    if (c >= 1) st[c * sstride] = make_float2(hr, hi);
    const double dl = ds[int64_t(c) * D];                 // sum of dt log2 e over the chunk
    const double rev = dl * aw;
    float er, ei;                                         // abar_c - 1
    cexpm1(float(dl) * ar, float(rev - __builtin_rint(rev)), er, ei);
    const float nr = hr + __builtin_fmaf(er, hr, __builtin_fmaf(-ei, hi, sc.x));
    const float ni = hi + __builtin_fmaf(er, hi, __builtin_fmaf(ei, hr, sc.y));
    hr = nr;
    hi = ni;
  }
  st[int64_t(nc - 1) * sstride] = make_float2(hr, hi);
}

// One recurrent step with complex A (decoding): h (B, D, N, 2) in place, y (B, D).
// kLPC lanes per (b, d), lane q holding states n = kSPL q + j as in the scan,
// always in the scan's precise form (E = abar - 1, the ZOH coefficient E / a),
// so a step continues a scan.  The lanes' partial sums of Re C h meet by
// butterflies in a fixed order.
template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS>
__global__ __launch_bounds__(256) void step_complex_kernel(StepArgs a, int64_t BD, int64_t D, int N) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int q = int(gid % kLPC);
  const int64_t ch = gid / kLPC;
  const bool live = ch < BD;
  const int64_t chc = live ? ch : BD - 1;                 // idle lanes still join the butterflies
  const int64_t b = chc / D, d = chc % D;
  const double b2 = double(a.bias ? a.bias[d] : 0.0f) * kLog2eD;
  const float b2h = float(b2), b2l = float(b2 - double(b2h));
  const float dl = step_log2(to_f32(static_cast<const In*>(a.delta)[chc]), b2h, b2l, SOFTPLUS);
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
    const double awd = double(ai) * kLn2Over2Pi;
    const float aw = float(awd), awl = float(awd - double(aw));
    float er, ei;                                                 // abar - 1
    cexpm1(dl * ar, __builtin_fmaf(dl, aw, dl * awl), er, ei);
    float cr = dt, ci = 0.0f;                                     // Euler
    if (DISC == SS_ZOH) {                                         // E / a (dt if a == 0)
      cr = __builtin_fmaf(er, iar, __builtin_fmaf(-ei, iai, m2 == 0.0f ? dt : 0.0f));
      ci = __builtin_fmaf(er, iai, ei * iar);
    }
    const typename Pair<In>::raw rb = Pair<In>::load(static_cast<const In*>(a.Bm) + (b * N + n) * 2);
    const typename Pair<In>::raw rc = Pair<In>::load(static_cast<const In*>(a.Cm) + (b * N + n) * 2);
    const float2 Bv = Pair<In>::f32(rb), Cv = Pair<In>::f32(rc);
    const float bur = Bv.x * uk, bui = Bv.y * uk;
    const float qr = cr * bur - ci * bui, qi = __builtin_fmaf(cr, bui, ci * bur);
    float* hp = a.h + (chc * N + n) * 2;
    const float hr = hp[0], hi = hp[1];
    const float nr = hr + __builtin_fmaf(er, hr, __builtin_fmaf(-ei, hi, qr));
    const float ni = hi + __builtin_fmaf(er, hi, __builtin_fmaf(ei, hr, qi));
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

int launch_fwd_complex(const ss_desc_t& d, const CplxPlan& plan, const void* u, const void* delta,
                       const float* A, const void* Bm, const void* Cm, const float* Dskip,
                       const float* bias, const void* z, const float* h0, void* y, float* h_last,
                       char* ws, void* stream) {
  CParams p{};
  p.u = u; p.delta = delta; p.A = A; p.Bm = Bm; p.Cm = Cm; p.Dskip = Dskip; p.bias = bias;
  p.z = z; p.h0 = h0; p.y = y; p.h_last = h_last;
  p.L = d.seqlen; p.D = d.dim; p.N = int32_t(d.dstate);
  p.ndblk = int32_t((d.dim + kChPerGroup - 1) / kChPerGroup);
  p.chunk_len = plan.chunk_len;
  p.nchunks = int32_t(plan.nchunks);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t cols = d.batch * p.ndblk;
  if (plan.nchunks > 1) {
    p.hend = reinterpret_cast<float2*>(ws + plan.off_hend);
    p.dsum = reinterpret_cast<double*>(ws + plan.off_dsum);
    p.grid_chunks = p.nchunks - 1;     // the last chunk's summary is never needed
    hipError_t e = dispatch_types(d, p, true, dim3(unsigned(cols * p.grid_chunks)), st);
    if (e != hipSuccess) return int(e);
    const int64_t lanes = d.batch * d.dstate * d.dim;
    hipLaunchKernelGGL(complex_walk_kernel, dim3(unsigned((lanes + 255) / 256)), dim3(256), 0, st,
                       p.hend, p.dsum, A, h0, d.batch, d.dim, int(d.dstate), p.nchunks);
    e = hipGetLastError();
    if (e != hipSuccess) return int(e);
  }
  p.grid_chunks = p.nchunks;
  return int(dispatch_types(d, p, false, dim3(unsigned(cols * p.grid_chunks)), st));
}

}  // namespace ss
