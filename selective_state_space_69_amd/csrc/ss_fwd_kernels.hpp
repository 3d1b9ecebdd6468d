// Forward selective scan for gfx950: kernel templates (instantiated per
// element-type pair in ss_fwd_<in>_<out>.hip, launched from ss_fwd.hip).
//
// Mapping: one workgroup per (batch row b, block of 64 channels, time chunk),
// made of NSPLIT wavefronts (1, 2 or 4).  Lane = channel d; wave w of the group
// keeps states n in [w*NS, (w+1)*NS), NS = 16 / NSPLIT, as fp32 in VGPRs and
// walks the chunk's time steps sequentially.  Every (b, t) row of B and C is
// shared by all channels (Broadcast over D: "A Survey of Mamba" summary,
// Selection), so it is the same for the whole wave: the rows are staged through
// LDS a block of 8 steps at a time and read back with broadcast loads.  Per
// element (b, t, d, n) the work is one v_exp_f32 and 4 (Euler) or 6 (exact ZOH)
// vector ops (about 14 with the precise decay of fp32 inputs and slowly
// decaying states); the discretised A_bar, B_bar and the states never touch memory
// ("A Visual Guide to Mamba" summary, Hardware-aware Algorithm: discretisation,
// scan and the C contraction fused in one kernel).  With NSPLIT > 1 the waves'
// partial sums over n of C h are added through LDS once per 8-step block; the
// wave that owns a step adds the D skip, applies the gate and stores y.  Splitting the states gives more
// waves per SIMD on wide problems, which hides the latency of the
// transcendental units; each wave repeats the cheap per-step softplus.
//
// Long or narrow problems are cut into time chunks (two-level carry):
//   1. summary pass: per chunk, the zero-start end state S and the summed step
//      sum(dt) (the chunk decay is exp(A * sum(dt)));
//   2. carry scan: start state of chunk c+1 = exp(A sum_c) * start_c + S_c, the
//      associative combine (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2) ("A Visual
//      Guide to Mamba" summary, The Scan Operation: segments combined
//      associatively), done as a wave64 scan over chunks;
//   3. output pass: each chunk re-runs from its true start state and writes y.
#pragma once

#include <type_traits>

#include "ss_fwd_common.hpp"

namespace ss {
namespace {

constexpr int kPrefetch = kBlk;  // time steps per block (u, delta, z ring; B, C staging)

template <int NS>
struct Chan {
  float A[NS];    // diagonal A[d, n]; unused states get -1 (inert: B = C = 0)
  float iA[NS];   // 1 / A (0 where A == 0)
};

// LDS per workgroup: B/C row staging, per wave 2 buffers x 8 steps x 2*NS floats
// (= 512 floats for the whole group); with NSPLIT > 1 also the shared step
// sizes and u, [2 buffers][8 steps][64 lanes][2], and the partial outputs,
// [2 buffers][NSPLIT waves][8 steps][64 lanes].  Lane is the fastest index, so
// the accesses of a wave hit consecutive banks.
template <int NSPLIT>
struct Lds {
  static constexpr int kNS = kMaxState / NSPLIT;
  static constexpr int kStage = 2 * kPrefetch * 2 * kNS;                 // floats per wave
  static constexpr int kAct = NSPLIT > 1 ? 2 * kWave * kPrefetch * 2 : 0;
  static constexpr int kPart = NSPLIT > 1 ? 2 * NSPLIT * kWave * kPrefetch : 0;
  static constexpr int kFloats = NSPLIT * kStage + kAct + kPart;
};

// Step ownership inside a block of 8 steps: step k belongs to wave k % NSPLIT,
// which alone computes its softplus step size (shared with the other waves
// through LDS), its gate, and its final output.
template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY,
          bool PRECISE, int NSPLIT, bool REV>
struct Scan {
  static constexpr int NS = kMaxState / NSPLIT;
  static constexpr int OWN = kPrefetch / NSPLIT;   // steps owned per block
  const FwdParams& p;
  const Chan<NS>& ch;
  float (&h)[NS];
  float Dd, bias2;
  float dsum;
  int64_t bidx;          // batch row
  TimeDir<REV> td;
  const In* ub;          // wave-uniform base pointers of (b, logical t = 0, d = 64 * dblk)
  const In* db;
  const In* zb;
  Out* yb;
  uint32_t vin, vout;    // per-lane byte offsets (vout is out of range for idle lanes)
  uint32_t rowb_in, rowb_out;
  int32_t t1, tlast;
  float* stage;          // this wave's row staging buffer (2 x 8 x 2*NS floats)
  float* act;            // shared step sizes and u (NSPLIT > 1)
  float* part;           // partial outputs (NSPLIT > 1)
  uint32_t lane;
  int wave, n0;          // wave index in the group, first state of this wave
  // Two-deep prefetch ring, slot = block parity: while block t runs, slot
  // (t / 8) & 1 receives block t + 16 and the other slot holds block t + 8.  A
  // load thus has a whole block of compute before its value is needed.  With
  // one wave it holds u of every step; with several, each step's owner loads
  // its u and publishes it (fp32) with the step size, so no wave loads and
  // widens the u of the others' steps.
  In ur[2][kPrefetch];                  // u of every step (NSPLIT == 1)
  In dr[2][OWN], zr[2][OWN], uo[2][OWN];   // delta, z, u of the owned steps
  typename Raw4<In>::type rowq[2];      // this lane's 16 (fp32) or 8 (bf16) bytes of rows
  float dl_own[OWN], g_own[OWN], u_own[OWN];   // step size, gate and u of the owned steps

  __device__ __forceinline__ int owned(int i) const { return i * NSPLIT + wave; }

  // Prefetch of block t into ring slot S: u of every step, delta, z and u of
  // the owned steps, B/C rows.  load_u issues one step's u, so that inside a
  // block each load can reuse the register its predecessor in the slot has
  // just released.
  template <typename T>
  __device__ __forceinline__ Rsrc at(const T* base, int32_t t) const {
    return make_rsrc(base + int64_t(td.blk(t)) * td.ts);
  }
  __device__ __forceinline__ Rsrc u_rsrc(int32_t t) const { return at(ub, t); }
  template <int S>
  __device__ __forceinline__ void load_u(const Rsrc& ru, int k, int32_t lim, bool clamp) {
    int32_t tt = k;
    if (clamp) tt = tt < lim ? tt : lim;
    ur[S][k] = buf_load<In>(ru, vin, td.pos(tt) * rowb_in);
  }
  template <int S>
  __device__ __forceinline__ void load_owned(int32_t t, bool clamp) {
    const Rsrc ru = u_rsrc(t), rd = at(db, t);
    const Rsrc rz = at(HAS_Z ? zb : ub, t);
    const int32_t lim = tlast - t;    // last valid step, relative to t
#pragma unroll
    for (int i = 0; i < OWN; ++i) {
      int32_t tt = owned(i);
      if (clamp) tt = tt < lim ? tt : lim;
      const uint32_t so = td.pos(tt) * rowb_in;
      dr[S][i] = buf_load<In>(rd, vin, so);
      if (HAS_Z && !SUMMARY) zr[S][i] = buf_load<In>(rz, vin, so);
      if (NSPLIT > 1) uo[S][i] = buf_load<In>(ru, vin, so);
    }
  }
  template <int S>
  __device__ __forceinline__ void load_ring(int32_t t, bool clamp) {
    if constexpr (NSPLIT == 1) {
      const Rsrc ru = u_rsrc(t);
#pragma unroll
      for (int k = 0; k < kPrefetch; ++k) load_u<S>(ru, k, tlast - t, clamp);
    }
    load_owned<S>(t, clamp);
  }

  // step size (log2 units) and gate of the owned steps of the block at t, from
  // ring slot S; steps at or past t1 get dt = 0
  template <int S>
  __device__ __forceinline__ void activations(int32_t t) {
#pragma unroll
    for (int i = 0; i < OWN; ++i) {
      float x2 = __builtin_fmaf(to_f32(dr[S][i]), kLog2e, bias2);  // (delta + bias) log2 e
      const bool pad = t + owned(i) >= t1;
      if (pad) x2 = SOFTPLUS ? -__builtin_inff() : 0.0f;
      dl_own[i] = SOFTPLUS ? softplus_log2(x2) : x2;               // dt * log2 e
      if (HAS_Z && !SUMMARY) g_own[i] = silu(to_f32(zr[S][i]));
      if constexpr (NSPLIT > 1) u_own[i] = pad ? 0.0f : to_f32(uo[S][i]);   // padded: inert
      else if (!SUMMARY) u_own[i] = to_f32(ur[S][i]);
    }
  }
  template <int S>
  __device__ __forceinline__ void publish() {
    if (NSPLIT == 1) return;
#pragma unroll
    for (int i = 0; i < OWN; ++i)
      reinterpret_cast<float2*>(act)[(S * kPrefetch + owned(i)) * kWave + lane] =
          make_float2(dl_own[i], DISC == kEuler ? u_own[i] * kLn2 : u_own[i]);   // Euler: u ln 2
  }

  // Rows of block [t, t + 8): per step, NS values of B then NS of C (this wave's
  // states), i.e. NS/2 groups of 4; lane l fetches group g = l % (NS/2) of step
  // k = (l / (NS/2)) % 8 (lanes beyond 4*NS repeat lower lanes' work).
  template <int S>
  __device__ __forceinline__ void fetch_rows(int32_t t) {
    constexpr int G = NS / 2;
    const uint32_t l = lane % uint32_t(4 * NS);
    const int k = int(l / G), g = int(l % G);
    int32_t tr = t + k;
    tr = tr < tlast ? tr : tlast;
    const int64_t rw = REV ? bidx * p.L + (p.L - 1) - tr : bidx * p.L + tr;
    const In* src = static_cast<const In*>(g < G / 2 ? p.Brow : p.Crow) +
                    rw * kMaxState + n0 + 4 * (g % (G / 2));
    rowq[S] = load_raw4(src);
  }
  template <int S>
  __device__ __forceinline__ void stage_rows() {
    constexpr int G = NS / 2;
    const uint32_t l = lane % uint32_t(4 * NS);
    const uint32_t off = S * (kPrefetch * 2 * NS) + (l / G) * (2 * NS) + 4 * (l % G);
    *reinterpret_cast<float4*>(stage + off) = unpack4(rowq[S]);
  }
  template <int S>
  __device__ __forceinline__ void read_rows(int k, float (&Bv)[NS], float (&Cv)[NS]) {
    const float4* q = reinterpret_cast<const float4*>(stage + S * (kPrefetch * 2 * NS) + k * 2 * NS);
#pragma unroll
    for (int m = 0; m < NS / 4; ++m) {
      const float4 v = q[m];
      Bv[4 * m] = v.x; Bv[4 * m + 1] = v.y; Bv[4 * m + 2] = v.z; Bv[4 * m + 3] = v.w;
    }
    if (!SUMMARY) {
#pragma unroll
      for (int m = 0; m < NS / 4; ++m) {
        const float4 v = q[NS / 4 + m];
        Cv[4 * m] = v.x; Cv[4 * m + 1] = v.y; Cv[4 * m + 2] = v.z; Cv[4 * m + 3] = v.w;
      }
    }
  }

  // One block of 8 steps starting at t, ring slot / LDS buffer S = (t / 8) & 1.
  // On entry slot S holds this block's u, the LDS buffer S its rows and step
  // sizes (behind a barrier), and the owned-step activations are computed;
  // slot S^1 holds block t + 8.  GUARD: the prefetch of block t + 16 is clamped
  // to the range and stores past t1 are skipped.
  template <bool GUARD, int S>
  __device__ __forceinline__ void block(int32_t t) {
    float g[OWN], us[OWN];
#pragma unroll
    for (int i = 0; i < OWN; ++i) {
      g[i] = g_own[i];
      us[i] = u_own[i];
    }
    // prefetch block t + 16 into slot S: owned-step inputs and rows now, with
    // one wave the u of step k right after step k has read its slot entry
    const int32_t tn0 = t + 2 * kPrefetch;
    const int32_t tn = tn0 < tlast ? tn0 : tlast;
    load_owned<S>(tn, GUARD);
    fetch_rows<S>(tn);
    const Rsrc ru = u_rsrc(tn);
    const Rsrc ry = at(yb, t);
    const float2* dls = reinterpret_cast<const float2*>(act) + S * kPrefetch * kWave + lane;
    float* parts = part + (S * NSPLIT + wave) * kPrefetch * kWave + lane;
    // the recurrence, one step at a time (rows and step sizes read one step ahead)
    float Bn[NS], Cn[NS];
    read_rows<S>(0, Bn, Cn);
    float2 dn;   // (dt log2 e, u) of the next step
    if constexpr (NSPLIT == 1) dn = make_float2(dl_own[0], 0.0f);
    else dn = dls[0];
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
      float Bv[NS], Cv[NS];
#pragma unroll
      for (int n = 0; n < NS; ++n) { Bv[n] = Bn[n]; Cv[n] = Cn[n]; }
      const float d2 = dn.x;
      float uk = dn.y;
      if (k + 1 < kPrefetch) {
        read_rows<S>(k + 1, Bn, Cn);
        if constexpr (NSPLIT == 1) dn = make_float2(dl_own[k + 1], 0.0f);
        else dn = dls[(k + 1) * kWave];
      }
      if constexpr (NSPLIT == 1) {
        uk = to_f32(ur[S][k]);
        load_u<S>(ru, k, tlast - tn, GUARD);
      }
      float acc0 = 0.0f, acc1 = 0.0f;   // two chains when a wave holds many states
      constexpr bool kTwo = NS > 4;
      if (DISC == kEuler) {
        const float dtu = NSPLIT > 1 ? d2 * uk : d2 * (kLn2 * uk);   // dt * u (shared u: u ln 2)
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          if (PRECISE) {
            float unused;
            const float e = precise_decay<false>(d2, ch.A[n], ch.iA[n], unused);   // A_bar - 1
            h[n] += __builtin_fmaf(e, h[n], dtu * Bv[n]);
          } else {
            const float a = hw_exp2(d2 * ch.A[n]);                // A_bar = exp(dt A)
            h[n] = __builtin_fmaf(a, h[n], dtu * Bv[n]);          // + dt B u
          }
          if (!SUMMARY) {
            if (kTwo && (n & 1)) acc1 = __builtin_fmaf(Cv[n], h[n], acc1);
            else acc0 = __builtin_fmaf(Cv[n], h[n], acc0);
          }
        }
      } else {
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          if (PRECISE) {
            // h <- h + (E h + coef B u): E = A_bar - 1, coef = E / A, full relative accuracy
            float coef;
            const float e = precise_decay<true>(d2, ch.A[n], ch.iA[n], coef);
            h[n] += __builtin_fmaf(e, h[n], coef * (Bv[n] * uk));
          } else if (SUMMARY) {
            // the chunk summary from a zero start keeps s = A h, as the
            // 32-channel kernel's states: s <- a (s + B u) - B u, one operation
            // fewer (every |A| >= kWeakA on this path; unscaled at the end)
            const float a = hw_exp2(d2 * ch.A[n]);
            const float bu = Bv[n] * uk;
            h[n] = __builtin_fmaf(a, h[n] + bu, -bu);
          } else {
            const float a = hw_exp2(d2 * ch.A[n]);                // A_bar = exp(dt A)
            const float coef = __builtin_fmaf(a, ch.iA[n], -ch.iA[n]);   // (A_bar - 1) / A
            h[n] = __builtin_fmaf(a, h[n], coef * (Bv[n] * uk));
          }
          if (!SUMMARY) {
            if (kTwo && (n & 1)) acc1 = __builtin_fmaf(Cv[n], h[n], acc1);
            else acc0 = __builtin_fmaf(Cv[n], h[n], acc0);
          }
        }
      }
      if (SUMMARY) {
        dsum += d2;
      } else {
        const float acc = kTwo ? acc0 + acc1 : acc0;
        if constexpr (NSPLIT > 1) {
          parts[k * kWave] = acc;                                  // partial C h
        } else {
          // one wave holds every state: y of step k is complete
          float yv = __builtin_fmaf(Dd, uk, acc);                  // + D skip
          if (HAS_Z) yv *= g[k];                                   // silu(z) gate
          if (!GUARD || t + k < t1) {
            const uint32_t so = td.pos(k) * rowb_out;
            if (p.acc) yv += to_f32(buf_load<Out>(ry, vout, so));
            buf_store<Out>(ry, vout, so, yv);
          }
        }
      }
    }
    // 4. activations of block t + 8 (slot S^1, loaded one block ago), its rows
    activations<S ^ 1>(t + kPrefetch);
    publish<S ^ 1>();
    stage_rows<S ^ 1>();
    if (NSPLIT > 1) __syncthreads();
    if (SUMMARY || NSPLIT == 1) return;
    // 5. outputs of the owned steps: sum of the waves' partials, skip, gate, store
#pragma unroll
    for (int i = 0; i < OWN; ++i) {
      const int k = owned(i);
      float yv = 0.0f;
#pragma unroll
      for (int w = 0; w < NSPLIT; ++w) yv += part[((S * NSPLIT + w) * kPrefetch + k) * kWave + lane];
      yv = __builtin_fmaf(Dd, us[i], yv);                          // + D skip
      if (HAS_Z) yv *= g[i];                                       // silu(z) gate
      if (!GUARD || t + k < t1) {
        const uint32_t so = td.pos(k) * rowb_out;
        if (p.acc) yv += to_f32(buf_load<Out>(ry, vout, so));
        buf_store<Out>(ry, vout, so, yv);
      }
    }
  }

  __device__ __forceinline__ void run(int32_t t0) {
    const int32_t t8 = t0 + kPrefetch < tlast ? t0 + kPrefetch : tlast;
    load_ring<0>(t0, true);
    fetch_rows<0>(t0);
    load_ring<1>(t8, true);
    fetch_rows<1>(t8);
    stage_rows<0>();
    activations<0>(t0);
    publish<0>();
    if (NSPLIT > 1) __syncthreads();
    int32_t t = t0;
    // pairs of full blocks whose prefetch (up to t + 31) stays inside the range
    for (; t + 4 * kPrefetch <= t1; t += 2 * kPrefetch) {
      block<false, 0>(t);
      block<false, 1>(t + kPrefetch);
    }
    for (; t < t1; t += 2 * kPrefetch) {
      block<true, 0>(t);
      if (t + kPrefetch < t1) block<true, 1>(t + kPrefetch);
    }
  }
};

// Minimum waves per SIMD the register allocation must allow: the one-wave
// layout keeps 16 states per lane and runs on very wide problems; the split
// layouts need several resident waves per SIMD to hide latency.
template <int NSPLIT>
constexpr int kMinWaves = NSPLIT == 1 ? 2 : 3;

template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY, int NSPLIT,
          bool REV>
__global__ __launch_bounds__(kWave * NSPLIT, kMinWaves<NSPLIT>) void fwd_kernel(FwdParams p) {
  constexpr int NS = kMaxState / NSPLIT;
  // wave-uniform by construction; readfirstlane lets the compiler keep it in an SGPR
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const int lane = int(threadIdx.x) % kWave;
  const int n0 = wave * NS;
  int64_t bid = blockIdx.x;
  const int dblk = int(bid % p.ndblk);
  bid /= p.ndblk;
  const int chunk = int(bid % p.grid_chunks);
  const int64_t b = bid / p.grid_chunks;
  const int64_t d = int64_t(dblk) * kWave + lane;
  const bool active = d < p.D;
  const int64_t dc = active ? d : p.D - 1;
  const uint32_t lane_c = uint32_t(dc - int64_t(dblk) * kWave);
  const int32_t t0 = int32_t(int64_t(chunk) * p.chunk_len);
  const int32_t t1 = int32_t(t0 + p.chunk_len < p.L ? t0 + p.chunk_len : p.L);
  const int N = p.N;

  Chan<NS> ch;
  bool weak = false;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int n = n0 + j;
    const float a = n < N ? p.A[dc * N + n] : -1.0f;
    ch.A[j] = a;
    ch.iA[j] = a == 0.0f ? 0.0f : 1.0f / a;
    weak |= __builtin_fabsf(a) < kWeakA;
  }

  float h[NS];
  if (SUMMARY) {
#pragma unroll
    for (int j = 0; j < NS; ++j) h[j] = 0.0f;
  } else if (chunk == 0) {
#pragma unroll
    for (int j = 0; j < NS; ++j)
      h[j] = (p.h0 && n0 + j < N) ? p.h0[(b * p.D + dc) * N + n0 + j] : 0.0f;
  } else {
    const float* hs = p.hend + (b * p.nchunks + chunk) * int64_t(N) * p.D + dc;
#pragma unroll
    for (int j = 0; j < NS; ++j) h[j] = n0 + j < N ? hs[int64_t(n0 + j) * p.D] : 0.0f;
  }

  __shared__ float4 lds4[(Lds<NSPLIT>::kFloats + 3) / 4];
  float* lds = reinterpret_cast<float*>(lds4);
  const int64_t base = b * p.L * p.D + (REV ? (p.L - 1) * p.D : 0) + int64_t(dblk) * kWave;
  auto setup = [&](auto& sc) {
    sc.stage = lds + wave * Lds<NSPLIT>::kStage;
    sc.act = lds + NSPLIT * Lds<NSPLIT>::kStage;
    sc.part = sc.act + Lds<NSPLIT>::kAct;
    sc.lane = uint32_t(lane);
    sc.wave = wave;
    sc.n0 = n0;
    sc.Dd = p.Dskip ? p.Dskip[dc] : 0.0f;
    sc.bias2 = (p.bias ? p.bias[dc] : 0.0f) * kLog2e;
    sc.dsum = 0.0f;
    sc.bidx = b;
    sc.td.ts = REV ? -p.D : p.D;
    sc.ub = static_cast<const In*>(p.u) + base;
    sc.db = static_cast<const In*>(p.delta) + base;
    sc.zb = p.z ? static_cast<const In*>(p.z) + base : nullptr;
    sc.yb = SUMMARY ? nullptr : static_cast<Out*>(p.y) + base;
    sc.vin = lane_c * uint32_t(sizeof(In));
    sc.vout = active ? lane_c * uint32_t(sizeof(Out)) : kOutOfRange;
    sc.rowb_in = uint32_t(p.D) * uint32_t(sizeof(In));
    sc.rowb_out = uint32_t(p.D) * uint32_t(sizeof(Out));
    sc.t1 = t1;
    sc.tlast = t1 - 1;
    sc.run(t0);
    return sc.dsum;
  };
  float dsum;
  // The precise decay (precise_decay): always for fp32 inputs, whose bound is
  // elementwise; for bf16 inputs where some state of the wave decays slowly
  // (|A| < kWeakA, A == 0 included; decided per wave, every wave still passes
  // the same barriers).  Other bf16 waves run the fast path.
  if constexpr (std::is_same<In, float>::value) {
    Scan<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, true, NSPLIT, REV> sc{p, ch, h};
    dsum = setup(sc);
  } else if (__any(weak)) {
    Scan<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, true, NSPLIT, REV> sc{p, ch, h};
    dsum = setup(sc);
  } else {
    Scan<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, false, NSPLIT, REV> sc{p, ch, h};
    dsum = setup(sc);
    if (SUMMARY && DISC == kZoh) {
#pragma unroll
      for (int j = 0; j < NS; ++j) h[j] *= ch.iA[j];       // s = A h -> h
    }
  }

  if (!active) return;
  if (SUMMARY) {
    float* hs = p.hend + (b * p.nchunks + chunk) * int64_t(N) * p.D + d;
#pragma unroll
    for (int j = 0; j < NS; ++j)
      if (n0 + j < N) hs[int64_t(n0 + j) * p.D] = h[j];
    if (wave == 0) p.dsum[(b * p.nchunks + chunk) * p.D + d] = dsum;
  } else if (p.h_last && t1 == p.L) {
#pragma unroll
    for (int j = 0; j < NS; ++j)
      if (n0 + j < N) p.h_last[(b * p.D + d) * N + n0 + j] = h[j];
  }
}

template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY, int NSPLIT,
          bool REV = false>
hipError_t launch_one(const FwdParams& p, int64_t nblocks, hipStream_t st) {
  hipLaunchKernelGGL((fwd_kernel<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, NSPLIT, REV>),
                     dim3(unsigned(nblocks)), dim3(kWave * NSPLIT), 0, st, p);
  return hipGetLastError();
}

// The reverse direction runs on the 4-wave layout only (its register use
// leaves room for the mirrored addressing); the chunk plan, and with it the
// workspace, is the forward one.
template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY>
hipError_t dispatch_split(const FwdParams& p, int nsplit, int64_t nblocks, hipStream_t st) {
  if (p.rev) return launch_one<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, 4, true>(p, nblocks, st);
  switch (nsplit) {
    case 4: return launch_one<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, 4>(p, nblocks, st);
    case 2: return launch_one<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, 2>(p, nblocks, st);
    default: return launch_one<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, 1>(p, nblocks, st);
  }
}

template <typename In, typename Out, int DISC>
hipError_t dispatch_flags(const FwdParams& p, int nsplit, bool has_z, bool softplus, bool summary,
                          int64_t nblocks, hipStream_t st) {
  if (summary) {
    // summaries are fp32 state: only the fp32-output instantiation has them
    if constexpr (std::is_same<Out, float>::value)
      return softplus ? dispatch_split<In, Out, DISC, false, true, true>(p, nsplit, nblocks, st)
                      : dispatch_split<In, Out, DISC, false, false, true>(p, nsplit, nblocks, st);
    else
      return hipErrorInvalidValue;
  }
  if (has_z)
    return softplus ? dispatch_split<In, Out, DISC, true, true, false>(p, nsplit, nblocks, st)
                    : dispatch_split<In, Out, DISC, true, false, false>(p, nsplit, nblocks, st);
  return softplus ? dispatch_split<In, Out, DISC, false, true, false>(p, nsplit, nblocks, st)
                  : dispatch_split<In, Out, DISC, false, false, false>(p, nsplit, nblocks, st);
}

template <typename In, typename Out>
hipError_t dispatch_disc(const FwdParams& p, int disc, int nsplit, bool has_z, bool softplus,
                         bool summary, int64_t nblocks, hipStream_t st) {
  return disc == kZoh
             ? dispatch_flags<In, Out, kZoh>(p, nsplit, has_z, softplus, summary, nblocks, st)
             : dispatch_flags<In, Out, kEuler>(p, nsplit, has_z, softplus, summary, nblocks, st);
}

}  // namespace
}  // namespace ss
