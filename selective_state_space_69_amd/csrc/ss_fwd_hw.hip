// Forward selective scan for gfx950, 32-channel workgroups.
//
// Same recurrence and block structure as ss_fwd.hip (8-step blocks, two-deep
// prefetch ring, B/C rows staged in LDS, step sizes and partial sums of C h
// exchanged through LDS once per block), with a different lane mapping: a
// workgroup covers 32 channels and all 16 states with 4 waves; lane l of wave
// w serves channel l % 32 and the two states n = 2o, 2o + 1 of its owner slot
// o = 2w + l / 32.  Each lane owns one step of every block (step o): it loads
// that step's delta, z and u, computes its softplus and gate, publishes the
// step size and u (fp32) to the other lanes of its channel through LDS, and
// later sums the eight owners' partials and stores y.
//
// Why: with two states per lane a problem has twice as many workgroups and
// four times as many waves as with 64 channels and four states per lane.  On
// the Mamba-2.8B shape (B = 8, D = 5120) the 64-channel kernel makes 640
// workgroups for 256 compute units (two or three per unit, so the slowest
// units do 20% more than the mean); here 1280 workgroups give exactly five per
// unit and five waves per SIMD, which also hides more latency.  The work per
// (b, t, d, n) element: one v_exp_f32 and 4 (Euler) or 5.5 (exact ZOH, with the
// scaled states below) other vector ops; about 14 in the precise path ("A Visual
// Guide to Mamba" summary, Hardware-aware Algorithm: discretisation, scan and C
// contraction fused, nothing of size (B, L, D, N) in memory).
#include "ss_fwd_common.hpp"

namespace ss {
namespace {

constexpr int kCh = 32;        // channels per workgroup
constexpr int kOwners = 8;     // 4 waves x 2 halves, each with 2 states
constexpr int kWaves = 4;
// LDS (floats), all double-buffered by block parity:
//   act   [2][8 steps][32 ch] x 2            step size (log2 units) and u
//   stage [2][8 owners][8 steps][4]          B[2o], B[2o+1], C[2o], C[2o+1]
//   part  [2][8 owners][8 steps + 1][32 ch]  partial sums of C h (the padding
//                                            row puts the two halves of a wave
//                                            on different banks)
constexpr int kActF = kBlk * kCh * 2;
constexpr int kStageF = kOwners * kBlk * 4;
constexpr int kPartRow = (kBlk + 1) * kCh;
constexpr int kPartF = kOwners * kPartRow;
constexpr int kLdsF = 2 * (kActF + kStageF + kPartF);

template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY,
          bool PRECISE, bool REV>
struct HalfScan {
  using Raw2 = typename std::conditional<sizeof(In) == 2, uint32_t, uint2>::type;
  // Exact ZOH outside the precise path keeps the lane's two states scaled by
  // A[0]: s = A[0] h.  State 0 then advances as s <- a (s + B u) - B u, one
  // operation fewer than a h + ((a - 1) / A) B u, state 1 as
  // s <- a s + (a - 1) (A[0] / A[1]) B u; the partial C s carries the factor
  // A[0], which the summing lane removes with the 1 / A[0] of the slot that
  // wrote it (an fma in place of the add).  The precise path (fp32 inputs, or
  // a slowly decaying state in the wave) keeps plain states and the decay as
  // E = A_bar - 1 (precise_decay).
  static constexpr bool kScaled = DISC == kZoh && !PRECISE;
  const FwdParams& p;
  float A[2], iA[2];
  float rA1;             // A[0] / A[1] (scaled form)
  float mo[kOwners];     // per owner slot: 1 / A[0] of the slot's lane if scaled, else 1
  float h[2];
  float Dd, bias2;
  float dsum;
  int64_t bidx;          // batch row
  TimeDir<REV> td;
  const In* ub;          // wave-uniform base pointers of (b, logical t = 0, d = 32 * dblk)
  const In* db;
  const In* zb;
  Out* yb;
  const In* brb;         // (b, t = 0) rows of B and C
  const In* crb;
  uint32_t vin;          // c * sizeof(In)
  uint32_t vown;         // vin + o * row bytes: the owned step inside a block
  uint32_t vout;         // c * sizeof(Out) + o * row bytes, out of range for idle lanes
  uint32_t vrow;         // this lane's B/C pair in the staged rows (bytes, step k_row)
  uint32_t rowb_in, rowb_out;
  int32_t t1, tlast;
  int o;                 // owner slot = owned step of every block
  int k_row;             // step whose B/C pair this lane fetches
  uint32_t c;            // channel within the group
  float* act;
  float* stage;
  float* part;
  float* stage_w;        // where this lane writes its staged pair (buffer 0)
  // two-deep prefetch ring, slot = block parity (as in ss_fwd.hip)
  In dr[2], zr[2], uo[2];
  Raw2 rb[2], rc[2];     // B and C pairs of the lane's fetch slot
  float dl_own, g_own, u_own;

  // prefetch of block t into ring slot S: delta, z and u of the owned step,
  // this lane's B/C pair.  Every lane reads u of the other steps from LDS,
  // where the step's owner publishes it (in fp32) with the step size.
  template <typename T>
  __device__ __forceinline__ Rsrc at(const T* base, int32_t t) const {
    return make_rsrc(base + int64_t(td.blk(t)) * td.ts);
  }
  template <int S>
  __device__ __forceinline__ void load_ring(int32_t t, bool clamp) {
    const Rsrc ru = at(ub, t), rd = at(db, t);
    const Rsrc rz = at(HAS_Z ? zb : ub, t);
    const int32_t lim = tlast - t;
    uint32_t vo = vown;
    if (clamp) vo = vin + td.pos(o < lim ? o : lim) * rowb_in;
    dr[S] = buf_load<In>(rd, vo, 0);
    if (HAS_Z && !SUMMARY) zr[S] = buf_load<In>(rz, vo, 0);
    uo[S] = buf_load<In>(ru, vo, 0);
    // B/C pair: step k_row of the block, states 2 * (owner) .. + 1
    const int64_t rw = td.row(bidx, p.L, t);
    const Rsrc rB = make_rsrc(brb + rw * kMaxState);
    const Rsrc rC = make_rsrc(crb + rw * kMaxState);
    uint32_t vr = vrow;
    if (clamp) vr = vrow - td.pos(k_row) * uint32_t(kMaxState * sizeof(In)) +
                    td.pos(k_row < lim ? k_row : lim) * uint32_t(kMaxState * sizeof(In));
    rb[S] = load_pair(rB, vr);
    if (!SUMMARY) rc[S] = load_pair(rC, vr);
  }
  __device__ __forceinline__ Raw2 load_pair(Rsrc r, uint32_t vo) {
    if constexpr (sizeof(In) == 2) {
      return __builtin_amdgcn_raw_buffer_load_b32(r, vo, 0, 0);
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, vo, 0, 0);
      return make_uint2(v[0], v[1]);
    }
  }
  __device__ __forceinline__ float2 unpack_pair(Raw2 w) const {
    if constexpr (sizeof(In) == 2)
      return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
    else
      return make_float2(__uint_as_float(w.x), __uint_as_float(w.y));
  }

  // step size (log2 units), gate and u of the owned step of the block at t
  template <int S, bool GUARD>
  __device__ __forceinline__ void activations(int32_t t) {
    float x2 = __builtin_fmaf(to_f32(dr[S]), kLog2e, bias2);   // (delta + bias) log2 e
    if (GUARD && t + o >= t1) x2 = SOFTPLUS ? -__builtin_inff() : 0.0f;
    dl_own = SOFTPLUS ? softplus_log2(x2) : x2;                 // dt * log2 e
    if (HAS_Z && !SUMMARY) g_own = silu(to_f32(zr[S]));
    u_own = to_f32(uo[S]);
    if (GUARD && t + o >= t1) u_own = 0.0f;                     // padded step: inert
  }
  template <int S>
  __device__ __forceinline__ void publish() {
    // Euler uses u only as dt u = (dt log2 e) (u ln 2): the ln 2 is applied here, once per step
    reinterpret_cast<float2*>(act + S * kActF)[o * kCh + c] =
        make_float2(dl_own, DISC == kEuler ? u_own * kLn2 : u_own);
    const float2 b2 = unpack_pair(rb[S]);
    const float2 c2 = SUMMARY ? make_float2(0.0f, 0.0f) : unpack_pair(rc[S]);
    *reinterpret_cast<float4*>(stage_w + S * kStageF) = make_float4(b2.x, b2.y, c2.x, c2.y);
  }

  // One block of 8 steps at t, parity S.  On entry the LDS buffer S holds the
  // block's step sizes and rows (behind a barrier) and the owned-step
  // activations are computed.
  template <bool GUARD, int S>
  __device__ __forceinline__ void block(int32_t t) {
    const float g = g_own, us = u_own;
    // prefetch block t + 16 into slot S: owned-step inputs and rows
    const int32_t tn0 = t + 2 * kBlk;
    const int32_t tn = tn0 < tlast ? tn0 : tlast;
    load_ring<S>(tn, GUARD);
    const float4* rows = reinterpret_cast<const float4*>(stage + S * kStageF + o * kBlk * 4);
    const float2* dls = reinterpret_cast<const float2*>(act + S * kActF) + c;   // (dt log2 e, u)
    float* parts = part + S * kPartF + o * kPartRow + c;
    float4 rn = rows[0];
    float2 dn = dls[0];
#pragma unroll
    for (int k = 0; k < kBlk; ++k) {
      const float4 r = rn;                         // B[2o], B[2o+1], C[2o], C[2o+1]
      const float d2 = dn.x;                       // dt * log2 e
      const float uk = dn.y;                       // u (Euler: u ln 2)
      if (k + 1 < kBlk) {
        rn = rows[k + 1];
        dn = dls[(k + 1) * kCh];
      }
      if (PRECISE) {
        // h <- h + (E h + coef B u), E = A_bar - 1 and coef to full relative accuracy
        float q0 = 0.0f, q1 = 0.0f;
        const float e0 = precise_decay<DISC == kZoh>(d2, A[0], iA[0], q0);
        const float e1 = precise_decay<DISC == kZoh>(d2, A[1], iA[1], q1);
        const float in0 = DISC == kEuler ? (d2 * uk) * r.x : q0 * (r.x * uk);   // Euler: dt u B
        const float in1 = DISC == kEuler ? (d2 * uk) * r.y : q1 * (r.y * uk);
        h[0] += __builtin_fmaf(e0, h[0], in0);
        h[1] += __builtin_fmaf(e1, h[1], in1);
      } else {
        const float a0 = hw_exp2(d2 * A[0]), a1 = hw_exp2(d2 * A[1]);   // A_bar = exp(dt A)
        if (DISC == kEuler) {
          const float dtu = d2 * uk;                                // dt * u
          h[0] = __builtin_fmaf(a0, h[0], dtu * r.x);
          h[1] = __builtin_fmaf(a1, h[1], dtu * r.y);
        } else {
          // scaled states (s = A[0] h)
          const float bu0 = r.x * uk, bu1 = r.y * uk;
          const float q1 = __builtin_fmaf(a1, rA1, -rA1);           // (A_bar - 1) A[0] / A[1]
          h[0] = __builtin_fmaf(a0, h[0] + bu0, -bu0);
          h[1] = __builtin_fmaf(a1, h[1], q1 * bu1);
        }
      }
      if (SUMMARY) dsum += d2;
      else parts[k * kCh] = __builtin_fmaf(r.w, h[1], r.z * h[0]);   // partial C h (x A[0] if scaled)
    }
    // activations, step sizes and rows of block t + 8 (slot S^1)
    activations<S ^ 1, GUARD>(t + kBlk);
    publish<S ^ 1>();
    __syncthreads();
    if (SUMMARY) return;
    // output of the owned step: the eight owners' partials, skip, gate, store
    float yv = 0.0f;
#pragma unroll
    for (int w = 0; w < kOwners; ++w) {
      const float pw = part[S * kPartF + w * kPartRow + o * kCh + c];
      if (DISC == kZoh) yv = __builtin_fmaf(mo[w], pw, yv);
      else yv += pw;
    }
    yv = __builtin_fmaf(Dd, us, yv);                                 // + D skip
    if (HAS_Z) yv *= g;                                              // silu(z) gate
    if (!GUARD || t + o < t1) {
      const Rsrc ry = at(yb, t);
      if (p.acc) yv += to_f32(buf_load<Out>(ry, vout, 0));
      buf_store<Out>(ry, vout, 0, yv);
    }
  }

  __device__ __forceinline__ void run(int32_t t0) {
    const int32_t t8 = t0 + kBlk < tlast ? t0 + kBlk : tlast;
    load_ring<0>(t0, true);
    load_ring<1>(t8, true);
    activations<0, true>(t0);
    publish<0>();
    __syncthreads();
    int32_t t = t0;
    for (; t + 4 * kBlk <= t1; t += 2 * kBlk) {
      block<false, 0>(t);
      block<false, 1>(t + kBlk);
    }
    for (; t < t1; t += 2 * kBlk) {
      block<true, 0>(t);
      if (t + kBlk < t1) block<true, 1>(t + kBlk);
    }
  }
};

template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY, bool REV>
// five waves per SIMD: five workgroups per compute unit
__global__ __launch_bounds__(kWave * kWaves, 5) void fwd_hw_kernel(FwdParams p) {
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const int lane = int(threadIdx.x) % kWave;
  const int half = lane / kCh;
  const int o = 2 * wave + half;
  const uint32_t c = uint32_t(lane % kCh);
  const int n0 = 2 * o;
  // Two neighbouring 32-channel groups share every 128-byte line of u, delta
  // and z: with each XCD on a contiguous range of groups both halves of a line
  // are fetched through the same L2.
  int64_t bid = xcd_contiguous(blockIdx.x, gridDim.x);
  const int dblk = int(bid % p.ndblk);
  bid /= p.ndblk;
  const int chunk = int(bid % p.grid_chunks);
  const int64_t b = bid / p.grid_chunks;
  const int64_t d = int64_t(dblk) * kCh + c;
  const bool active = d < p.D;
  const int64_t dc = active ? d : p.D - 1;
  const uint32_t c_c = uint32_t(dc - int64_t(dblk) * kCh);
  const int32_t t0 = int32_t(int64_t(chunk) * p.chunk_len);
  const int32_t t1 = int32_t(t0 + p.chunk_len < p.L ? t0 + p.chunk_len : p.L);
  const int N = p.N;

  __shared__ float4 lds4[kLdsF / 4];
  float* lds = reinterpret_cast<float*>(lds4);
  const int64_t base = b * p.L * p.D + (REV ? (p.L - 1) * p.D : 0) + int64_t(dblk) * kCh;

  float Av[2];
  bool weak = false;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    Av[j] = n0 + j < N ? p.A[dc * N + n0 + j] : -1.0f;   // unused states: inert
    weak |= __builtin_fabsf(Av[j]) < kWeakA;
  }
  float hs[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (SUMMARY || n0 + j >= N) hs[j] = 0.0f;
    else if (chunk == 0) hs[j] = p.h0 ? p.h0[(b * p.D + dc) * N + n0 + j] : 0.0f;
    else hs[j] = p.hend[((b * p.nchunks + chunk) * N + n0 + j) * p.D + dc];
  }

  float dsum = 0.0f;
  auto go = [&](auto& sc) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      sc.A[j] = Av[j];
      sc.iA[j] = Av[j] == 0.0f ? 0.0f : 1.0f / Av[j];
      sc.h[j] = hs[j];
    }
    sc.Dd = p.Dskip ? p.Dskip[dc] : 0.0f;
    sc.bias2 = (p.bias ? p.bias[dc] : 0.0f) * kLog2e;
    sc.dsum = 0.0f;
    sc.bidx = b;
    sc.td.ts = REV ? -p.D : p.D;
    sc.ub = static_cast<const In*>(p.u) + base;
    sc.db = static_cast<const In*>(p.delta) + base;
    sc.zb = p.z ? static_cast<const In*>(p.z) + base : nullptr;
    sc.yb = SUMMARY ? nullptr : static_cast<Out*>(p.y) + base;
    sc.brb = static_cast<const In*>(p.Brow);
    sc.crb = static_cast<const In*>(p.Crow);
    sc.rowb_in = uint32_t(p.D) * uint32_t(sizeof(In));
    sc.rowb_out = uint32_t(p.D) * uint32_t(sizeof(Out));
    sc.vin = c_c * uint32_t(sizeof(In));
    sc.vown = sc.vin + sc.td.pos(o) * sc.rowb_in;
    sc.vout = active ? c_c * uint32_t(sizeof(Out)) + sc.td.pos(o) * sc.rowb_out : kOutOfRange;
    // fetch slot of this lane: step k_row = l % 8 of the block, owner 2w + (l / 8) % 2
    // (lanes 16..63 repeat lanes 0..15)
    sc.k_row = lane % kBlk;
    const int fo = 2 * wave + (lane / kBlk) % 2;
    sc.vrow = (sc.td.pos(sc.k_row) * kMaxState + 2 * fo) * uint32_t(sizeof(In));
    sc.t1 = t1;
    sc.tlast = t1 - 1;
    sc.o = o;
    sc.c = c;
    sc.act = lds;
    sc.stage = lds + 2 * kActF;
    sc.part = sc.stage + 2 * kStageF;
    sc.stage_w = sc.stage + (fo * kBlk + sc.k_row) * 4;
    constexpr bool scaled = std::decay_t<decltype(sc)>::kScaled;
    if (scaled) {
      sc.rA1 = Av[0] * sc.iA[1];
      sc.h[0] *= Av[0];
      sc.h[1] *= Av[0];
    }
    if (DISC == kZoh && !SUMMARY) {
      // owner multipliers through the (not yet used) partial-sum buffer
      sc.part[o * kPartRow + c] = scaled ? sc.iA[0] : 1.0f;   // 1 in a precise wave
      __syncthreads();
#pragma unroll
      for (int w = 0; w < kOwners; ++w) sc.mo[w] = sc.part[w * kPartRow + c];
    }
    sc.run(t0);
    dsum = sc.dsum;
    hs[0] = scaled ? sc.h[0] * sc.iA[0] : sc.h[0];
    hs[1] = scaled ? sc.h[1] * sc.iA[0] : sc.h[1];
  };
  // The precise path: always for fp32 inputs (their bound is elementwise), and
  // for bf16 inputs where some state of the wave decays slowly (|A| < kWeakA,
  // A == 0 included; decided per wave, every wave still passes the same
  // barriers).  bf16 waves whose states all have |A| >= kWeakA run the fast
  // path: their memory is at most 4 / dt steps, and the decay's rounding stays
  // far inside the bf16 bound.
  if constexpr (std::is_same<In, float>::value) {
    HalfScan<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, true, REV> sc{p};
    go(sc);
  } else if (__any(weak)) {
    HalfScan<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, true, REV> sc{p};
    go(sc);
  } else {
    HalfScan<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, false, REV> sc{p};
    go(sc);
  }

  if (!active) return;
  if (SUMMARY) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (n0 + j < N) p.hend[((b * p.nchunks + chunk) * N + n0 + j) * p.D + d] = hs[j];
    if (o == 0) p.dsum[(b * p.nchunks + chunk) * p.D + d] = dsum;
  } else if (p.h_last && t1 == p.L) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (n0 + j < N) p.h_last[(b * p.D + d) * N + n0 + j] = hs[j];
  }
}

template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY>
hipError_t launch_one(const FwdParams& p, int64_t nblocks, hipStream_t st) {
  if (p.rev)
    hipLaunchKernelGGL((fwd_hw_kernel<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, true>),
                       dim3(unsigned(nblocks)), dim3(kWave * kWaves), 0, st, p);
  else
    hipLaunchKernelGGL((fwd_hw_kernel<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, false>),
                       dim3(unsigned(nblocks)), dim3(kWave * kWaves), 0, st, p);
  return hipGetLastError();
}

template <typename In, typename Out, int DISC>
hipError_t dispatch_flags(const FwdParams& p, bool has_z, bool softplus, bool summary,
                          int64_t nblocks, hipStream_t st) {
  if (summary) {
    return softplus ? launch_one<In, Out, DISC, false, true, true>(p, nblocks, st)
                    : launch_one<In, Out, DISC, false, false, true>(p, nblocks, st);
  }
  if (has_z)
    return softplus ? launch_one<In, Out, DISC, true, true, false>(p, nblocks, st)
                    : launch_one<In, Out, DISC, true, false, false>(p, nblocks, st);
  return softplus ? launch_one<In, Out, DISC, false, true, false>(p, nblocks, st)
                  : launch_one<In, Out, DISC, false, false, false>(p, nblocks, st);
}

template <typename In, typename Out>
hipError_t dispatch_disc(const FwdParams& p, int disc, bool has_z, bool softplus, bool summary,
                         int64_t nblocks, hipStream_t st) {
  return disc == kZoh ? dispatch_flags<In, Out, kZoh>(p, has_z, softplus, summary, nblocks, st)
                      : dispatch_flags<In, Out, kEuler>(p, has_z, softplus, summary, nblocks, st);
}

}  // namespace

hipError_t launch_fwd_hw(const ss_desc_t& d, const FwdParams& p, bool summary, int64_t nblocks,
                         hipStream_t st) {
  const bool has_z = p.z != nullptr, sp = d.delta_softplus != 0;
  if (d.in_dtype == SS_BF16) {
    if (summary || d.out_dtype == SS_F32)
      return dispatch_disc<uint16_t, float>(p, d.disc, has_z, sp, summary, nblocks, st);
    return dispatch_disc<uint16_t, uint16_t>(p, d.disc, has_z, sp, false, nblocks, st);
  }
  if (summary || d.out_dtype == SS_F32)
    return dispatch_disc<float, float>(p, d.disc, has_z, sp, summary, nblocks, st);
  return dispatch_disc<float, uint16_t>(p, d.disc, has_z, sp, false, nblocks, st);
}

}  // namespace ss
