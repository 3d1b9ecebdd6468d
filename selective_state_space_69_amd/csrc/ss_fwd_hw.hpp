// Forward selective scan for gfx950 with the states of a channel spread over
// the lanes: SPL (2 or 1) states per lane, 16 / SPL owner slots per channel.
//
// Same recurrence and block structure as the 64-channel kernel
// (ss_fwd_kernels.hpp: a two-deep prefetch ring, B/C rows staged in LDS, step
// sizes and partial sums of C h exchanged through LDS once per block), with a
// different lane mapping: a workgroup of 4 waves
// covers kCh = 256 SPL / 16 channels (32 or 16) and all 16 states; lane l of
// wave w serves channel l % kCh and the SPL states n = SPL o .. SPL o + SPL - 1
// of its owner slot o = (64 / kCh) w + l / kCh.  A block has one step per
// owner slot (8 or 16 steps), and each lane owns step o of every block: it
// loads that step's delta, z and u, computes its softplus and gate, publishes
// the step size and u (fp32) to the other lanes of its channel through LDS,
// and later sums the owners' partials and stores y.
//
// Why: spreading the states over more lanes gives a problem more waves.  With
// two states per lane the Mamba-2.8B shape (B = 8, D = 5120) makes 1280
// workgroups, exactly five per compute unit and five waves per SIMD (the
// 64-channel kernel makes 640, two or three per unit, so the slowest units do
// 20% more than the mean).  Narrower problems (Mamba-130M: B = 8, D = 1536; or
// B = 2 at D = 5120) would leave a SIMD with one or two waves, which stall on
// transcendental and LDS latency; one state per lane doubles the waves again
// (three per SIMD at B = 8, D = 1536), so that they run in one pass instead of
// in time chunks, which cost a second pass over the recurrence.  The work per
// (b, t, d, n) element: one v_exp_f32 and 4 (Euler) or 5.5 (exact ZOH, with the
// scaled states below) other vector ops; about 14 in the precise path ("A Visual
// Guide to Mamba" summary, Hardware-aware Algorithm: discretisation, scan and C
// contraction fused, nothing of size (B, L, D, N) in memory).
#pragma once

#include <type_traits>

#include "ss_fwd_common.hpp"

namespace ss {
namespace {

template <int SPL>
struct HwLayout {
  static_assert(SPL == 1 || SPL == 2, "one or two states per lane");
  static constexpr int kWaves = 4;
  static constexpr int kOwners = kMaxState / SPL;        // owner slots per channel
  static constexpr int kSteps = kOwners;                 // steps per block: one per owner
  static constexpr int kCh = kWaves * kWave / kOwners;   // channels per workgroup
  static constexpr int kOwnersPerWave = kWave / kCh;
  // LDS (floats), all double-buffered by block parity.  The layouts put what
  // one lane reads next to each other, so that a 16-byte read covers two steps
  // of act (and of stage with one state per lane), and part is read four (one
  // state) or two (two states) owners at a time:
  //   act   [2][ch][steps x 2 + 4]         (dt log2 e, u) of step k at 2 k
  //   stage [2][owners][steps][2 SPL]      B of the owner's states, then C
  //   part  [2][ch][steps][owners] + pad   partial C h of owner w for step k
  // The paddings spread the channels one access touches over all 64 banks
  // (16 channels a wave: 4 floats; 32: 2, which keeps the part rows 8-byte
  // aligned).  Against a [steps][ch] layout read one step at a time this
  // halves the LDS instructions of the 32-channel kernel's loop and takes 4%
  // off its time (Mamba-2.8B shape).
  static constexpr int kActStride = kSteps * 2 + 4;
  static constexpr int kPartStride = kSteps * kOwners + (SPL == 1 ? 4 : 2);
  static constexpr int kActF = kCh * kActStride;
  static constexpr int kStageF = kOwners * kSteps * 2 * SPL;
  static constexpr int kPartF = kCh * kPartStride;
  static constexpr int kLdsF = 2 * (kActF + kStageF + kPartF);
};

template <int SPL, typename In> struct HwRaw;
template <> struct HwRaw<2, uint16_t> { using type = uint32_t; };
template <> struct HwRaw<2, float> { using type = uint2; };
template <> struct HwRaw<1, uint16_t> { using type = uint32_t; };
template <> struct HwRaw<1, float> { using type = uint32_t; };

template <int SPL, typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY,
          bool PRECISE, bool REV>
struct HwScan {
  using Lay = HwLayout<SPL>;
  static constexpr int kOwners = Lay::kOwners;
  static constexpr int kSteps = Lay::kSteps;
  static constexpr int kCh = Lay::kCh;
  using Raw = typename HwRaw<SPL, In>::type;
  // Exact ZOH outside the precise path keeps the lane's states scaled by
  // A[0]: s = A[0] h.  State 0 then advances as s <- a (s + B u) - B u, one
  // operation fewer than a h + ((a - 1) / A) B u, state 1 as
  // s <- a s + (a - 1) (A[0] / A[1]) B u; the partial C s carries the factor
  // A[0], which the summing lane removes with the 1 / A[0] of the slot that
  // wrote it (an fma in place of the add).  The precise path (fp32 inputs, or
  // a slowly decaying state in the wave) keeps plain states and the decay as
  // E = A_bar - 1 (precise_decay).
  static constexpr bool kScaled = DISC == kZoh && !PRECISE;
  const FwdParams& p;
  float A[SPL], iA[SPL];
  float rA1;             // A[0] / A[1] (scaled form, two states)
  float mo[kOwners];     // per owner slot: 1 / A[0] of the slot's lane if scaled, else 1
  float h[SPL];
  float Dd, bias2;
  float dsum;
  int64_t bidx;          // batch row
  TimeDir<REV, kSteps> td;
  const In* ub;          // wave-uniform base pointers of (b, logical t = 0, d = kCh * dblk)
  const In* db;
  const In* zb;
  Out* yb;
  const In* brb;         // (b, t = 0) rows of B and C
  const In* crb;
  uint32_t vin;          // c * sizeof(In)
  uint32_t vown;         // vin + o * row bytes: the owned step inside a block
  uint32_t vout;         // c * sizeof(Out) + o * row bytes, out of range for idle lanes
  uint32_t vrow;         // this lane's B/C values in the staged rows (bytes, step k_row)
  uint32_t rowb_in, rowb_out;
  int32_t t1, tlast;
  int o;                 // owner slot = owned step of every block
  int k_row;             // step whose B/C values this lane fetches
  uint32_t c;            // channel within the group
  float* act;
  float* stage;
  float* part;
  float* stage_w;        // where this lane writes its staged values (buffer 0)
  // two-deep prefetch ring, slot = block parity (as in ss_fwd_kernels.hpp)
  In dr[2], zr[2], uo[2];
  Raw rb[2], rc[2];      // B and C values of the lane's fetch slot
  float dl_own, g_own, u_own;

  // prefetch of block t into ring slot S: delta, z and u of the owned step,
  // this lane's B/C values.  Every lane reads u of the other steps from LDS,
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
    // B/C values: step k_row of the block, states SPL * (owner) ..
    const int64_t rw = td.row(bidx, p.L, t);
    const Rsrc rB = make_rsrc(brb + rw * kMaxState);
    const Rsrc rC = make_rsrc(crb + rw * kMaxState);
    uint32_t vr = vrow;
    if (clamp) vr = vrow - td.pos(k_row) * uint32_t(kMaxState * sizeof(In)) +
                    td.pos(k_row < lim ? k_row : lim) * uint32_t(kMaxState * sizeof(In));
    rb[S] = load_vals(rB, vr);
    if (!SUMMARY) rc[S] = load_vals(rC, vr);
  }
  __device__ __forceinline__ Raw load_vals(Rsrc r, uint32_t vo) {
    if constexpr (SPL == 1 && sizeof(In) == 2) {
      return uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, vo, 0, 0));
    } else if constexpr (sizeof(In) == 2 || SPL == 1) {
      return __builtin_amdgcn_raw_buffer_load_b32(r, vo, 0, 0);
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, vo, 0, 0);
      return make_uint2(v[0], v[1]);
    }
  }
  // the SPL values of a fetch as fp32 (x, y for two states; x for one)
  __device__ __forceinline__ float2 unpack_vals(Raw w) const {
    if constexpr (SPL == 1) {
      return make_float2(sizeof(In) == 2 ? __uint_as_float(w << 16) : __uint_as_float(w), 0.0f);
    } else if constexpr (sizeof(In) == 2) {
      return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
    } else {
      return make_float2(__uint_as_float(w.x), __uint_as_float(w.y));
    }
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
    *reinterpret_cast<float2*>(act + S * Lay::kActF + c * Lay::kActStride + 2 * o) =
        make_float2(dl_own, DISC == kEuler ? u_own * kLn2 : u_own);
    const float2 b2 = unpack_vals(rb[S]);
    const float2 c2 = SUMMARY ? make_float2(0.0f, 0.0f) : unpack_vals(rc[S]);
    if constexpr (SPL == 2)
      *reinterpret_cast<float4*>(stage_w + S * Lay::kStageF) = make_float4(b2.x, b2.y, c2.x, c2.y);
    else
      *reinterpret_cast<float2*>(stage_w + S * Lay::kStageF) = make_float2(b2.x, c2.x);
  }

  // One block of kSteps steps at t, parity S.  On entry the LDS buffer S holds
  // the block's step sizes and rows (behind a barrier) and the owned-step
  // activations are computed.
  template <bool GUARD, int S>
  __device__ __forceinline__ void block(int32_t t) {
    const float g = g_own, us = u_own;
    // prefetch block t + 2 kSteps into slot S: owned-step inputs and rows
    const int32_t tn0 = t + 2 * kSteps;
    const int32_t tn = tn0 < tlast ? tn0 : tlast;
    load_ring<S>(tn, GUARD);
    steps<S>();
    // activations, step sizes and rows of block t + kSteps (slot S^1)
    activations<S ^ 1, GUARD>(t + kSteps);
    publish<S ^ 1>();
    __syncthreads();
    if (SUMMARY) return;
    // output of the owned step: the owners' partials, skip, gate, store
    float yv = 0.0f;
    const float* pr = part + S * Lay::kPartF + c * Lay::kPartStride + o * kOwners;
    if constexpr (SPL == 1) {
#pragma unroll
      for (int q = 0; q < kOwners / 4; ++q) {
        const float4 pw = reinterpret_cast<const float4*>(pr)[q];
        if (DISC == kZoh) {
          yv = __builtin_fmaf(mo[4 * q], pw.x, yv);
          yv = __builtin_fmaf(mo[4 * q + 1], pw.y, yv);
          yv = __builtin_fmaf(mo[4 * q + 2], pw.z, yv);
          yv = __builtin_fmaf(mo[4 * q + 3], pw.w, yv);
        } else {
          yv += pw.x;
          yv += pw.y;
          yv += pw.z;
          yv += pw.w;
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < kOwners / 2; ++q) {
        const float2 pw = reinterpret_cast<const float2*>(pr)[q];
        if (DISC == kZoh) {
          yv = __builtin_fmaf(mo[2 * q], pw.x, yv);
          yv = __builtin_fmaf(mo[2 * q + 1], pw.y, yv);
        } else {
          yv += pw.x;
          yv += pw.y;
        }
      }
    }
    yv = __builtin_fmaf(Dd, us, yv);                                 // + D skip
    if (HAS_Z) yv *= g;                                              // silu(z) gate
    if (!GUARD || t + o < t1) {
      const Rsrc ry = at(yb, t);
      if (p.acc) yv += to_f32(buf_load<Out>(ry, vout, 0));
      buf_store<Out>(ry, vout, 0, yv);
    }
  }

  // one step of the lane's states: step size d2 (log2 units), u (Euler: u ln 2),
  // the states' B and C; the partial C h (x A[0] if scaled) is returned
  __device__ __forceinline__ float step(float d2, float uk, const float (&Bv)[SPL],
                                        const float (&Cv)[SPL]) {
    if (PRECISE) {
      // h <- h + (E h + coef B u), E = A_bar - 1 and coef to full relative accuracy
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        float q = 0.0f;
        const float e = precise_decay<DISC == kZoh>(d2, A[j], iA[j], q);
        const float in = DISC == kEuler ? (d2 * uk) * Bv[j] : q * (Bv[j] * uk);   // Euler: dt u B
        h[j] += __builtin_fmaf(e, h[j], in);
      }
    } else {
      float a[SPL];
#pragma unroll
      for (int j = 0; j < SPL; ++j) a[j] = hw_exp2(d2 * A[j]);    // A_bar = exp(dt A)
      if (DISC == kEuler) {
        const float dtu = d2 * uk;                                 // dt * u
#pragma unroll
        for (int j = 0; j < SPL; ++j) h[j] = __builtin_fmaf(a[j], h[j], dtu * Bv[j]);
      } else {
        // scaled states (s = A[0] h)
        const float bu0 = Bv[0] * uk;
        if constexpr (SPL == 2) {
          const float bu1 = Bv[1] * uk;
          const float q1 = __builtin_fmaf(a[1], rA1, -rA1);        // (A_bar - 1) A[0] / A[1]
          h[0] = __builtin_fmaf(a[0], h[0] + bu0, -bu0);
          h[1] = __builtin_fmaf(a[1], h[1], q1 * bu1);
        } else {
          h[0] = __builtin_fmaf(a[0], h[0] + bu0, -bu0);
        }
      }
    }
    if (SUMMARY) {
      dsum += d2;
      return 0.0f;
    }
    float pc = Cv[0] * h[0];
    if constexpr (SPL == 2) pc = __builtin_fmaf(Cv[1], h[1], pc);
    return pc;
  }

  // the block's steps: two steps per 16-byte read of act (and of stage with
  // one state per lane); partial of step k to part[c][k][o]
  template <int S>
  __device__ __forceinline__ void steps() {
    const float4* rows = reinterpret_cast<const float4*>(stage + S * Lay::kStageF + o * kSteps * 2 * SPL);
    const float4* dls = reinterpret_cast<const float4*>(act + S * Lay::kActF + c * Lay::kActStride);
    float* parts = part + S * Lay::kPartF + c * Lay::kPartStride + o;
    float4 dn = dls[0];
    if constexpr (SPL == 1) {
      // (B, C) of steps k, k + 1 in one read
      float4 rn = rows[0];
#pragma unroll
      for (int k = 0; k < kSteps; k += 2) {
        const float4 r = rn, dd = dn;
        if (k + 2 < kSteps) {
          rn = rows[k / 2 + 1];
          dn = dls[k / 2 + 1];
        }
        {
          const float Bv[1] = {r.x}, Cv[1] = {r.y};
          const float pc = step(dd.x, dd.y, Bv, Cv);
          if (!SUMMARY) parts[k * kOwners] = pc;
        }
        {
          const float Bv[1] = {r.z}, Cv[1] = {r.w};
          const float pc = step(dd.z, dd.w, Bv, Cv);
          if (!SUMMARY) parts[(k + 1) * kOwners] = pc;
        }
      }
    } else {
      // (B0, B1, C0, C1) of steps k and k + 1 in two reads
      float4 rn[2] = {rows[0], rows[1]};
#pragma unroll
      for (int k = 0; k < kSteps; k += 2) {
        const float4 dd = dn, r0 = rn[0], r1 = rn[1];
        if (k + 2 < kSteps) {
          dn = dls[k / 2 + 1];
          rn[0] = rows[k + 2];
          rn[1] = rows[k + 3];
        }
        const float B0[SPL] = {r0.x, r0.y}, C0[SPL] = {r0.z, r0.w};
        const float B1[SPL] = {r1.x, r1.y}, C1[SPL] = {r1.z, r1.w};
        const float pc0 = step(dd.x, dd.y, B0, C0);
        const float pc1 = step(dd.z, dd.w, B1, C1);
        if (!SUMMARY) {
          parts[k * kOwners] = pc0;
          parts[(k + 1) * kOwners] = pc1;
        }
      }
    }
  }

  __device__ __forceinline__ void run(int32_t t0) {
    const int32_t t8 = t0 + kSteps < tlast ? t0 + kSteps : tlast;
    load_ring<0>(t0, true);
    load_ring<1>(t8, true);
    activations<0, true>(t0);
    publish<0>();
    __syncthreads();
    int32_t t = t0;
    for (; t + 4 * kSteps <= t1; t += 2 * kSteps) {
      block<false, 0>(t);
      block<false, 1>(t + kSteps);
    }
    for (; t < t1; t += 2 * kSteps) {
      block<true, 0>(t);
      if (t + kSteps < t1) block<true, 1>(t + kSteps);
    }
  }
};

// The kernel body for SPL states per lane; the __global__ wrappers carry the
// launch bounds of each layout.
template <int SPL, typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY,
          bool REV>
__device__ __forceinline__ void fwd_hw_body(const FwdParams& p) {
  using Lay = HwLayout<SPL>;
  constexpr int kCh = Lay::kCh, kSteps = Lay::kSteps, kOwners = Lay::kOwners;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const int lane = int(threadIdx.x) % kWave;
  const int o = Lay::kOwnersPerWave * wave + lane / kCh;
  const uint32_t c = uint32_t(lane % kCh);
  const int n0 = SPL * o;
  // Neighbouring channel groups share every 128-byte line of u, delta and z:
  // with each XCD on a contiguous range of groups the parts of a line are
  // fetched through the same L2.
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

  __shared__ float4 lds4[Lay::kLdsF / 4];
  float* lds = reinterpret_cast<float*>(lds4);
  const int64_t base = b * p.L * p.D + (REV ? (p.L - 1) * p.D : 0) + int64_t(dblk) * kCh;

  float Av[SPL];
  bool weak = false;
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    Av[j] = n0 + j < N ? p.A[dc * N + n0 + j] : -1.0f;   // unused states: inert
    weak |= __builtin_fabsf(Av[j]) < kWeakA;
  }
  float hs[SPL];
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    if (SUMMARY || n0 + j >= N) hs[j] = 0.0f;
    else if (chunk == 0) hs[j] = p.h0 ? p.h0[(b * p.D + dc) * N + n0 + j] : 0.0f;
    else hs[j] = p.hend[((b * p.nchunks + chunk) * N + n0 + j) * p.D + dc];
  }

  float dsum = 0.0f;
  auto go = [&](auto& sc) {
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
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
    // fetch slot of this lane: step k_row = l % kSteps of the block, owner
    // slot (64 / kCh) w + (l / kSteps) % (64 / kCh) (two states per lane:
    // lanes 16..63 repeat lanes 0..15)
    sc.k_row = lane % kSteps;
    const int fo = Lay::kOwnersPerWave * wave + (lane / kSteps) % Lay::kOwnersPerWave;
    sc.vrow = (sc.td.pos(sc.k_row) * kMaxState + SPL * fo) * uint32_t(sizeof(In));
    sc.t1 = t1;
    sc.tlast = t1 - 1;
    sc.o = o;
    sc.c = c;
    sc.act = lds;
    sc.stage = lds + 2 * Lay::kActF;
    sc.part = sc.stage + 2 * Lay::kStageF;
    sc.stage_w = sc.stage + (fo * kSteps + sc.k_row) * 2 * SPL;
    constexpr bool scaled = std::decay_t<decltype(sc)>::kScaled;
    if (scaled) {
      if constexpr (SPL == 2) sc.rA1 = Av[0] * sc.iA[1];
#pragma unroll
      for (int j = 0; j < SPL; ++j) sc.h[j] *= Av[0];
    }
    if (DISC == kZoh && !SUMMARY) {
      // owner multipliers through the (not yet used) partial-sum buffer
      sc.part[int(c) * Lay::kPartStride + o] = scaled ? sc.iA[0] : 1.0f;   // 1 in a precise wave
      __syncthreads();
#pragma unroll
      for (int w = 0; w < kOwners; ++w) sc.mo[w] = sc.part[int(c) * Lay::kPartStride + w];
    }
    sc.run(t0);
    dsum = sc.dsum;
#pragma unroll
    for (int j = 0; j < SPL; ++j) hs[j] = scaled ? sc.h[j] * sc.iA[0] : sc.h[j];
  };
  // The precise path: always for fp32 inputs (their bound is elementwise), and
  // for bf16 inputs where some state of the wave decays slowly (|A| < kWeakA,
  // A == 0 included; decided per wave, every wave still passes the same
  // barriers).  bf16 waves whose states all have |A| >= kWeakA run the fast
  // path: their memory is at most 4 / dt steps, and the decay's rounding stays
  // far inside the bf16 bound.
  if constexpr (std::is_same<In, float>::value) {
    HwScan<SPL, In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, true, REV> sc{p};
    go(sc);
  } else if (__any(weak)) {
    HwScan<SPL, In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, true, REV> sc{p};
    go(sc);
  } else {
    HwScan<SPL, In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, false, REV> sc{p};
    go(sc);
  }

  if (!active) return;
  if (SUMMARY) {
#pragma unroll
    for (int j = 0; j < SPL; ++j)
      if (n0 + j < N) p.hend[((b * p.nchunks + chunk) * N + n0 + j) * p.D + d] = hs[j];
    if (o == 0) p.dsum[(b * p.nchunks + chunk) * p.D + d] = dsum;
  } else if (p.h_last && t1 == p.L) {
#pragma unroll
    for (int j = 0; j < SPL; ++j)
      if (n0 + j < N) p.h_last[(b * p.D + d) * N + n0 + j] = hs[j];
  }
  (void)kSteps;
}

}  // namespace
}  // namespace ss
