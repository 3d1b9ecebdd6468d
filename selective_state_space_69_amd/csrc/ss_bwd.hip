// Backward selective scan for gfx950, with recomputation.
//
// The states are never stored in memory: they are rebuilt from the inputs
// ("A Visual Guide to Mamba" summary, Hardware-aware Algorithm: recomputation;
// "A Survey of Mamba" summary, hardware-aware computation).  Time is cut into
// chunks of 32 steps.  Per chunk:
//   - one summary pass gives its zero-start end state and its local adjoint
//     (what it sends back to the chunk before it with nothing entering from
//     its end);
//   - carry scans turn those into its true start state and the adjoint carry
//     entering it from its end (ss_carry.hip; the adjoint recurrence
//     lambda_t = gy_t C_t + A_bar_{t+1} lambda_{t+1} is the same linear scan run
//     backwards in time);
//   - a workgroup of 4 waves (lane = channel d, 4 states per wave) stages the
//     chunk's step sizes, gated output gradients, inputs and B/C rows in LDS,
//     runs the chunk forward keeping one state checkpoint per 4-step block in
//     registers, then walks the blocks backwards: recompute the block (A_bar
//     and h kept in registers), reverse sweep, gradients.
// Reductions: dB, dC over the 64 channels of a block through LDS (exact ZOH) or
// by a cross-lane reduce-scatter (permlane swaps and DPP; Euler), then over
// channel blocks; dA, dD_skip and ddelta_bias per channel over the chunk, then
// over chunks and batch rows.
// All partial sums are added in a fixed order: the backward is deterministic.
// The chunk's inputs are all fetched at its start (one round trip to memory)
// and kept in LDS (41 KB); the main kernel holds at most 168 VGPRs (three waves
// per SIMD): exact ZOH keeps scaled states s = A h off its guarded path, which
// needs no cached coefficients.
#include "ss_device.hpp"

namespace ss {
namespace {

constexpr int kZoh = SS_ZOH;
constexpr int kEuler = SS_EULER;
constexpr int kNW = 4;                 // waves per workgroup
constexpr int kNS = kMaxState / kNW;   // states per wave
constexpr int kKB = 4;                 // steps per block (one owned step per wave)
constexpr int kNB = 8;                 // blocks per chunk
constexpr int kChunk = kKB * kNB;      // steps per chunk (matches the backward plan)

struct BwdParams {
  const void* u;
  const void* delta;
  const void* z;
  const void* dy;
  const float* A;
  const void* Brow;      // (B, L, 16) rows in the input type
  const void* Crow;
  const float* Dskip;
  const float* bias;
  const float* h0;
  // (B, nc, N, D): chunk c's zero-start end state from the summary pass (c <= nc - 2),
  // then, after the forward carry walk, the start state of chunk c (c >= 1)
  float* hstart;
  float* dsum;           // (B, nc, D): sum of dt * log2 e over chunk c (c <= nc - 2)
  // (B, nc, N, D): chunk c's local adjoint from the summary pass (c >= 1), then,
  // after the reverse carry walk, the adjoint entering chunk c from its end
  float* lam;
  float* du;
  float* ddelta;
  float* dz;
  float* dh0;
  float* pB;             // (B, L, nblk, N)
  float* pC;
  float* pA;             // (B, nc, N, D)
  float* pD;             // (B, nc, D)
  float* pbias;
  int64_t L, D;
  int32_t N, ndblk, nchunks;
};

// (delta + bias) log2 e -> dt log2 e
template <bool SOFTPLUS>
__device__ __forceinline__ float step_log2(float x2) {
  return SOFTPLUS ? softplus_log2(x2) : x2;
}

__device__ __forceinline__ float sigmoid_log2(float x2) {   // 1 / (1 + e^-x), x2 = x log2 e
  return hw_rcp(1.0f + hw_exp2(-x2));
}

// ---------------------------------------------------------------- reduce-scatter
// Pairing stages of the cross-lane reduce-scatter below: lanes at distance 32
// and 16 (permlane swaps: the pair's two sums come out of one swap + add),
// then 8 (row rotate) and the mirror pairs inside each 8-lane group.  After
// each stage a lane keeps the half of its values selected by one bit of its
// lane id.
__device__ __forceinline__ float swap_add32(float lo, float hi) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_add16(float lo, float hi) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// x from the lane that DPP control CTRL selects (every control used here has a
// source in range for every lane, so the bound-control zero never applies; it
// lets the move fold into the consuming add)
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
template <int CTRL>
__device__ __forceinline__ float dpp_pair(float lo, float hi, bool upper) {
  const float send = upper ? lo : hi;
  const float keep = upper ? hi : lo;
  return keep + dpp<CTRL>(send);
}
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppQuadXor2 = 0x4e;   // quad_perm [2, 3, 0, 1]
constexpr int kDppQuadXor1 = 0xb1;   // quad_perm [1, 0, 3, 2]

// 16 values per lane -> lanes 4i .. 4i+3 hold the sum over the 64 lanes of
// value i: the pairing stages down to one value per lane, then two
// butterflies inside each quad.
__device__ __forceinline__ float reduce_scatter16(const float (&v)[16], uint32_t lane) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = swap_add32(v[i], v[i + 8]);
  float b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = swap_add16(a[i], a[i + 4]);
  const bool u3 = (lane >> 3) & 1u, u2 = (lane >> 2) & 1u;
  float c[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) c[i] = dpp_pair<kDppRowRor8>(b[i], b[i + 2], u3);
  float d = dpp_pair<kDppRowHalfMirror>(c[0], c[1], u2);
  d += dpp<kDppQuadXor2>(d);
  d += dpp<kDppQuadXor1>(d);
  return d;
}

// 16 values per lane -> their sums over the wave's 64 lanes, through the wave's
// own 3 KB of LDS, 8 values at a time: every lane writes its 8 values as rows
// [value][lane] (rows padded to 68 floats), then lane l adds the 8 entries of
// row l / 8 written by lanes 8 (l % 8) .. 8 (l % 8) + 7 (two 16-byte reads; the
// 16 lanes of one read pass cover all 64 banks once) and the 8 lanes of a row
// combine their sums with two quad butterflies and a half-row mirror.  After
// half h, lanes 8i .. 8i+7 hold the sum of value 8h + i.  Every lane adds in the
// same fixed order.  LDS requests of one wave are served in order, so the rows
// a half reads are the ones it wrote, and the next half's writes land after
// those reads; the wavefront-scope fences keep the compiler from reordering them.
constexpr int kRedRow = kWave + 4;
__device__ __forceinline__ void reduce_lds16(const float (&v)[16], float* xw, uint32_t lane,
                                             float (&out)[2]) {
  const int i = int(lane >> 3), q = int(lane & 7u);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int k = 0; k < 8; ++k) xw[k * kRedRow + lane] = v[8 * h + k];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const float4 a = *reinterpret_cast<const float4*>(xw + i * kRedRow + 8 * q);
    const float4 b = *reinterpret_cast<const float4*>(xw + i * kRedRow + 8 * q + 4);
    float r = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
    r += dpp<kDppQuadXor1>(r);
    r += dpp<kDppQuadXor2>(r);
    r += dpp<kDppRowHalfMirror>(r);
    out[h] = r;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
}

// ---------------------------------------------------------------- main kernel
// LDS (floats): step sizes, gated output gradients and inputs u
// [32 steps][64 lanes], B/C rows [32 steps][B 16, C 16], per-step partials of
// du, d(dt) and y [4 waves][3][4 steps][64 lanes]: 41 KB, three workgroups per CU.
constexpr int kActF = kChunk * kWave;
constexpr int kRowF = kChunk * 2 * kMaxState;
constexpr int kXchF = kNW * 3 * kKB * kWave;
constexpr int kLdsFloats = 3 * kActF + kRowF + kXchF;

// Buffer resources of the (B, L, D) tensors for one chunk and 64-channel group,
// based at element (b, t0, first channel of the group): step k of the chunk and
// lane l reach their element at soffset k * step bytes, voffset l * element
// size.  Idle lanes (past D) carry an out-of-range voffset: their loads read 0
// and their stores are dropped.  (k < 32 and D <= 2^24 keep every offset
// inside 32 bits.)
template <typename In>
struct ChunkIO {
  Rsrc dl, dy, z, u;         // inputs, In
  Rsrc du, ddelta, dz;       // outputs, fp32
  uint32_t vin, vout;        // lane offsets (bytes)
  uint32_t sin, sout;        // bytes per step

  __device__ __forceinline__ ChunkIO(const BwdParams& p, int64_t b, int32_t t0, int dblk,
                                     uint32_t lane, bool active) {
    const int64_t e0 = (b * p.L + t0) * p.D + int64_t(dblk) * kWave;
    dl = make_rsrc(static_cast<const In*>(p.delta) + e0);
    dy = make_rsrc(static_cast<const In*>(p.dy) + e0);
    z = make_rsrc(p.z ? static_cast<const In*>(p.z) + e0 : static_cast<const In*>(p.dy) + e0);
    u = make_rsrc(static_cast<const In*>(p.u) + e0);
    du = make_rsrc(p.du + e0);
    ddelta = make_rsrc(p.ddelta + e0);
    dz = make_rsrc(p.dz ? p.dz + e0 : p.du + e0);
    vin = active ? lane * uint32_t(sizeof(In)) : kOutOfRange;
    vout = active ? lane * uint32_t(sizeof(float)) : kOutOfRange;
    sin = uint32_t(p.D) * uint32_t(sizeof(In));
    sout = uint32_t(p.D) * uint32_t(sizeof(float));
  }
};

// Stages chunk [t0, t1) in LDS: per step and lane the step size dt log2 e, the
// gated upstream gradient gy and the input u (all 0 past t1, gy and u 0 on idle
// lanes), and the chunk's B/C rows.  Wave w prepares the steps k with
// k % 4 == w; every load is issued before any is used.  The caller places the
// barrier.
template <typename In, bool HAS_Z, bool SOFTPLUS>
__device__ __forceinline__ void stage_chunk(const BwdParams& p, const ChunkIO<In>& io, float* lds,
                                            int64_t row0, int32_t t0, int32_t t1, int wave,
                                            uint32_t lane, float bias2, float amask) {
  float* actDl = lds;                            // [32 steps][64 lanes]
  float* actGy = lds + kActF;
  float* actU = lds + 2 * kActF;
  float* rows = lds + 3 * kActF;                 // [32 steps][B 16, C 16]
  In rdl[kNB], rdy[kNB], rz[kNB], ru[kNB];
#pragma unroll
  for (int s = 0; s < kNB; ++s) {
    const int32_t t = t0 + s * kNW + wave;
    const uint32_t so = uint32_t((t < t1 ? t : t1 - 1) - t0) * io.sin;
    rdl[s] = buf_load<In>(io.dl, io.vin, so);
    rdy[s] = buf_load<In>(io.dy, io.vin, so);
    if (HAS_Z) rz[s] = buf_load<In>(io.z, io.vin, so);
    ru[s] = buf_load<In>(io.u, io.vin, so);
  }
  // 256 threads, 4 values each: step tid / 8, B (parts 0-3) or C (4-7)
  const int tid = wave * kWave + int(lane);
  const int rk8 = tid / 8, rpart = tid % 8;
  const auto rraw = load_raw4(static_cast<const In*>(rpart < 4 ? p.Brow : p.Crow) +
                              (row0 + (t0 + rk8 < t1 ? t0 + rk8 : t1 - 1)) * kMaxState +
                              4 * (rpart % 4));
#pragma unroll
  for (int s = 0; s < kNB; ++s) {
    const int k = s * kNW + wave;
    const bool valid = t0 + k < t1;
    const float x2 = __builtin_fmaf(to_f32(rdl[s]), kLog2e, bias2);
    float gy = to_f32(rdy[s]);
    if (HAS_Z) {
      const float zf = to_f32(rz[s]);
      gy *= zf * sigmoid_log2(zf * kLog2e);      // dy silu(z)
    }
    actDl[k * kWave + lane] = valid ? step_log2<SOFTPLUS>(x2) : 0.0f;
    actGy[k * kWave + lane] = valid ? gy * amask : 0.0f;
    actU[k * kWave + lane] = valid ? to_f32(ru[s]) * amask : 0.0f;
  }
  *reinterpret_cast<float4*>(rows + rk8 * 2 * kMaxState + 4 * rpart) = unpack4(rraw);
}

template <typename In, int DISC, bool HAS_Z, bool SOFTPLUS, bool SAFE>
__device__ __forceinline__ void bwd_chunk(const BwdParams& p, float* lds, int64_t b, int dblk,
                                          int chunk, int wave, uint32_t lane) {
  const int n0 = wave * kNS;
  const int N = p.N;
  const int64_t D = p.D;
  const int64_t d = int64_t(dblk) * kWave + lane;
  const bool active = d < D;
  const int64_t dc = active ? d : D - 1;
  const float amask = active ? 1.0f : 0.0f;
  const int32_t t0 = chunk * kChunk;
  const int32_t t1 = int32_t(t0 + kChunk < p.L ? t0 + kChunk : p.L);
  const int64_t row0 = b * p.L;
  const ChunkIO<In> io(p, b, t0, dblk, lane, active);

  float A[kNS], iA[kNS];
#pragma unroll
  for (int j = 0; j < kNS; ++j) {
    const int n = n0 + j;
    const float a = n < N ? p.A[dc * N + n] : -1.0f;
    A[j] = a;
    iA[j] = a == 0.0f ? 0.0f : 1.0f / a;
  }
  const float Dd = p.Dskip ? p.Dskip[dc] : 0.0f;
  const float bias2 = (p.bias ? p.bias[dc] : 0.0f) * kLog2e;

  float* actDl = lds;                            // [32 steps][64 lanes]
  float* actGy = lds + kActF;                    // [32 steps][64 lanes]
  float* actU = lds + 2 * kActF;                 // [32 steps][64 lanes]
  float* rows = lds + 3 * kActF;                 // [32 steps][B 16, C 16]
  float* xch = rows + kRowF;                     // [4 waves][3][4 steps][64 lanes]
  // ---- phase A1: the chunk's inputs and rows to LDS, with the loads of the
  //      chunk's start state and of the adjoint carry entering it from its end
  float h[kNS], nu[kNS];
  if (chunk == 0) {
#pragma unroll
    for (int j = 0; j < kNS; ++j) h[j] = (p.h0 && n0 + j < N) ? p.h0[(b * D + dc) * N + n0 + j] : 0.0f;
  } else {
    const float* hs = p.hstart + (b * p.nchunks + chunk) * int64_t(N) * D + dc;
#pragma unroll
    for (int j = 0; j < kNS; ++j) h[j] = n0 + j < N ? hs[int64_t(n0 + j) * D] : 0.0f;
  }
  if (chunk == p.nchunks - 1) {
#pragma unroll
    for (int j = 0; j < kNS; ++j) nu[j] = 0.0f;
  } else {
    const float* ls = p.lam + (b * p.nchunks + chunk) * int64_t(N) * D + dc;
#pragma unroll
    for (int j = 0; j < kNS; ++j) nu[j] = n0 + j < N ? ls[int64_t(n0 + j) * D] : 0.0f;
  }
  stage_chunk<In, HAS_Z, SOFTPLUS>(p, io, lds, row0, t0, t1, wave, lane, bias2, amask);
  __syncthreads();
  // this wave's 4 states of the B (m = 0) or C (m = 1) row of step kk
  auto row_of = [&](int kk, int m) -> float4 {
    return *reinterpret_cast<const float4*>(rows + kk * 2 * kMaxState + m * kMaxState + n0);
  };


  // ---- phase A2: forward over the chunk, one checkpoint per block.  Exact
  //      ZOH off the guarded path (every |A| >= kWeakA) runs on scaled states
  //      s = A h, as the forward does: s <- a (s + B u) - B u, one operation
  //      fewer than a h + ((a - 1) / A) B u; the checkpoints hold s.
  constexpr bool kScaledCk = DISC == kZoh && !SAFE;
  float ck[kNB][kNS];
  if (kScaledCk) {
#pragma unroll
    for (int j = 0; j < kNS; ++j) h[j] *= A[j];
  }
#pragma unroll
  for (int jb = 0; jb < kNB; ++jb) {
#pragma unroll
    for (int j = 0; j < kNS; ++j) ck[jb][j] = h[j];
#pragma unroll
    for (int k = 0; k < kKB; ++k) {
      const int kk = jb * kKB + k;
      const float dl = actDl[kk * kWave + lane];
      const float uf = actU[kk * kWave + lane];
      const float dtu = dl * kLn2 * uf;            // Euler: B_bar u = dt u B
      const float4 B4 = row_of(kk, 0);
      const float Bv[kNS] = {B4.x, B4.y, B4.z, B4.w};
#pragma unroll
      for (int j = 0; j < kNS; ++j) {
        const float a = hw_exp2(dl * A[j]);
        if (DISC == kEuler) {
          h[j] = __builtin_fmaf(a, h[j], dtu * Bv[j]);
        } else if (kScaledCk) {
          const float bu = Bv[j] * uf;
          h[j] = __builtin_fmaf(a, h[j] + bu, -bu);
        } else {
          const float coef = zoh_coef_guarded(a, iA[j], dl * kLn2, dl * A[j]);
          h[j] = __builtin_fmaf(a, h[j], coef * (Bv[j] * uf));
        }
      }
    }
  }

  // ---- phase B: blocks in reverse
  // nu: adjoint carried from later steps, A_bar_{t+1} lambda_{t+1}
  // dA = dA + dAc / A (dAc: exact ZOH's term through d coef / dA)
  float dA[kNS], dAc[kNS];
#pragma unroll
  for (int j = 0; j < kNS; ++j) dA[j] = dAc[j] = 0.0f;
  float dDacc = 0.0f, dbacc = 0.0f;
  // The sums over the 64 channels of a block's [4 steps][4 states] dB or dC
  // values.  Exact ZOH takes them through LDS (reduce_lds16: after half h the
  // first lane of each 8-lane row holds value 8h + lane / 8, i.e. step
  // 2h + lane / 32 of the block, state n0 + (lane / 8) % 4); Euler, whose
  // shorter sweep leaves less work to cover the LDS round trips, by the
  // cross-lane reduce-scatter (the first lane of each quad holds value
  // lane / 4: step lane / 16, state n0 + (lane / 4) % 4).  That lane stores it
  // into the pB / pC rows (based at the chunk's first step, this group and this
  // wave's states); the other lanes get an out-of-range offset.
  constexpr bool kLdsRed = DISC == kZoh;
  float* const xw = xch + wave * 3 * kKB * kWave;          // this wave's slice
  const int rk = kLdsRed ? int(lane >> 5) : int(lane >> 4);
  const int rj = kLdsRed ? int((lane >> 3) & 3u) : int((lane >> 2) & 3u);
  const bool rwrite = (lane & (kLdsRed ? 7u : 3u)) == 0 && n0 + rj < N;
  const int64_t rbase = ((row0 + t0) * p.ndblk + dblk) * N + n0;
  const Rsrc rpB = make_rsrc(p.pB + rbase), rpC = make_rsrc(p.pC + rbase);
  const uint32_t rstep = uint32_t(p.ndblk) * uint32_t(N) * uint32_t(sizeof(float));   // per step
  const uint32_t rvoff = rwrite ? uint32_t(rk) * rstep + uint32_t(rj) * uint32_t(sizeof(float))
                                : kOutOfRange;

#pragma unroll
  for (int jb = kNB - 1; jb >= 0; --jb) {
    if (t0 + jb * kKB >= t1) continue;          // wave-uniform: block past the end
    // raw inputs of the step this wave owns in the block (k = wave), fetched
    // now and used by the block's outputs at its end
    In zo{}, go{}, dlo{};
    {
      const int32_t tw = t0 + jb * kKB + wave;
      const uint32_t so = uint32_t((tw < t1 ? tw : t1 - 1) - t0) * io.sin;
      if (HAS_Z) {
        zo = buf_load<In>(io.z, io.vin, so);
        go = buf_load<In>(io.dy, io.vin, so);
      }
      if (SOFTPLUS) dlo = buf_load<In>(io.dl, io.vin, so);
    }
    float uf[kKB], dl[kKB], gy[kKB], yp[kKB];
    float hs[kKB][kNS];
    float red[kKB * kNS];
    // recompute the block from its checkpoint (scaled states: s runs as in the
    // checkpoint pass, h = s / A); dC = gy h
    float hb[kNS], sc[kNS];
#pragma unroll
    for (int j = 0; j < kNS; ++j) {
      sc[j] = ck[jb][j];
      hb[j] = kScaledCk ? sc[j] * iA[j] : sc[j];
      h[j] = hb[j];
    }
#pragma unroll
    for (int k = 0; k < kKB; ++k) {
      const int kk = jb * kKB + k;
      dl[k] = actDl[kk * kWave + lane];
      gy[k] = actGy[kk * kWave + lane];
      uf[k] = actU[kk * kWave + lane];
      const float4 B4 = row_of(kk, 0), C4 = row_of(kk, 1);
      const float Bv[kNS] = {B4.x, B4.y, B4.z, B4.w}, Cv[kNS] = {C4.x, C4.y, C4.z, C4.w};
      const float dtu0 = dl[k] * kLn2;            // dt
      const float dtu = dtu0 * uf[k];
      float y0 = 0.0f;
#pragma unroll
      for (int j = 0; j < kNS; ++j) {
        const float a = hw_exp2(dl[k] * A[j]);
        if (DISC == kEuler) {
          h[j] = __builtin_fmaf(a, h[j], dtu * Bv[j]);
        } else if (kScaledCk) {
          const float bu = Bv[j] * uf[k];
          sc[j] = __builtin_fmaf(a, sc[j] + bu, -bu);
          h[j] = sc[j] * iA[j];
        } else {
          const float coef = zoh_coef_guarded(a, iA[j], dtu0, dl[k] * A[j]);
          h[j] = __builtin_fmaf(a, h[j], coef * (Bv[j] * uf[k]));
        }
        hs[k][j] = h[j];
        y0 = __builtin_fmaf(Cv[j], h[j], y0);
        red[k * kNS + j] = gy[k] * h[j];                       // dC
      }
      yp[k] = y0;
    }
    // a block's rows are 4 steps: the lane's step (2h + rk in half h of the
    // LDS form) must lie before t1
    const uint32_t rv0 = t0 + jb * kKB + rk < t1 ? rvoff : kOutOfRange;
    const uint32_t rv1 = kLdsRed && t0 + jb * kKB + 2 + rk < t1 ? rvoff + 2 * rstep : kOutOfRange;
    auto reduce_store = [&](Rsrc rp) {
      const uint32_t so = uint32_t(jb * kKB) * rstep;
      if constexpr (kLdsRed) {
        float r[2];
        reduce_lds16(red, xw, lane, r);
        buf_store<float>(rp, rv0, so, r[0]);
        buf_store<float>(rp, rv1, so, r[1]);
      } else {
        buf_store<float>(rp, rv0, so, reduce_scatter16(red, lane));
      }
    };
    reduce_store(rpC);
    // reverse sweep.  Per step, with lam = d loss / d h_t and nu = A_bar lam:
    //   dB = lam coef u (coef = dt for Euler, (A_bar - 1) / A for exact ZOH)
    //   du = sum_n lam coef B
    //   d(dt) = sum_n nu h_{t-1} A + u sum_n (lam B [Euler] | nu B [ZOH])
    //   dA += nu h_{t-1} dt  (+ lam B u d coef / dA for ZOH, with
    //         d coef / dA = (dt A_bar - coef) / A; the 1 / A is applied once per
    //         chunk; the guarded path takes its series where |dt A| < kZohSeries)
    float dup[kKB], ddp[kKB];
#pragma unroll
    for (int k = kKB - 1; k >= 0; --k) {
      const int kk = jb * kKB + k;
      const float4 B4 = row_of(kk, 0), C4 = row_of(kk, 1);
      const float Bv[kNS] = {B4.x, B4.y, B4.z, B4.w}, Cv[kNS] = {C4.x, C4.y, C4.z, C4.w};
      const float dtn = dl[k] * kLn2;           // dt
      const float udt = uf[k] * dtn;            // u dt
      float sLB = 0.0f, sdd = 0.0f, sdu = 0.0f;
#pragma unroll
      for (int j = 0; j < kNS; ++j) {
        const float a = hw_exp2(dl[k] * A[j]);     // same value as in the recompute
        const float hp = k > 0 ? hs[k - 1][j] : hb[j];
        const float lam = __builtin_fmaf(gy[k], Cv[j], nu[j]);
        nu[j] = a * lam;
        const float nh = nu[j] * hp;
        sdd = __builtin_fmaf(nh, A[j], sdd);
        dA[j] = __builtin_fmaf(nh, dtn, dA[j]);
        if (DISC == kEuler) {
          red[k * kNS + j] = lam * udt;                   // dB
          sLB = __builtin_fmaf(lam, Bv[j], sLB);
        } else {
          const float x2 = dl[k] * A[j];         // dt A log2 e
          // lam coef: lam (a - 1) / A off the guarded path
          const float cl = SAFE ? lam * zoh_coef_guarded(a, iA[j], dtn, x2)
                                : __builtin_fmaf(a, lam, -lam) * iA[j];
          const float db = cl * uf[k];
          red[k * kNS + j] = db;                          // dB
          sdu = __builtin_fmaf(cl, Bv[j], sdu);
          sLB = __builtin_fmaf(nu[j], Bv[j], sLB);
          const float dac = Bv[j] * __builtin_fmaf(udt, nu[j], -db);
          if (SAFE) {
            // near dt A = 0 the quotient form cancels: the series of d coef / dA
            const bool ser = __builtin_unpredictable(__builtin_fabsf(x2) < kZohSeries * kLog2e);
            dA[j] = __builtin_fmaf(ser ? lam * Bv[j] * uf[k] : 0.0f,
                                   zoh_dcoef_series(dtn, x2 * kLn2), dA[j]);
            dAc[j] += ser ? 0.0f : dac;
          } else {
            dAc[j] += dac;
          }
        }
      }
      dup[k] = DISC == kEuler ? dtn * sLB : sdu;
      ddp[k] = __builtin_fmaf(uf[k], sLB, sdd);
    }
    reduce_store(rpB);
    // per-step partials of this wave -> LDS
#pragma unroll
    for (int k = 0; k < kKB; ++k) {
      xch[((wave * 3 + 0) * kKB + k) * kWave + lane] = dup[k];
      xch[((wave * 3 + 1) * kKB + k) * kWave + lane] = ddp[k];
      xch[((wave * 3 + 2) * kKB + k) * kWave + lane] = yp[k];
    }
    __syncthreads();
    // output of the step this wave owns (k = wave)
    {
      const int k = wave;
      const int32_t t = t0 + jb * kKB + k;
      float sdu = 0.0f, sdd = 0.0f, sy = 0.0f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        sdu += xch[((w * 3 + 0) * kKB + k) * kWave + lane];
        sdd += xch[((w * 3 + 1) * kKB + k) * kWave + lane];
        sy += xch[((w * 3 + 2) * kKB + k) * kWave + lane];
      }
      if (t < t1) {
        const uint32_t so = uint32_t(t - t0) * io.sout;
        const int kk = jb * kKB + k;
        const float ui = actU[kk * kWave + lane], gyk = actGy[kk * kWave + lane];
        if (HAS_Z) {
          // dz = dy * y * d silu(z) / dz, y the pre-gate output
          const float zf = to_f32(zo), g = to_f32(go);
          const float sz = sigmoid_log2(zf * kLog2e);
          const float y = __builtin_fmaf(Dd, ui, sy);
          buf_store<float>(io.dz, io.vout, so, g * y * sz * __builtin_fmaf(zf, 1.0f - sz, 1.0f));
        }
        buf_store<float>(io.du, io.vout, so, __builtin_fmaf(gyk, Dd, sdu));
        float ddv = sdd;                                 // d loss / d dt
        if (SOFTPLUS) ddv *= sigmoid_log2(__builtin_fmaf(to_f32(dlo), kLog2e, bias2));   // through softplus
        buf_store<float>(io.ddelta, io.vout, so, ddv);
        dDacc = __builtin_fmaf(gyk, ui, dDacc);
        dbacc += ddv;
      }
    }
    __syncthreads();
  }

  if (chunk == 0 && p.dh0 && active) {
#pragma unroll
    for (int j = 0; j < kNS; ++j)
      if (n0 + j < N) p.dh0[(b * D + d) * N + n0 + j] = nu[j];
  }
  if (active) {
    float* pa = p.pA + (b * p.nchunks + chunk) * int64_t(N) * D + d;
#pragma unroll
    for (int j = 0; j < kNS; ++j)
      if (n0 + j < N) pa[int64_t(n0 + j) * D] = DISC == kEuler ? dA[j] : __builtin_fmaf(iA[j], dAc[j], dA[j]);
  }
  // dD_skip and ddelta_bias: the four waves' per-channel sums, added by wave 0
  xch[(wave * 2 + 0) * kWave + lane] = dDacc;
  xch[(wave * 2 + 1) * kWave + lane] = dbacc;
  __syncthreads();
  if (wave == 0 && active) {
    float sD = 0.0f, sb = 0.0f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      sD += xch[(w * 2 + 0) * kWave + lane];
      sb += xch[(w * 2 + 1) * kWave + lane];
    }
    p.pD[(b * p.nchunks + chunk) * D + d] = sD;
    p.pbias[(b * p.nchunks + chunk) * D + d] = sb;
  }
}

// Three waves per SIMD (at most 168 VGPRs).  Exact ZOH's guarded path (a
// workgroup holding a slowly decaying state) spills a few values to scratch at
// this bound; the fast path does not.
template <typename In, int DISC, bool HAS_Z, bool SOFTPLUS>
__global__ __launch_bounds__(kWave * kNW, 3) void bwd_kernel(BwdParams p) {
  __shared__ float4 lds4[kLdsFloats / 4];
  float* lds = reinterpret_cast<float*>(lds4);
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const uint32_t lane = threadIdx.x % kWave;
  int64_t bid = blockIdx.x;
  const int dblk = int(bid % p.ndblk);
  bid /= p.ndblk;
  const int chunk = int(bid % p.nchunks);
  const int64_t b = bid / p.nchunks;
  // exact ZOH with a slowly decaying state (|A| < kWeakA, A == 0 included) in
  // the block takes the guarded path (all waves agree)
  bool weak = false;
  if (DISC == kZoh) {
    const int64_t d = int64_t(dblk) * kWave + lane;
    const int64_t dc = d < p.D ? d : p.D - 1;
    for (int n = 0; n < p.N; ++n) weak |= __builtin_fabsf(p.A[dc * p.N + n]) < kWeakA;
  }
  if (DISC == kZoh && __syncthreads_or(weak))
    bwd_chunk<In, DISC, HAS_Z, SOFTPLUS, true>(p, lds, b, dblk, chunk, wave, lane);
  else
    bwd_chunk<In, DISC, HAS_Z, SOFTPLUS, false>(p, lds, b, dblk, chunk, wave, lane);
}

// ---------------------------------------------------------------- chunk summaries
// One pass over chunk c yields what both carry scans need, for the 4 states of
// each wave and the 64 channels of the workgroup:
//  - forward (c <= nc - 2): the end state from a zero start, into hstart[b][c],
//    and the chunk's sum of dt log2 e, into dsum[b][c];
//  - reverse (c >= 1): the adjoint at the chunk's start with nothing entering
//    from its end, sum over t of (A_bar_t0 ... A_bar_t) gy_t C_t, into
//    lam[b][c]; it is accumulated forward in time with a running product of
//    A_bar, so the two summaries share one exponential per (t, n).
template <typename In, int DISC, bool HAS_Z, bool SOFTPLUS, bool SAFE>
__device__ __forceinline__ void summary_chunk(const BwdParams& p, float* lds, int64_t b, int dblk,
                                              int chunk, int wave, uint32_t lane) {
  const int n0 = wave * kNS;
  const int N = p.N;
  const int64_t D = p.D;
  const int64_t d = int64_t(dblk) * kWave + lane;
  const bool active = d < D;
  const int64_t dc = active ? d : D - 1;
  const int32_t t0 = chunk * kChunk;
  const int32_t t1 = int32_t(t0 + kChunk < p.L ? t0 + kChunk : p.L);
  const int64_t row0 = b * p.L;
  const float bias2 = (p.bias ? p.bias[dc] : 0.0f) * kLog2e;
  const ChunkIO<In> io(p, b, t0, dblk, lane, active);
  stage_chunk<In, HAS_Z, SOFTPLUS>(p, io, lds, row0, t0, t1, wave, lane, bias2,
                                   active ? 1.0f : 0.0f);
  float A[kNS], iA[kNS];
#pragma unroll
  for (int j = 0; j < kNS; ++j) {
    const int n = n0 + j;
    const float a = n < N ? p.A[dc * N + n] : -1.0f;
    A[j] = a;
    iA[j] = a == 0.0f ? 0.0f : 1.0f / a;
  }
  __syncthreads();
  const float* actDl = lds;
  const float* actGy = lds + kActF;
  const float* actU = lds + 2 * kActF;
  const float* rows = lds + 3 * kActF;
  float h[kNS], P[kNS], R[kNS];
#pragma unroll
  for (int j = 0; j < kNS; ++j) {
    h[j] = 0.0f;
    P[j] = 1.0f;
    R[j] = 0.0f;
  }
  float dsum = 0.0f;
#pragma unroll 4
  for (int k = 0; k < kChunk; ++k) {
    const float dl = actDl[k * kWave + lane];
    const float uf = actU[k * kWave + lane];
    const float gy = actGy[k * kWave + lane];
    const float4 B4 = *reinterpret_cast<const float4*>(rows + k * 2 * kMaxState + n0);
    const float4 C4 = *reinterpret_cast<const float4*>(rows + k * 2 * kMaxState + kMaxState + n0);
    const float Bv[kNS] = {B4.x, B4.y, B4.z, B4.w}, Cv[kNS] = {C4.x, C4.y, C4.z, C4.w};
    const float dtu = dl * kLn2 * uf;
#pragma unroll
    for (int j = 0; j < kNS; ++j) {
      const float a = hw_exp2(dl * A[j]);
      if (DISC == kEuler) {
        h[j] = __builtin_fmaf(a, h[j], dtu * Bv[j]);
      } else if (SAFE) {
        const float coef = zoh_coef_guarded(a, iA[j], dl * kLn2, dl * A[j]);
        h[j] = __builtin_fmaf(a, h[j], coef * (Bv[j] * uf));
      } else {
        // scaled state s = A h, as in the main kernel's checkpoint pass
        const float bu = Bv[j] * uf;
        h[j] = __builtin_fmaf(a, h[j] + bu, -bu);
      }
      P[j] *= a;
      R[j] = __builtin_fmaf(P[j], gy * Cv[j], R[j]);
    }
    dsum += dl;
  }
  if (!active) return;
  const int64_t slot = (b * p.nchunks + chunk) * int64_t(N) * D + d;
  if (chunk <= p.nchunks - 2) {
#pragma unroll
    for (int j = 0; j < kNS; ++j)
      if (n0 + j < N) p.hstart[slot + int64_t(n0 + j) * D] = DISC == kZoh && !SAFE ? h[j] * iA[j] : h[j];
    if (wave == 0) p.dsum[(b * p.nchunks + chunk) * D + d] = dsum;
  }
  if (chunk >= 1) {
#pragma unroll
    for (int j = 0; j < kNS; ++j)
      if (n0 + j < N) p.lam[slot + int64_t(n0 + j) * D] = R[j];
  }
}

// five workgroups per CU (LDS 28 KB each): at most 96 VGPRs
template <typename In, int DISC, bool HAS_Z, bool SOFTPLUS>
__global__ __launch_bounds__(kWave * kNW, 5) void summary_kernel(BwdParams p) {
  __shared__ float4 lds4[(3 * kActF + kRowF) / 4];
  float* lds = reinterpret_cast<float*>(lds4);
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const uint32_t lane = threadIdx.x % kWave;
  int64_t bid = blockIdx.x;
  const int dblk = int(bid % p.ndblk);
  bid /= p.ndblk;
  const int chunk = int(bid % p.nchunks);
  const int64_t b = bid / p.nchunks;
  bool weak = false;   // as in bwd_kernel
  if (DISC == kZoh) {
    const int64_t d = int64_t(dblk) * kWave + lane;
    const int64_t dc = d < p.D ? d : p.D - 1;
    for (int n = 0; n < p.N; ++n) weak |= __builtin_fabsf(p.A[dc * p.N + n]) < kWeakA;
  }
  if (DISC == kZoh && __syncthreads_or(weak))
    summary_chunk<In, DISC, HAS_Z, SOFTPLUS, true>(p, lds, b, dblk, chunk, wave, lane);
  else
    summary_chunk<In, DISC, HAS_Z, SOFTPLUS, false>(p, lds, b, dblk, chunk, wave, lane);
}

// ---------------------------------------------------------------- reductions
// dB, dC (B, L, N): the per-(b, t) rows of partials summed over channel groups.
__device__ __forceinline__ void reduce_rows(const float* __restrict__ pB,
                                            const float* __restrict__ pC, float* __restrict__ dB,
                                            float* __restrict__ dC, int64_t rows, int nblk, int N,
                                            int64_t gid) {
  if (gid >= rows * N) return;
  const int64_t r = gid / N;
  const int n = int(gid % N);
  const float* qb = pB + r * nblk * N + n;
  const float* qc = pC + r * nblk * N + n;
  float sb = 0.0f, sc = 0.0f;
#pragma unroll 8
  for (int k = 0; k < nblk; ++k) {
    sb += qb[k * N];
    sc += qc[k * N];
  }
  dB[gid] = sb;
  dC[gid] = sc;
}

// dA (D, N), dD_skip and ddelta_bias (D): sums over (batch row, chunk) of the
// per-chunk partials.  A workgroup takes 64 columns (column = n * D + d; n == N
// holds the two per-channel vectors) and splits the terms over 16 thread
// groups, each with 8 interleaved running sums, so 128 loads per column are in
// flight.  Every addition happens in a fixed order: the result is deterministic.
constexpr int kRedCols = 64, kRedGroups = 16, kRedAcc = 8;
constexpr int kRedThreads = kRedCols * kRedGroups;
__device__ __forceinline__ void reduce_chan(const float* __restrict__ pA,
                                            const float* __restrict__ pD,
                                            const float* __restrict__ pbias, float* __restrict__ dA,
                                            float* __restrict__ dD, float* __restrict__ dbias,
                                            int64_t B, int64_t D, int N, int nchunks, int64_t blk,
                                            float (&part)[2][kRedGroups][kRedCols]) {
  const int c = int(threadIdx.x) % kRedCols, g = int(threadIdx.x) / kRedCols;
  const int64_t col = blk * kRedCols + c;
  const bool valid = col < D * (N + 1);
  const int64_t d = valid ? col % D : 0;
  const int n = valid ? int(col / D) : 0;
  const int64_t terms = B * nchunks;
  // group g adds terms g, g + 16, g + 32, ...; running sum m takes every 8th of them
  auto sum = [&](const float* x, int64_t stride) {
    float acc[kRedAcc];
#pragma unroll
    for (int m = 0; m < kRedAcc; ++m) acc[m] = 0.0f;
    int64_t k = g;
    for (; k + (kRedAcc - 1) * kRedGroups < terms; k += kRedAcc * kRedGroups) {
#pragma unroll
      for (int m = 0; m < kRedAcc; ++m) acc[m] += x[(k + m * kRedGroups) * stride];
    }
    for (int m = 0; k < terms; k += kRedGroups, ++m) acc[m] += x[k * stride];
    return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  };
  float s0 = 0.0f, s1 = 0.0f;
  if (valid) {
    if (n < N) {
      s0 = sum(pA + int64_t(n) * D + d, int64_t(N) * D);
    } else {
      s0 = sum(pD + d, D);
      s1 = sum(pbias + d, D);
    }
  }
  part[0][g][c] = s0;
  part[1][g][c] = s1;
  __syncthreads();
  if (g != 0 || !valid) return;
  float t0 = 0.0f, t1 = 0.0f;
#pragma unroll
  for (int q = 0; q < kRedGroups; ++q) {
    t0 += part[0][q][c];
    t1 += part[1][q][c];
  }
  if (n < N) {
    dA[d * N + n] = t0;
  } else {
    if (dD) dD[d] = t0;
    if (dbias) dbias[d] = t1;
  }
}

// Both reductions in one launch: workgroups [0, nchan) take the channel
// columns, the rest kRedThreads (b, t, n) entries of dB and dC each (the two
// are independent; every workgroup takes one branch as a whole).
__global__ __launch_bounds__(kRedThreads) void reduce_kernel(BwdParams p, float* dA, float* dB,
                                                            float* dC, float* dD, float* dbias,
                                                            int64_t B, int64_t nchan) {
  __shared__ float part[2][kRedGroups][kRedCols];
  const int64_t blk = blockIdx.x;
  if (blk < nchan) {
    reduce_chan(p.pA, p.pD, p.pbias, dA, dD, dbias, B, p.D, p.N, p.nchunks, blk, part);
  } else {
    reduce_rows(p.pB, p.pC, dB, dC, B * p.L, p.ndblk, p.N,
                (blk - nchan) * kRedThreads + threadIdx.x);
  }
}

template <typename In, bool HAS_Z, bool SOFTPLUS>
hipError_t launch_main(const ss_desc_t& d, const BwdParams& p, int64_t blocks, hipStream_t st) {
  if (d.disc == SS_ZOH)
    hipLaunchKernelGGL((bwd_kernel<In, kZoh, HAS_Z, SOFTPLUS>), dim3(unsigned(blocks)),
                       dim3(kWave * kNW), 0, st, p);
  else
    hipLaunchKernelGGL((bwd_kernel<In, kEuler, HAS_Z, SOFTPLUS>), dim3(unsigned(blocks)),
                       dim3(kWave * kNW), 0, st, p);
  return hipGetLastError();
}

template <typename In, bool HAS_Z, bool SOFTPLUS>
hipError_t launch_summary(const ss_desc_t& d, const BwdParams& p, int64_t blocks, hipStream_t st) {
  if (d.disc == SS_ZOH)
    hipLaunchKernelGGL((summary_kernel<In, kZoh, HAS_Z, SOFTPLUS>), dim3(unsigned(blocks)),
                       dim3(kWave * kNW), 0, st, p);
  else
    hipLaunchKernelGGL((summary_kernel<In, kEuler, HAS_Z, SOFTPLUS>), dim3(unsigned(blocks)),
                       dim3(kWave * kNW), 0, st, p);
  return hipGetLastError();
}

template <typename In>
hipError_t dispatch_bwd(const ss_desc_t& d, const BwdParams& p, bool summary, int64_t blocks,
                        hipStream_t st) {
  const bool z = p.z != nullptr, sp = d.delta_softplus != 0;
  if (summary) {
    if (z) return sp ? launch_summary<In, true, true>(d, p, blocks, st) : launch_summary<In, true, false>(d, p, blocks, st);
    return sp ? launch_summary<In, false, true>(d, p, blocks, st) : launch_summary<In, false, false>(d, p, blocks, st);
  }
  if (z) return sp ? launch_main<In, true, true>(d, p, blocks, st) : launch_main<In, true, false>(d, p, blocks, st);
  return sp ? launch_main<In, false, true>(d, p, blocks, st) : launch_main<In, false, false>(d, p, blocks, st);
}

}  // namespace

int launch_bwd(const ss_desc_t& d, const BwdPlan& plan, const BwdArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (plan.tp.chunk_len != kChunk && plan.tp.nchunks > 1) return int(hipErrorInvalidValue);
  char* ws = a.ws;
  void* Brow = plan.packed_rows ? static_cast<void*>(ws + plan.off_brow) : const_cast<void*>(a.Bm);
  void* Crow = plan.packed_rows ? static_cast<void*>(ws + plan.off_crow) : const_cast<void*>(a.Cm);
  float* hend = reinterpret_cast<float*>(ws + plan.off_hend);
  float* dsum = reinterpret_cast<float*>(ws + plan.off_dsum);
  float* lam = reinterpret_cast<float*>(ws + plan.off_lam);
  if (plan.packed_rows) {
    const int e = launch_pack_rows(d, a.Bm, a.Cm, Brow, Crow, stream);
    if (e != 0) return e;
  }
  const int nc = int(plan.tp.nchunks);
  const int ndblk = int(plan.nblk);
  BwdParams p{};
  p.u = a.u; p.delta = a.delta; p.z = a.z; p.dy = a.dy; p.A = a.A;
  p.Brow = Brow; p.Crow = Crow; p.Dskip = a.Dskip; p.bias = a.bias; p.h0 = a.h0;
  p.hstart = hend; p.dsum = dsum; p.lam = lam;
  p.du = a.du; p.ddelta = a.ddelta; p.dz = a.dz; p.dh0 = a.dh0;
  p.pB = reinterpret_cast<float*>(ws + plan.off_pB);
  p.pC = reinterpret_cast<float*>(ws + plan.off_pC);
  p.pA = reinterpret_cast<float*>(ws + plan.off_pA);
  p.pD = reinterpret_cast<float*>(ws + plan.off_pD);
  p.pbias = reinterpret_cast<float*>(ws + plan.off_pbias);
  p.L = d.seqlen; p.D = d.dim; p.N = int32_t(d.dstate); p.ndblk = ndblk; p.nchunks = nc;
  const int64_t cols = d.batch * ndblk;
  hipError_t e;
  if (nc > 1) {
    // both chunk summaries in one pass, then the forward and the reverse carry scans
    e = d.in_dtype == SS_BF16 ? dispatch_bwd<uint16_t>(d, p, true, cols * nc, st)
                              : dispatch_bwd<float>(d, p, true, cols * nc, st);
    if (e != hipSuccess) return int(e);
    const int ec = launch_chunk_carry_pair(hend, lam, dsum, a.A, a.h0, d.batch, d.dim,
                                           int(d.dstate), nc, stream);
    if (ec != 0) return ec;
  }
  e = d.in_dtype == SS_BF16 ? dispatch_bwd<uint16_t>(d, p, false, cols * nc, st)
                            : dispatch_bwd<float>(d, p, false, cols * nc, st);
  if (e != hipSuccess) return int(e);
  const int64_t rows = d.batch * d.seqlen;
  const int64_t nchan = (d.dim * (d.dstate + 1) + kRedCols - 1) / kRedCols;
  const int64_t nrow = (rows * d.dstate + kRedThreads - 1) / kRedThreads;
  hipLaunchKernelGGL(reduce_kernel, dim3(unsigned(nchan + nrow)), dim3(kRedThreads), 0, st, p,
                     a.dA, a.dB, a.dC, a.dDskip, a.dbias, d.batch, nchan);
  return int(hipGetLastError());
}

}  // namespace ss
