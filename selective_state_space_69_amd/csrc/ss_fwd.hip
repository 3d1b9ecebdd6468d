// Forward selective scan for gfx950.
//
// Mapping: one wavefront per (batch row b, block of 64 channels, time chunk).
// Lane = channel d.  Each lane keeps its channel's N <= 16 fp32 states in VGPRs
// and walks its time range sequentially; every (b, t) row of B and C is shared
// by all channels (Broadcast over D: "A Survey of Mamba" summary, Selection), so
// the row is the same for the whole wave and sits in SGPRs.  Per element
// (b, t, d, n) the work is one v_exp_f32 and 4 (Euler) or 6 (exact ZOH) vector
// ops; the discretised A_bar, B_bar and the states never touch memory
// ("A Visual Guide to Mamba" summary, Hardware-aware Algorithm: discretisation,
// scan and the C contraction fused in one kernel).
//
// Long or narrow problems are cut into time chunks (two-level carry):
//   1. summary pass: per chunk, the zero-start end state S and the summed step
//      sum(dt) (the chunk decay is exp(A * sum(dt)));
//   2. carry scan: start state of chunk c+1 = exp(A sum_c) * start_c + S_c, the
//      associative combine (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2) applied
//      left to right ("A Visual Guide to Mamba" summary, The Scan Operation);
//   3. output pass: each chunk re-runs from its true start state and writes y.
#include "ss_device.hpp"

namespace ss {
namespace {

constexpr int kZoh = SS_ZOH;
constexpr int kEuler = SS_EULER;
constexpr int kPrefetch = 8;  // time steps of u, delta, z in flight per lane

struct FwdParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  const float* bias;
  const void* z;
  const float* h0;
  void* y;
  float* h_last;
  float* hend;   // (B, nchunks, N, D)
  float* dsum;   // (B, nchunks, D)
  int64_t L, D;
  int64_t chunk_len;
  int32_t N, ndblk, nchunks, grid_chunks;
};

// Per-lane constants of a channel.
struct Chan {
  float A[kMaxState];    // diagonal A[d, n]; unused states get -1 (inert: B = C = 0)
  float iA[kMaxState];   // 1 / A (0 where A == 0)
  float zm[kMaxState];   // 1 where A == 0 (exact ZOH falls back to dt * B there)
};

template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY, bool SAFE,
          bool FULLN>
__device__ __forceinline__ void scan_range(const FwdParams& p, const Chan& ch, float (&h)[kMaxState],
                                           int64_t b, int64_t dblk, uint32_t lane_c, bool active,
                                           int32_t t0, int32_t t1, float Dd, float bias2,
                                           float& dsum) {
  const int64_t D = p.D;
  const int N = FULLN ? kMaxState : p.N;
  constexpr uint32_t kIn = sizeof(In), kOut = sizeof(Out);
  const uint32_t rowb_in = uint32_t(D) * kIn;      // bytes between time steps
  const uint32_t rowb_out = uint32_t(D) * kOut;
  const uint32_t vin = lane_c * kIn, vout = lane_c * kOut;
  // wave-uniform pointers of (b, t = 0, d = 64 * dblk)
  const int64_t base = b * p.L * D + dblk * kWave;
  const In* ub = static_cast<const In*>(p.u) + base;
  const In* db = static_cast<const In*>(p.delta) + base;
  const In* zb = HAS_Z ? static_cast<const In*>(p.z) + base : nullptr;
  Out* yb = SUMMARY ? nullptr : static_cast<Out*>(p.y) + base;
  const In* Bp = static_cast<const In*>(p.Bm);
  const In* Cp = static_cast<const In*>(p.Cm);
  const int64_t row0 = b * p.L;
  const int32_t tlast = t1 - 1;

  // prefetch ring of u, delta, z, kPrefetch steps deep (indices clamped to the
  // last step of the range, so every load is in bounds)
  In ur[kPrefetch], dr[kPrefetch], zr[kPrefetch];
  {
    const Rsrc ru = make_rsrc(ub + int64_t(t0) * D), rd = make_rsrc(db + int64_t(t0) * D);
    const Rsrc rz = make_rsrc(HAS_Z ? zb + int64_t(t0) * D : ub);
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
      const int32_t tt = t0 + k < tlast ? t0 + k : tlast;
      const uint32_t so = uint32_t(tt - t0) * rowb_in;
      ur[k] = buf_load<In>(ru, vin, so);
      dr[k] = buf_load<In>(rd, vin, so);
      if (HAS_Z && !SUMMARY) zr[k] = buf_load<In>(rz, vin, so);
    }
  }
  RowRaw<In> bn, cn;
  load_row_raw<In, FULLN>(Bp, row0 + t0, N, bn);
  if (!SUMMARY) load_row_raw<In, FULLN>(Cp, row0 + t0, N, cn);

  // Time steps run in blocks of kPrefetch; steps past t1 (only in a ragged
  // last block) get dt = 0, which leaves the state unchanged, and store nothing.
  for (int32_t t = t0; t < t1; t += kPrefetch) {
    const Rsrc ru = make_rsrc(ub + int64_t(t) * D), rd = make_rsrc(db + int64_t(t) * D);
    const Rsrc rz = make_rsrc(HAS_Z ? zb + int64_t(t) * D : ub);
    const Rsrc ry = make_rsrc(SUMMARY ? static_cast<const void*>(ub) : static_cast<const void*>(yb + int64_t(t) * D));
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
      const int32_t tt = t + k;
      const bool valid = tt < t1;                       // wave-uniform
      const float uf = to_f32(ur[k]);
      const float df = to_f32(dr[k]);
      const float zf = (HAS_Z && !SUMMARY) ? to_f32(zr[k]) : 0.0f;
      {
        const int32_t tn = tt + kPrefetch < tlast ? tt + kPrefetch : tlast;
        const uint32_t so = uint32_t(tn - t) * rowb_in;
        ur[k] = buf_load<In>(ru, vin, so);
        dr[k] = buf_load<In>(rd, vin, so);
        if (HAS_Z && !SUMMARY) zr[k] = buf_load<In>(rz, vin, so);
      }
      float Bv[kMaxState], Cv[kMaxState];
      unpack_row(bn, Bv);
      if (!SUMMARY) unpack_row(cn, Cv);
      {
        const int32_t tn = tt + 1 < tlast ? tt + 1 : tlast;
        load_row_raw<In, FULLN>(Bp, row0 + tn, N, bn);
        if (!SUMMARY) load_row_raw<In, FULLN>(Cp, row0 + tn, N, cn);
      }

      float dl;                                          // dt * log2(e)
      if (SOFTPLUS) {
        const float x2 = valid ? __builtin_fmaf(df, kLog2e, bias2) : -__builtin_inff();
        dl = softplus_log2(x2);
      } else {
        dl = valid ? __builtin_fmaf(df, kLog2e, bias2) : 0.0f;
      }
      float acc0 = 0.0f, acc1 = 0.0f;
      if (DISC == kEuler) {
        const float dtu = dl * (kLn2 * uf);              // dt * u
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) {
          const float a = hw_exp2(dl * ch.A[n]);         // A_bar = exp(dt A)
          h[n] = __builtin_fmaf(a, h[n], dtu * Bv[n]);   // + dt B u
          if (!SUMMARY) {
            if (n & 1) acc1 = __builtin_fmaf(Cv[n], h[n], acc1);
            else acc0 = __builtin_fmaf(Cv[n], h[n], acc0);
          }
        }
      } else {
        const float dt = SAFE ? dl * kLn2 : 0.0f;
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) {
          const float a = hw_exp2(dl * ch.A[n]);              // A_bar = exp(dt A)
          float coef = __builtin_fmaf(a, ch.iA[n], -ch.iA[n]);  // (A_bar - 1) / A
          if (SAFE) coef = __builtin_fmaf(dt, ch.zm[n], coef);  // dt where A == 0
          h[n] = __builtin_fmaf(a, h[n], coef * (Bv[n] * uf));
          if (!SUMMARY) {
            if (n & 1) acc1 = __builtin_fmaf(Cv[n], h[n], acc1);
            else acc0 = __builtin_fmaf(Cv[n], h[n], acc0);
          }
        }
      }
      if (SUMMARY) {
        dsum += dl;
      } else {
        float yv = __builtin_fmaf(Dd, uf, acc0 + acc1);      // C h + D u
        if (HAS_Z) yv *= silu(zf);                            // gate
        if (active && valid) buf_store<Out>(ry, vout, uint32_t(k) * rowb_out, yv);
      }
    }
  }
}

template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY>
__global__ __launch_bounds__(kWave) void fwd_kernel(FwdParams p) {
  const int lane = threadIdx.x;
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

  Chan ch;
  bool zero = false;
#pragma unroll
  for (int n = 0; n < kMaxState; ++n) {
    const float a = n < N ? p.A[dc * N + n] : -1.0f;
    ch.A[n] = a;
    ch.iA[n] = a == 0.0f ? 0.0f : 1.0f / a;
    ch.zm[n] = a == 0.0f ? 1.0f : 0.0f;
    zero |= (a == 0.0f);
  }
  const float Dd = p.Dskip ? p.Dskip[dc] : 0.0f;
  const float bias2 = (p.bias ? p.bias[dc] : 0.0f) * kLog2e;

  float h[kMaxState];
  if (SUMMARY) {
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) h[n] = 0.0f;
  } else if (chunk == 0) {
#pragma unroll
    for (int n = 0; n < kMaxState; ++n)
      h[n] = (p.h0 && n < N) ? p.h0[(b * p.D + dc) * N + n] : 0.0f;
  } else {
    const float* hs = p.hend + (b * p.nchunks + chunk) * int64_t(N) * p.D + dc;
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) h[n] = n < N ? hs[int64_t(n) * p.D] : 0.0f;
  }

  float dsum = 0.0f;
  // exact ZOH needs the dt * B fallback only where some A entry is exactly 0
  const bool safe = DISC == kZoh && __any(zero);
  if (N == kMaxState) {
    if (safe)
      scan_range<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, true, true>(p, ch, h, b, dblk, lane_c, active, t0, t1, Dd, bias2, dsum);
    else
      scan_range<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, false, true>(p, ch, h, b, dblk, lane_c, active, t0, t1, Dd, bias2, dsum);
  } else {
    // N < 16: unused states carry A = -1 and B = C = 0; always the guarded ZOH form
    scan_range<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY, DISC == kZoh, false>(p, ch, h, b, dblk, lane_c, active, t0, t1, Dd, bias2, dsum);
  }

  if (!active) return;
  if (SUMMARY) {
    float* hs = p.hend + (b * p.nchunks + chunk) * int64_t(N) * p.D + d;
#pragma unroll
    for (int n = 0; n < kMaxState; ++n)
      if (n < N) hs[int64_t(n) * p.D] = h[n];
    p.dsum[(b * p.nchunks + chunk) * p.D + d] = dsum;
  } else if (p.h_last && t1 == p.L) {
#pragma unroll
    for (int n = 0; n < kMaxState; ++n)
      if (n < N) p.h_last[(b * p.D + d) * N + n] = h[n];
  }
}

// Carry scan over chunks, one lane per (b, n, d).  In place on hend: slot c of
// a chunk summary becomes the start state of chunk c (slot 0 is unused: chunk 0
// starts from h0).  The decay of chunk c is exp2(A * sum of dt*log2e).
__global__ __launch_bounds__(256) void carry_scan_kernel(float* __restrict__ hend,
                                                         const float* __restrict__ dsum,
                                                         const float* __restrict__ A,
                                                         const float* __restrict__ h0,
                                                         int64_t B, int64_t D, int N, int nchunks) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = B * N * D;
  if (gid >= total) return;
  const int64_t d = gid % D;
  const int n = int((gid / D) % N);
  const int64_t b = gid / (D * N);
  const float a = A[d * N + n];
  float carry = h0 ? h0[(b * D + d) * N + n] : 0.0f;
  const int64_t sstride = int64_t(N) * D;
  float* hs = hend + (b * nchunks) * sstride + int64_t(n) * D + d;
  const float* ds = dsum + (b * nchunks) * D + d;
  int c = 0;
  for (; c + 4 <= nchunks - 1; c += 4) {
    float S[4], P[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      S[k] = hs[(c + k) * sstride];
      P[k] = hw_exp2(a * ds[(c + k) * D]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (c + k >= 1) hs[(c + k) * sstride] = carry;
      carry = __builtin_fmaf(P[k], carry, S[k]);
    }
  }
  for (; c < nchunks - 1; ++c) {
    const float S = hs[c * sstride];
    const float P = hw_exp2(a * ds[c * D]);
    if (c >= 1) hs[c * sstride] = carry;
    carry = __builtin_fmaf(P, carry, S);
  }
  hs[(nchunks - 1) * sstride] = carry;
}

template <typename In, typename Out, int DISC, bool HAS_Z, bool SOFTPLUS, bool SUMMARY>
hipError_t launch_one(const FwdParams& p, int64_t nblocks, hipStream_t st) {
  hipLaunchKernelGGL((fwd_kernel<In, Out, DISC, HAS_Z, SOFTPLUS, SUMMARY>), dim3(unsigned(nblocks)),
                     dim3(kWave), 0, st, p);
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

hipError_t dispatch(const ss_desc_t& d, const FwdParams& p, bool summary, int64_t nblocks,
                    hipStream_t st) {
  const bool has_z = p.z != nullptr, sp = d.delta_softplus != 0;
  if (d.in_dtype == SS_BF16) {
    if (summary || d.out_dtype == SS_F32)
      return dispatch_disc<uint16_t, float>(p, d.disc, has_z, sp, summary, nblocks, st);
    return dispatch_disc<uint16_t, uint16_t>(p, d.disc, has_z, sp, summary, nblocks, st);
  }
  if (summary || d.out_dtype == SS_F32)
    return dispatch_disc<float, float>(p, d.disc, has_z, sp, summary, nblocks, st);
  return dispatch_disc<float, uint16_t>(p, d.disc, has_z, sp, summary, nblocks, st);
}

}  // namespace

int launch_fwd(const ss_desc_t& d, const FwdPlan& plan, const FwdArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  FwdParams p{};
  p.u = a.u; p.delta = a.delta; p.A = a.A; p.Bm = a.Bm; p.Cm = a.Cm;
  p.Dskip = a.Dskip; p.bias = a.bias; p.z = a.z; p.h0 = a.h0;
  p.y = a.y; p.h_last = a.h_last; p.hend = a.hend; p.dsum = a.dsum;
  p.L = d.seqlen; p.D = d.dim; p.N = int32_t(d.dstate);
  p.chunk_len = plan.tp.chunk_len;
  p.nchunks = int32_t(plan.tp.nchunks);
  p.ndblk = int32_t((d.dim + kWave - 1) / kWave);
  const int64_t cols = d.batch * p.ndblk;
  if (p.nchunks > 1) {
    p.grid_chunks = p.nchunks - 1;   // the last chunk's summary is never needed
    hipError_t e = dispatch(d, p, true, cols * p.grid_chunks, st);
    if (e != hipSuccess) return int(e);
    const int64_t total = d.batch * d.dstate * d.dim;
    hipLaunchKernelGGL(carry_scan_kernel, dim3(unsigned((total + 255) / 256)), dim3(256), 0, st,
                       a.hend, a.dsum, a.A, a.h0, d.batch, d.dim, int(d.dstate), p.nchunks);
    e = hipGetLastError();
    if (e != hipSuccess) return int(e);
  }
  p.grid_chunks = p.nchunks;
  return int(dispatch(d, p, false, cols * p.grid_chunks, st));
}

}  // namespace ss
