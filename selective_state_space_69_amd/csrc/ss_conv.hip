// Causal depthwise Conv1d + SiLU for gfx950: the step before the selective scan
// that turns the expanded input x into u (Gu & Dao wiki note, "Mamba
// architecture": Linear -> Conv1d -> SiLU -> SSM; "A Visual Guide to Mamba"
// summary, "Mamba block": a convolution before the selective SSM).
//
// Memory-bound streaming: each input is read once and each output written once.
// A thread takes VEC = 4 adjacent channels (one 8-byte bf16 or 16-byte fp32
// vector, so a wave moves 512 B or 1 KB of a (b, t) row) and walks a segment of
// 64 time steps with the last K - 1 inputs in registers; the taps, bias and
// window never leave registers.  Segments start K - 1 steps early (the halo)
// and are independent, so a launch has B * ceil(L / 64) * ceil(D / 1024)
// workgroups.  The backward walks the same segments with a K - 1 step halo on
// both sides: dx[s] = sum_k w[k] gp[s + K - 1 - k] needs the next K - 1 output
// gradients; per-segment partial sums of dw and dbias are added in a fixed order
// by a second kernel, so the result is deterministic.
#include "ss_device.hpp"

namespace ss {
namespace {

constexpr int kThreads = 256;
constexpr int kSeg = kConvSeg;        // time steps per segment

template <typename T, int VEC>
__device__ __forceinline__ void load_vec(const T* p, float (&v)[VEC]) {
  if constexpr (VEC == 4) {
    const float4 f = unpack4(*reinterpret_cast<const typename Raw4<T>::type*>(p));
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else {
    v[0] = to_f32(*p);
  }
}
// raw (undecoded) VEC channels of one row, and their decoding
template <typename T, int VEC>
struct RawV {
  using type = typename Raw4<T>::type;
};
template <typename T>
struct RawV<T, 1> {
  using type = T;
};
template <typename T, int VEC>
__device__ __forceinline__ typename RawV<T, VEC>::type load_raw_vec(const T* p) {
  if constexpr (VEC == 4) return *reinterpret_cast<const typename Raw4<T>::type*>(p);
  else return *p;
}
template <typename T, int VEC>
__device__ __forceinline__ void unpack_raw_vec(typename RawV<T, VEC>::type r, float (&v)[VEC]) {
  if constexpr (VEC == 4) {
    const float4 f = unpack4(r);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else {
    v[0] = to_f32(r);
  }
}
__device__ __forceinline__ void load_f32(const float* p, float (&v)[4]) {
  const float4 f = *reinterpret_cast<const float4*>(p);
  v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
}
__device__ __forceinline__ void load_f32(const float* p, float (&v)[1]) { v[0] = *p; }

template <typename T, int VEC>
__device__ __forceinline__ void store_vec(T* p, const float (&v)[VEC]) {
  if constexpr (VEC == 4) {
    if constexpr (sizeof(T) == 4) {
      *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      uint2 w;
      w.x = uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16);
      w.y = uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16);
      *reinterpret_cast<uint2*>(p) = w;
    }
  } else {
    store_out<T>(p, v[0]);
  }
}

__device__ __forceinline__ float sigmoid(float p) { return hw_rcp(1.0f + hw_exp2(-p * kLog2e)); }

struct ConvParams {
  const void* x;
  const float* w;      // (D, K)
  const float* bias;   // (D) or null
  void* u;             // fwd output
  const float* du;     // bwd input
  float* dx;
  float* pdw;          // (B * nseg, D, K) partial dw
  float* pdb;          // (B * nseg, D) partial dbias
  int64_t L, D;
  int32_t nseg, ncblk;
};

// block index -> (b, segment, channel block); thread -> first channel
struct Where {
  int64_t b;
  int32_t seg;
  int64_t c0;
  bool active;
};
template <int VEC>
__device__ __forceinline__ Where where(const ConvParams& p) {
  int64_t bid = blockIdx.x;
  const int cblk = int(bid % p.ncblk);
  bid /= p.ncblk;
  Where w;
  w.seg = int32_t(bid % p.nseg);
  w.b = bid / p.nseg;
  w.c0 = (int64_t(cblk) * kThreads + threadIdx.x) * VEC;
  w.active = w.c0 < p.D;
  return w;
}

template <typename In, typename Out, int VEC, int K, bool SILU>
__global__ __launch_bounds__(kThreads) void conv_fwd_kernel(ConvParams p) {
  const Where at = where<VEC>(p);
  if (!at.active) return;
  const In* x = static_cast<const In*>(p.x) + at.b * p.L * p.D + at.c0;
  Out* u = static_cast<Out*>(p.u) + at.b * p.L * p.D + at.c0;
  float w[K][VEC], bias[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    bias[j] = p.bias ? p.bias[at.c0 + j] : 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) w[k][j] = p.w[(at.c0 + j) * K + k];
  }
  const int64_t t0 = int64_t(at.seg) * kSeg;
  const int64_t t1 = t0 + kSeg < p.L ? t0 + kSeg : p.L;
  float win[K][VEC];   // win[k] = x[t - K + 1 + k]; win[K-1] is the current step
#pragma unroll
  for (int k = 0; k < K - 1; ++k) {
    const int64_t tt = t0 - (K - 1) + k;
    if (tt >= 0) load_vec<In, VEC>(x + tt * p.D, win[k]);
    else
#pragma unroll
      for (int j = 0; j < VEC; ++j) win[k][j] = 0.0f;
  }
  // the segment in blocks of kPf steps; the raw rows of the next block are
  // fetched while the current one is computed, so loads stay in flight
  constexpr int kPf = 8;
  using R = typename RawV<In, VEC>::type;
  R buf[2][kPf];
  auto fetch = [&](R (&dst)[kPf], int64_t tb) {
#pragma unroll
    for (int i = 0; i < kPf; ++i) {
      const int64_t t = tb + i < t1 ? tb + i : t1 - 1;
      dst[i] = load_raw_vec<In, VEC>(x + t * p.D);
    }
  };
  fetch(buf[0], t0);
#pragma unroll
  for (int blk = 0; blk < kSeg / kPf; ++blk) {
    const int64_t tb = t0 + int64_t(blk) * kPf;
    if (tb >= t1) break;                            // uniform: the segment's end
    if (blk + 1 < kSeg / kPf && tb + kPf < t1) fetch(buf[(blk + 1) & 1], tb + kPf);
#pragma unroll
    for (int i = 0; i < kPf; ++i) {
      const int64_t t = tb + i;
      if (t >= t1) break;
      unpack_raw_vec<In, VEC>(buf[blk & 1][i], win[K - 1]);
      float o[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        float s = bias[j];
#pragma unroll
        for (int k = 0; k < K; ++k) s = __builtin_fmaf(w[k][j], win[k][j], s);
        o[j] = SILU ? s * sigmoid(s) : s;
      }
      store_vec<Out, VEC>(u + t * p.D, o);
#pragma unroll
      for (int k = 0; k < K - 1; ++k)
#pragma unroll
        for (int j = 0; j < VEC; ++j) win[k][j] = win[k + 1][j];
    }
  }
}

template <typename In, int VEC, int K, bool SILU>
__global__ __launch_bounds__(kThreads) void conv_bwd_kernel(ConvParams p) {
  const Where at = where<VEC>(p);
  if (!at.active) return;
  const int64_t base = at.b * p.L * p.D + at.c0;
  const In* x = static_cast<const In*>(p.x) + base;
  const float* du = p.du + base;
  float* dx = p.dx + base;
  float w[K][VEC], bias[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    bias[j] = p.bias ? p.bias[at.c0 + j] : 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) w[k][j] = p.w[(at.c0 + j) * K + k];
  }
  const int64_t t0 = int64_t(at.seg) * kSeg;
  const int64_t t1 = t0 + kSeg < p.L ? t0 + kSeg : p.L;
  float win[K][VEC];   // x[t - K + 1 + k]
  float gw[K][VEC];    // gw[k] = gp[t - K + 1 + k]: the last K pre-activation gradients
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int j = 0; j < VEC; ++j) { win[k][j] = 0.0f; gw[k][j] = 0.0f; }
#pragma unroll
  for (int k = 0; k < K - 1; ++k) {
    const int64_t tt = t0 - (K - 1) + k;
    if (tt >= 0) load_vec<In, VEC>(x + tt * p.D, win[k]);
  }
  float dw[K][VEC], db[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    db[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) dw[k][j] = 0.0f;
  }
  // t runs over the segment and K - 1 steps past it (dx of the segment's last
  // steps needs those output gradients); steps at or past L contribute nothing
  const int64_t tend = t1 + K - 1;
#pragma unroll 4
  for (int64_t t = t0; t < tend; ++t) {
    float g[VEC];
    if (t < p.L) {
      load_vec<In, VEC>(x + t * p.D, win[K - 1]);
      float d[VEC];
      load_f32(du + t * p.D, d);
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        float s = bias[j];
#pragma unroll
        for (int k = 0; k < K; ++k) s = __builtin_fmaf(w[k][j], win[k][j], s);
        if (SILU) {
          const float sg = sigmoid(s);
          g[j] = d[j] * sg * __builtin_fmaf(s, 1.0f - sg, 1.0f);   // silu'(s)
        } else {
          g[j] = d[j];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < VEC; ++j) g[j] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < K - 1; ++k)
#pragma unroll
      for (int j = 0; j < VEC; ++j) gw[k][j] = gw[k + 1][j];
#pragma unroll
    for (int j = 0; j < VEC; ++j) gw[K - 1][j] = g[j];
    if (t < t1) {
      // tap k of output t read x[t - K + 1 + k]
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        db[j] += g[j];
#pragma unroll
        for (int k = 0; k < K; ++k) dw[k][j] = __builtin_fmaf(g[j], win[k][j], dw[k][j]);
      }
    }
    const int64_t s = t - (K - 1);       // dx[s] = sum_k w[k] gp[s + K - 1 - k] = sum_k w[k] gw[K-1-k]
    if (s >= t0 && s < t1) {
      float o[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        float a = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) a = __builtin_fmaf(w[k][j], gw[K - 1 - k][j], a);
        o[j] = a;
      }
      store_vec<float, VEC>(dx + s * p.D, o);
    }
#pragma unroll
    for (int k = 0; k < K - 1; ++k)
#pragma unroll
      for (int j = 0; j < VEC; ++j) win[k][j] = win[k + 1][j];
  }
  const int64_t part = at.b * p.nseg + at.seg;
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    if (p.pdb) p.pdb[part * p.D + at.c0 + j] = db[j];
#pragma unroll
    for (int k = 0; k < K; ++k) p.pdw[(part * p.D + at.c0 + j) * K + k] = dw[k][j];
  }
}

// dw (D, K) and dbias (D): sums over the B * nseg segment partials.  A
// workgroup takes 64 outputs and splits the terms over 4 thread groups, each
// with 4 interleaved running sums; every addition happens in a fixed order.
constexpr int kRedCols = 64, kRedGroups = 4;
__global__ __launch_bounds__(kRedCols * kRedGroups) void conv_reduce_kernel(
    const float* __restrict__ pdw, const float* __restrict__ pdb, float* __restrict__ dw,
    float* __restrict__ db, int64_t parts, int64_t D, int K) {
  __shared__ float part[kRedGroups][kRedCols];
  const int c = int(threadIdx.x) % kRedCols, g = int(threadIdx.x) / kRedCols;
  const int64_t gid = int64_t(blockIdx.x) * kRedCols + c;
  const int64_t nw = D * K;
  const bool valid = gid < nw + (db ? D : 0);
  const bool isw = gid < nw;
  float s = 0.0f;
  if (valid) {
    const float* src = isw ? pdw + gid : pdb + (gid - nw);
    const int64_t stride = isw ? nw : D;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int64_t k = g;
    for (; k + 3 * kRedGroups < parts; k += 4 * kRedGroups) {
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m] += src[(k + m * kRedGroups) * stride];
    }
    for (int m = 0; k < parts; k += kRedGroups, ++m) acc[m] += src[k * stride];
    s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  }
  part[g][c] = s;
  __syncthreads();
  if (g != 0 || !valid) return;
  const float t = (part[0][c] + part[1][c]) + (part[2][c] + part[3][c]);
  if (isw) dw[gid] = t;
  else db[gid - nw] = t;
}

// One decode step per (b, d): window [state, x], state shifts by one.
template <typename In, typename Out, int K, bool SILU>
__global__ __launch_bounds__(256) void conv_step_kernel(float* __restrict__ state, const In* x,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ bias, Out* u,
                                                        int64_t B, int64_t D) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= B * D) return;
  const int64_t d = gid % D;
  float* st = state + gid * (K - 1);
  const float xv = to_f32(x[gid]);
  float s = bias ? bias[d] : 0.0f;
  float win[K];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) win[k] = st[k];
  win[K - 1] = xv;
#pragma unroll
  for (int k = 0; k < K; ++k) s = __builtin_fmaf(w[d * K + k], win[k], s);
#pragma unroll
  for (int k = 0; k < K - 1; ++k) st[k] = win[k + 1];
  store_out<Out>(u + gid, SILU ? s * sigmoid(s) : s);
}

template <template <int, bool> class F, typename... Args>
hipError_t by_width(int K, bool silu, Args... args) {
  switch (K) {
    case 1: return silu ? F<1, true>::go(args...) : F<1, false>::go(args...);
    case 2: return silu ? F<2, true>::go(args...) : F<2, false>::go(args...);
    case 3: return silu ? F<3, true>::go(args...) : F<3, false>::go(args...);
    default: return silu ? F<4, true>::go(args...) : F<4, false>::go(args...);
  }
}

template <typename In, typename Out, int VEC>
struct FwdL {
  template <int K, bool S>
  struct At {
    static hipError_t go(const ConvParams& p, dim3 g, hipStream_t st) {
      hipLaunchKernelGGL((conv_fwd_kernel<In, Out, VEC, K, S>), g, dim3(kThreads), 0, st, p);
      return hipGetLastError();
    }
  };
};
template <typename In, int VEC>
struct BwdL {
  template <int K, bool S>
  struct At {
    static hipError_t go(const ConvParams& p, dim3 g, hipStream_t st) {
      hipLaunchKernelGGL((conv_bwd_kernel<In, VEC, K, S>), g, dim3(kThreads), 0, st, p);
      return hipGetLastError();
    }
  };
};
template <typename In, typename Out>
struct StepL {
  template <int K, bool S>
  struct At {
    static hipError_t go(float* state, const void* x, const float* w, const float* bias, void* u,
                         int64_t B, int64_t D, hipStream_t st) {
      hipLaunchKernelGGL((conv_step_kernel<In, Out, K, S>), dim3(unsigned((B * D + 255) / 256)),
                         dim3(256), 0, st, state, static_cast<const In*>(x), w, bias,
                         static_cast<Out*>(u), B, D);
      return hipGetLastError();
    }
  };
};

ConvParams make_params(const ss_conv_desc_t& d, const ConvPlan& plan) {
  ConvParams p{};
  p.L = d.seqlen;
  p.D = d.dim;
  p.nseg = int32_t(plan.nseg);
  p.ncblk = int32_t((d.dim + kThreads * plan.vec - 1) / (kThreads * plan.vec));
  return p;
}

template <typename In, typename Out>
hipError_t fwd_typed(const ss_conv_desc_t& d, const ConvPlan& plan, const ConvParams& p,
                     hipStream_t st) {
  const dim3 g(unsigned(d.batch * p.nseg * p.ncblk));
  if (plan.vec == 4) return by_width<FwdL<In, Out, 4>::template At>(d.width, d.silu != 0, p, g, st);
  return by_width<FwdL<In, Out, 1>::template At>(d.width, d.silu != 0, p, g, st);
}

template <typename In>
hipError_t bwd_typed(const ss_conv_desc_t& d, const ConvPlan& plan, const ConvParams& p,
                     hipStream_t st) {
  const dim3 g(unsigned(d.batch * p.nseg * p.ncblk));
  if (plan.vec == 4) return by_width<BwdL<In, 4>::template At>(d.width, d.silu != 0, p, g, st);
  return by_width<BwdL<In, 1>::template At>(d.width, d.silu != 0, p, g, st);
}

template <typename In, typename Out>
hipError_t step_typed(const ss_conv_desc_t& d, float* state, const void* x, const float* w,
                      const float* bias, void* u, hipStream_t st) {
  return by_width<StepL<In, Out>::template At>(d.width, d.silu != 0, state, x, w, bias, u,
                                               d.batch, d.dim, st);
}

}  // namespace

int launch_conv_fwd(const ss_conv_desc_t& d, const ConvPlan& plan, const void* x, const float* w,
                    const float* bias, void* u, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  ConvParams p = make_params(d, plan);
  p.x = x; p.w = w; p.bias = bias; p.u = u;
  hipError_t e;
  if (d.in_dtype == SS_BF16)
    e = d.out_dtype == SS_BF16 ? fwd_typed<uint16_t, uint16_t>(d, plan, p, st)
                               : fwd_typed<uint16_t, float>(d, plan, p, st);
  else
    e = d.out_dtype == SS_BF16 ? fwd_typed<float, uint16_t>(d, plan, p, st)
                               : fwd_typed<float, float>(d, plan, p, st);
  return int(e);
}

int launch_conv_bwd(const ss_conv_desc_t& d, const ConvPlan& plan, const void* x, const float* w,
                    const float* bias, const float* du, float* dx, float* dw, float* dbias,
                    char* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  ConvParams p = make_params(d, plan);
  p.x = x; p.w = w; p.bias = bias; p.du = du; p.dx = dx;
  p.pdw = reinterpret_cast<float*>(ws + plan.off_dw);
  p.pdb = dbias ? reinterpret_cast<float*>(ws + plan.off_db) : nullptr;
  hipError_t e = d.in_dtype == SS_BF16 ? bwd_typed<uint16_t>(d, plan, p, st)
                                       : bwd_typed<float>(d, plan, p, st);
  if (e != hipSuccess) return int(e);
  const int64_t parts = d.batch * plan.nseg;
  const int64_t outs = d.dim * d.width + (dbias ? d.dim : 0);
  hipLaunchKernelGGL(conv_reduce_kernel, dim3(unsigned((outs + kRedCols - 1) / kRedCols)),
                     dim3(kRedCols * kRedGroups), 0, st, p.pdw, p.pdb, dw, dbias, parts, d.dim,
                     int(d.width));
  return int(hipGetLastError());
}

int launch_conv_step(const ss_conv_desc_t& d, float* state, const void* x, const float* w,
                     const float* bias, void* u, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (d.in_dtype == SS_BF16)
    e = d.out_dtype == SS_BF16 ? step_typed<uint16_t, uint16_t>(d, state, x, w, bias, u, st)
                               : step_typed<uint16_t, float>(d, state, x, w, bias, u, st);
  else
    e = d.out_dtype == SS_BF16 ? step_typed<float, uint16_t>(d, state, x, w, bias, u, st)
                               : step_typed<float, float>(d, state, x, w, bias, u, st);
  return int(e);
}

}  // namespace ss
