// Device-side building blocks shared by the scan kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ss_internal.h"

namespace ss {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// Hardware transcendental instructions (v_exp_f32 = 2^x, v_log_f32 = log2 x,
// v_rcp_f32 = 1/x), about 1 ulp, issued at half the fp32 FMA rate on gfx950.
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Raw buffer access: a wave-uniform 64-bit base in a buffer resource (SGPRs),
// a 32-bit per-lane byte offset (VGPR) and a 32-bit uniform byte offset (SGPR),
// so address arithmetic stays on the scalar unit.  Callers keep every real
// access inside its tensor.
// An access whose total offset is >= 2^31 - 1 (num_records) is dropped (loads
// return 0): idle lanes store with kOutOfRange instead of branching.
using Rsrc = __amdgpu_buffer_rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ Rsrc make_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), short(0), 0x7fffffff, 0x00020000);
}
template <typename T> __device__ __forceinline__ T buf_load(Rsrc r, uint32_t voff, uint32_t soff);
template <> __device__ __forceinline__ uint16_t buf_load<uint16_t>(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
template <> __device__ __forceinline__ float buf_load<float>(Rsrc r, uint32_t voff, uint32_t soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
template <typename T> __device__ __forceinline__ void buf_store(Rsrc r, uint32_t voff, uint32_t soff, float v);
template <> __device__ __forceinline__ void buf_store<float>(Rsrc r, uint32_t voff, uint32_t soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
}

// Workgroups are handed to the 8 XCDs round-robin (workgroup i to XCD i % 8),
// and each XCD has its own L2.  This bijection on [0, G) gives each XCD a
// contiguous range of logical workgroup indices, so neighbours that share
// input lines (adjacent channel groups, the heads of one batch row) meet in
// one L2 instead of being fetched by every XCD.
__device__ __forceinline__ int64_t xcd_contiguous(int64_t i, int64_t G) {
  const int64_t xi = i % 8, q8 = G / 8, r8 = G % 8;
  return xi * q8 + (xi < r8 ? xi : r8) + i / 8;
}

// Element types: fp32, or bf16 carried as its raw uint16 bit pattern.
template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) {
  return __uint_as_float(uint32_t(x) << 16);
}

// Four consecutive elements (8 bytes of bf16 or 16 bytes of fp32): loaded in
// their storage form (Raw4), widened to fp32 where they are used, so that a
// prefetch does not make the wave wait for the load.
template <typename T> struct Raw4;
template <> struct Raw4<float> { using type = float4; };
template <> struct Raw4<uint16_t> { using type = uint2; };
template <typename T> __device__ __forceinline__ typename Raw4<T>::type load_raw4(const T* p) {
  return *reinterpret_cast<const typename Raw4<T>::type*>(p);
}
__device__ __forceinline__ float4 unpack4(float4 v) { return v; }
__device__ __forceinline__ float4 unpack4(uint2 w) {
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}

// fp32 -> bf16 with round-to-nearest-even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t x = __float_as_uint(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) return uint16_t((x >> 16) | 0x40u);
  x += 0x7fffu + ((x >> 16) & 1u);
  return uint16_t(x >> 16);
}

template <typename T> __device__ __forceinline__ void store_out(T* p, float v);
template <> __device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float v) {
  *p = f32_to_bf16(v);
}
template <> __device__ __forceinline__ void buf_store<uint16_t>(Rsrc r, uint32_t voff, uint32_t soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, voff, soff, 0);
}

// Step size in log2 units: softplus(x) * log2(e) = log2(1 + 2^x2) with
// x2 = x * log2(e), written as max(x2, 0) + log2(1 + e), e = 2^-|x2| in (0, 1].
// log1p without cancellation: u1 = fl(1 + e) and r = e - (u1 - 1) give
// 1 + e = u1 + r exactly (Fast2Sum, 1 >= e), so
// log2(1 + e) = log2(u1) + log2(1 + r / u1) = log2(u1) + r log2(e) / u1 to
// within (r / u1)^2 < 2^-48.  The correction needs 1/u1 only roughly: it is
// exact where it matters (u1 == 1, e < 2^-24, where the whole answer is
// r log2 e = e log2 e) and below 2^-24 of the result elsewhere, so 1/u1 is
// replaced by 2 - u1 (relative error (u1 - 1)^2 / u1).  Small steps keep full
// relative accuracy down to the smallest normal e.
__device__ __forceinline__ float softplus_log2(float x2) {
  const float e = hw_exp2(-__builtin_fabsf(x2));
  const float u1 = 1.0f + e;
  const float r = e - (u1 - 1.0f);                               // exact rounding error of u1
  const float k = __builtin_fmaf(-u1, kLog2e, 2.0f * kLog2e);    // log2(e) (2 - u1)
  return __builtin_fmaxf(x2, 0.0f) + __builtin_fmaf(r, k, hw_log2(u1));
}

// Exact-ZOH input coefficient coef = (exp(x) - 1) / A with x = dt A ("Mamba: S4
// epic upgrade", S4 intro: zero-order hold).  Formed as (Abar - 1) / A from the
// rounded Abar it carries an absolute error of about 2^-24 / |A|, harmless for
// |A| >= kWeakA but not below: states that decay that slowly take the guarded
// path, where |x| < kZohSeries uses the series dt (1 + x/2 + x^2/6 + x^3/24)
// (truncation < x^4 / 120 relative) and larger |x| the quotient (relative error
// about 2^-24 / |x| < 1.2e-6).  A == 0 falls in the series (coef = dt).  The
// series is evaluated in x2 = x log2 e, the exponential's own argument.
constexpr float kWeakA = 0.25f;
constexpr float kZohSeries = 0.05f;
// x2 = x log2 e (the argument the exponential already takes), dt = x2 ln2 / A
__device__ __forceinline__ float zoh_coef_guarded(float abar, float iA, float dt, float x2) {
  constexpr float l1 = kLn2 / 2.0f, l2 = kLn2 * kLn2 / 6.0f, l3 = kLn2 * kLn2 * kLn2 / 24.0f;
  const float ser = dt * __builtin_fmaf(x2, __builtin_fmaf(x2, __builtin_fmaf(x2, l3, l2), l1), 1.0f);
  const float quot = __builtin_fmaf(abar, iA, -iA);
  // a select, not a branch: the choice varies from lane to lane and step to step
  return __builtin_unpredictable(__builtin_fabsf(x2) < kZohSeries * kLog2e) ? ser : quot;
}
// Precise decay.  A state that a step barely decays (|x| = |dt A| small) is
// remembered for about 1/|x| steps, and A_bar = exp(x) rounded to fp32 is off
// by up to an ulp near 1 (~6e-8 absolute): that error compounds over the
// memory to about 6e-8/|x| of the state, which for a constant step and input
// of one sign leaves the fp32 bound at |x| ~ 1e-4.  The precise form carries
// the decay as E = exp(x) - 1 instead, h <- h + (E h + coef B u), with E from
// the series x (1 + x/2 + x^2/6 + x^3/24) where |x| < kZohSeries (truncation
// below x^4 / 120 relative) and exp2 - 1 elsewhere (there the memory is under
// 20 steps); the exact-ZOH input coefficient coef = E / A comes from the same
// series as dt (1 + x/2 + ...), so A == 0 gives coef = dt.  Everything is in
// the exponential's own argument y2 = x log2 e = d2 A, d2 = dt log2 e:
// exp(x) - 1 = y2 Q(y2) and coef = d2 Q(y2) with Q(y2) = ln2 P(y2 ln2).
constexpr float kSeries2 = kZohSeries * kLog2e;
__device__ __forceinline__ float expm1_factor(float y2) {
  constexpr float q0 = kLn2, q1 = kLn2 * kLn2 / 2.0f, q2 = kLn2 * kLn2 * kLn2 / 6.0f,
                  q3 = kLn2 * kLn2 * kLn2 * kLn2 / 24.0f;
  return __builtin_fmaf(y2, __builtin_fmaf(y2, __builtin_fmaf(y2, q3, q2), q1), q0);
}
// E = exp(x) - 1 for y2 = x log2 e, to full relative accuracy
__device__ __forceinline__ float precise_expm1(float y2) {
  const float a = hw_exp2(y2);
  const float ser = y2 * expm1_factor(y2);
  // a select, not a branch: the choice varies from lane to lane and step to step
  return __builtin_unpredictable(__builtin_fabsf(y2) < kSeries2) ? ser : a - 1.0f;
}
// E (returned) and, for exact ZOH, coef = E / A (with iA = 1 / A, 0 for A == 0)
template <bool ZOH>
__device__ __forceinline__ float precise_decay(float d2, float A, float iA, float& coef) {
  const float y2 = d2 * A;
  const float a = hw_exp2(y2);
  const float q = expm1_factor(y2);
  const bool small = __builtin_unpredictable(__builtin_fabsf(y2) < kSeries2);
  const float e = small ? y2 * q : a - 1.0f;
  if (ZOH) coef = small ? d2 * q : e * iA;
  return e;
}

// d coef / dA for |x| < kZohSeries: dt^2 (1/2 + x/3 + x^2/8 + x^3/30), the series
// of (x e^x - e^x + 1) / x^2 (truncation < x^4 / 144)
__device__ __forceinline__ float zoh_dcoef_series(float dt, float x) {
  return dt * dt *
         __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 30.0f, 0.125f), 1.0f / 3.0f),
                        0.5f);
}

// silu(z) = z * sigmoid(z) = z / (1 + 2^(-z log2 e)); saturates cleanly at +-inf.
__device__ __forceinline__ float silu(float z) {
  return z * hw_rcp(1.0f + hw_exp2(-z * kLog2e));
}

}  // namespace ss
