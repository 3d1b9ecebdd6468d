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
// so address arithmetic stays on the scalar unit.  Range checking is disabled
// (num_records = max); callers keep every access inside its tensor.
using Rsrc = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ Rsrc make_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), short(0), -1, 0x00020000);
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

// Element types: fp32, or bf16 carried as its raw uint16 bit pattern.
template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) {
  return __uint_as_float(uint32_t(x) << 16);
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
// x2 = x * log2(e), written as max(x2, 0) + log2(1 + 2^-|x2|).  The log of
// 1 + e is corrected for the rounding of 1 + e (log1p by the Goldberg/Kahan
// trick log(u) * e / (u - 1)), so small steps keep full relative accuracy.
__device__ __forceinline__ float softplus_log2(float x2) {
  const float e = hw_exp2(-__builtin_fabsf(x2));
  const float u1 = 1.0f + e;
  const float dm = __builtin_fmaxf(u1 - 1.0f, 0x1p-100f);
  return __builtin_fmaxf(x2, 0.0f) + hw_log2(u1) * (e * hw_rcp(dm));
}

// silu(z) = z * sigmoid(z) = z / (1 + 2^(-z log2 e)); saturates cleanly at +-inf.
__device__ __forceinline__ float silu(float z) {
  return z * hw_rcp(1.0f + hw_exp2(-z * kLog2e));
}

// One row of B or C (N values, N <= 16) for a time step.  The row is the same
// for every lane of the wave, so it is read through the constant address space:
// scalar loads into SGPRs (bf16 unpacked by scalar shifts), which the vector
// FMAs then take as free operands.  Raw dwords are kept so the load for the next
// step can be issued one step ahead.  Unused states read 0.
using ConstU32 = __attribute__((address_space(4))) const uint32_t;

template <typename In>
struct RowRaw {
  uint32_t w[sizeof(In) == 2 ? kMaxState / 2 : kMaxState];
};

template <typename In, bool FULLN>
__device__ __forceinline__ void load_row_raw(const In* base, int64_t row, int N, RowRaw<In>& r) {
  constexpr int kW = sizeof(In) == 2 ? kMaxState / 2 : kMaxState;
  if constexpr (FULLN) {
    ConstU32* q = (ConstU32*)(base + row * kMaxState);  // generic -> constant address space
#pragma unroll
    for (int k = 0; k < kW; ++k) r.w[k] = q[k];
  } else {
    // generic N: element loads, packed into the same raw layout
#pragma unroll
    for (int k = 0; k < kW; ++k) r.w[k] = 0;
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) {
      if (n < N) {
        if constexpr (sizeof(In) == 2) {
          const uint32_t v = reinterpret_cast<const uint16_t*>(base)[row * N + n];
          r.w[n >> 1] |= (n & 1) ? (v << 16) : v;
        } else {
          r.w[n] = reinterpret_cast<const uint32_t*>(base)[row * N + n];
        }
      }
    }
  }
}

template <typename In>
__device__ __forceinline__ void unpack_row(const RowRaw<In>& r, float (&v)[kMaxState]) {
  if constexpr (sizeof(In) == 2) {
#pragma unroll
    for (int k = 0; k < kMaxState / 2; ++k) {
      v[2 * k] = __uint_as_float(r.w[k] << 16);
      v[2 * k + 1] = __uint_as_float(r.w[k] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int k = 0; k < kMaxState; ++k) v[k] = __uint_as_float(r.w[k]);
  }
}

}  // namespace ss
