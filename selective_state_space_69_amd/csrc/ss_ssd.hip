// Structured state-space duality (SSD, Mamba-2) forward on the matrix cores.
//
// The layer ("A Survey of Mamba" summary, section Mamba-2): per batch row and
// head the SSM is y = M x with the semiseparable matrix
//     M[t][s] = C_t . B_s * exp(sum_{s<u<=t} dt_u A) * dt_s      (s <= t)
// plus the skip D x.  Cut time into chunks of Q = 64 steps.  Inside a chunk the
// block of M is dense and small (Q x Q): it is built from G = C B^T and applied
// to the chunk's x as matrix products.  Everything older reaches the chunk
// through the state H (N x P) at its start:
//     y_t  += exp(l_t) C_t . H                       (l_t: log decay since chunk start)
//     H    <- exp(l_end) H + sum_s exp(l_end - l_s) dt_s B_s x_s^T
// so a head walks its chunks in order with H on chip and reads each input once.
//
// One workgroup = one (batch row, head), 4 waves, P = N = 64.  Every product is
// a 64 x 64 x 64 contraction done with v_mfma_f32_16x16x32_bf16 tiles:
//   G^T = B C^T   (k = n)    M^T tiles land with one t and 4 consecutive s per
//                            lane: after the mask, a t-row of M is the A operand
//   Y   = M X     (k = s)    diagonal block
//   Y  += C H     (k = n)    off-diagonal part; H stays in its accumulator layout
//   H  += B^T X'  (k = s)    X' = x scaled by exp(l_end - l_s) dt_s
// Wave w owns t-tile w of M and Y (work 1..4 tiles of G) and p-tile w of H; the
// C H products of p-tile w are handed to the t-tile owners through LDS.
//
// Inputs are bf16 and enter the products exactly.  The operands the method
// computes (M, H, X') are split into bf16 hi + lo parts and multiplied twice,
// so each product carries about 16 significant bits per operand and fp32
// accumulation; the result tracks an fp32 evaluation (no bf16 rounding of
// intermediate values).
//
// K order: an MFMA A operand takes 8 consecutive k per lane (k = 8g..8g+7,
// g = lane / 16) while an accumulator holds 4 consecutive rows per lane
// (4g..4g+3).  Every contraction here therefore numbers its 32-wide k block j
// as (32j + 4g + 0..3, 32j + 16 + 4g + 0..3): the accumulator rows of two
// adjacent 16-row tiles are then exactly the k slots a lane must supply, for M
// (from the G^T tiles) and for H alike, and the LDS operands are read in the
// same order.
#include "ss_device.hpp"

namespace ss {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kQ = 64;          // chunk length
constexpr int kDim = 64;        // P = N = 64
constexpr int kNW = 4;          // waves per workgroup
constexpr int kThreads = kNW * kWave;

// LDS tiles: 64 rows of 16 units of 8 bytes (4 bf16).  Unit u of row r sits at
// u ^ (4 * ((r >> 2) & 3)): the operand reads (16 rows x units 8j+g), the
// row-major staging writes and the transposing staging writes all spread over
// the banks evenly.
struct Tile {
  uint2 u[kDim][16];
};
__device__ __forceinline__ int swz(int row, int unit) { return unit ^ (((row >> 2) & 3) << 2); }

struct Smem {
  Tile bs;                    // B rows   [s][n]
  Tile cs;                    // C rows   [t][n]
  Tile bt;                    // B^T      [n][s]
  Tile xt;                    // x^T      [p][s]
  f32x4 yo[4][4][kWave];      // exp(l_t) C H, [t-tile][p-tile][lane]
  float lam[kQ];              // l_t in log2 units (inclusive, from the chunk start)
  float dts[kQ];              // dt_t
};

// MFMA operand of k block j from row `row` of a tile: 8 bf16 at columns
// 32j + 4g .. +3 and 32j + 16 + 4g .. +3.
__device__ __forceinline__ u32x4 ld_op(const Tile& t, int row, int j, int g) {
  const uint2 a = t.u[row][swz(row, 8 * j + g)];
  const uint2 b = t.u[row][swz(row, 8 * j + 4 + g)];
  u32x4 r;
  r.x = a.x; r.y = a.y; r.z = b.x; r.w = b.y;
  return r;
}

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// hi + lo split of 8 fp32 values (k slot order) into two bf16 operands.
__device__ __forceinline__ void split8(const float (&v)[8], u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16(v[2 * i], v[2 * i + 1]);
    const float r0 = v[2 * i] - __uint_as_float(h[i] << 16);
    const float r1 = v[2 * i + 1] - __uint_as_float(h[i] & 0xffff0000u);
    l[i] = pack_bf16(r0, r1);
  }
  hi.x = h[0]; hi.y = h[1]; hi.z = h[2]; hi.w = h[3];
  lo.x = l[0]; lo.y = l[1]; lo.z = l[2]; lo.w = l[3];
}

__device__ __forceinline__ void bf16x8_to_f32(u32x4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp0(float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(src), CTRL, ROW_MASK, 0xf,
                                                    false));
}

// Inclusive sum over the 64 lanes: row_shr 1, 2, 4, 8 inside rows of 16, then
// row_bcast:15 and row_bcast:31 carry the row totals upwards.
__device__ __forceinline__ float wave_inclusive_sum(float v) {
  v += dpp0<0x111, 0xf>(v);
  v += dpp0<0x112, 0xf>(v);
  v += dpp0<0x114, 0xf>(v);
  v += dpp0<0x118, 0xf>(v);
  v += dpp0<0x142, 0xa>(v);
  v += dpp0<0x143, 0xc>(v);
  return v;
}

// 4 x 4 bf16 block: rows in[i] (cols 0,1 | cols 2,3) -> columns out[j] (rows 0,1 | rows 2,3).
__device__ __forceinline__ void transpose4(const uint2 (&in)[4], uint2 (&out)[4]) {
  auto lo2 = [](uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); };
  auto hi2 = [](uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); };
  out[0] = make_uint2(lo2(in[0].x, in[1].x), lo2(in[2].x, in[3].x));
  out[1] = make_uint2(hi2(in[0].x, in[1].x), hi2(in[2].x, in[3].x));
  out[2] = make_uint2(lo2(in[0].y, in[1].y), lo2(in[2].y, in[3].y));
  out[3] = make_uint2(hi2(in[0].y, in[1].y), hi2(in[2].y, in[3].y));
}

struct SsdArgs {
  const uint16_t* x;       // (B, L, H, P) bf16
  const uint16_t* dt;      // (B, L, H) bf16
  const float* A;          // (H)
  const uint16_t* Bm;      // (B, L, G, N) bf16
  const uint16_t* Cm;      // (B, L, G, N) bf16
  const float* D;          // (H) or null
  const float* dt_bias;    // (H) or null
  void* y;                 // (B, L, H, P)
  int64_t L;
  int H, G;
};

template <typename Out, bool SOFTPLUS>
__global__ __launch_bounds__(kThreads, 3) void ssd_fwd_kernel(SsdArgs a) {
  __shared__ Smem sm;
  const int tid = int(threadIdx.x);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int c16 = lane & 15, g = lane >> 4;
  const int h = int(blockIdx.x % unsigned(a.H));
  const int64_t b = int64_t(blockIdx.x / unsigned(a.H));
  const int grp = h / (a.H / a.G);
  const int64_t L = a.L;
  const int nc = int((L + kQ - 1) / kQ);

  const float Dh = a.D ? a.D[h] : 0.0f;
  const float biash = a.dt_bias ? a.dt_bias[h] : 0.0f;

  // staging: thread = 4 x 4 block (rows 4 rb .. +3, columns 4 cb .. +3) of each chunk tile
  const int rb = tid >> 4, cb = tid & 15;
  const int64_t xrow = int64_t(a.H) * kDim, brow = int64_t(a.G) * kDim;   // row strides
  const uint16_t* xg = a.x + (b * L * a.H + h) * kDim + 4 * cb;
  const uint16_t* bg = a.Bm + (b * L * a.G + grp) * kDim + 4 * cb;
  const uint16_t* cg = a.Cm + (b * L * a.G + grp) * kDim + 4 * cb;
  const uint16_t* dtg = a.dt + b * L * a.H + h;
  uint2 xr[4], br[4], cr[4];
  uint16_t dtr = 0;
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t s = int64_t(c) * kQ + 4 * rb + i;
      if (s < L) {
        xr[i] = *reinterpret_cast<const uint2*>(xg + s * xrow);
        br[i] = *reinterpret_cast<const uint2*>(bg + s * brow);
        cr[i] = *reinterpret_cast<const uint2*>(cg + s * brow);
      } else {
        xr[i] = br[i] = cr[i] = make_uint2(0u, 0u);
      }
    }
    if (w == 0) {
      const int64_t s = int64_t(c) * kQ + lane;
      dtr = s < L ? dtg[s * a.H] : uint16_t(0);
    }
  };

  // state H[n][p]: tile ni holds rows 16 ni + 4g + r, column 16 w + c16
  f32x4 hacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) hacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_chunk(0);
  for (int c = 0; c < nc; ++c) {
    __syncthreads();   // the previous chunk's tiles are no longer read
    {
      uint2 tr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * rb + i;
        sm.bs.u[r][swz(r, cb)] = br[i];
        sm.cs.u[r][swz(r, cb)] = cr[i];
      }
      transpose4(br, tr);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * cb + j;
        sm.bt.u[r][swz(r, rb)] = tr[j];
      }
      transpose4(xr, tr);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * cb + j;
        sm.xt.u[r][swz(r, rb)] = tr[j];
      }
      if (w == 0) {
        // step sizes and the running log2 decay of the chunk (zero past the end)
        const bool valid = int64_t(c) * kQ + lane < L;
        const float v = to_f32(dtr) + biash;
        float dt2;   // dt * log2(e)
        if constexpr (SOFTPLUS) dt2 = softplus_log2(v * kLog2e);
        else dt2 = v * kLog2e;
        if (!valid) dt2 = 0.0f;
        sm.lam[lane] = wave_inclusive_sum(dt2 * a.A[h]);
        sm.dts[lane] = dt2 * kLn2;
      }
    }
    __syncthreads();
    if (c + 1 < nc) load_chunk(c + 1);
    const float lam_end = sm.lam[kQ - 1];

    // p-role: off-diagonal outputs exp(l_t) C_t . H for p-tile w, every t-tile
    {
      u32x4 hh[2], hl[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float v[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = hacc[2 * j][r];
          v[4 + r] = hacc[2 * j + 1][r];
        }
        split8(v, hh[j], hl[j]);
      }
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x4 cop = ld_op(sm.cs, 16 * ti + c16, j, g);
          acc = mfma(cop, hh[j], acc);
          acc = mfma(cop, hl[j], acc);
        }
        const f32x4 lt = *reinterpret_cast<const f32x4*>(&sm.lam[16 * ti + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= hw_exp2(lt[r]);
        sm.yo[ti][w][lane] = acc;
      }
    }

    // t-role: M^T tiles of t-tile w (s-tiles 0..w), masked and split
    u32x4 mh[2], ml[2];
    {
      const int t = 16 * w + c16;
      const float lamt = sm.lam[t];
      const u32x4 ct0 = ld_op(sm.cs, t, 0, g), ct1 = ld_op(sm.cs, t, 1, g);
      float m[4][4];
#pragma unroll
      for (int si = 0; si < 4; ++si) {
        if (si > w) {
#pragma unroll
          for (int r = 0; r < 4; ++r) m[si][r] = 0.0f;
          continue;
        }
        f32x4 gacc = {0.f, 0.f, 0.f, 0.f};
        gacc = mfma(ld_op(sm.bs, 16 * si + c16, 0, g), ct0, gacc);
        gacc = mfma(ld_op(sm.bs, 16 * si + c16, 1, g), ct1, gacc);
        const f32x4 ls = *reinterpret_cast<const f32x4*>(&sm.lam[16 * si + 4 * g]);
        const f32x4 ds = *reinterpret_cast<const f32x4*>(&sm.dts[16 * si + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = 16 * si + 4 * g + r;
          float v = gacc[r] * (hw_exp2(lamt - ls[r]) * ds[r]);
          if (s == t) v += Dh;
          m[si][r] = s <= t ? v : 0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float v[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = m[2 * j][r];
          v[4 + r] = m[2 * j + 1][r];
        }
        split8(v, mh[j], ml[j]);
      }
    }
    __syncthreads();   // yo complete

    // t-role: Y = yo + M X for t-tile w, every p-tile; store
    {
      const int nkb = (w >> 1) + 1;
#pragma unroll
      for (int pi = 0; pi < 4; ++pi) {
        f32x4 acc = sm.yo[w][pi][lane];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (j >= nkb) continue;
          const u32x4 xop = ld_op(sm.xt, 16 * pi + c16, j, g);
          acc = mfma(mh[j], xop, acc);
          acc = mfma(ml[j], xop, acc);
        }
        Out* yp = static_cast<Out*>(a.y) +
                  ((b * L + int64_t(c) * kQ + 16 * w + 4 * g) * a.H + h) * kDim + 16 * pi + c16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (int64_t(c) * kQ + 16 * w + 4 * g + r < L) store_out(yp + int64_t(r) * xrow, acc[r]);
        }
      }
    }

    // p-role: H <- exp(l_end) H + B^T X', X' = exp(l_end - l_s) dt_s x_s (p-tile w)
    {
      u32x4 xh[2], xl[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float v[8];
        bf16x8_to_f32(ld_op(sm.xt, 16 * w + c16, j, g), v);
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(&sm.lam[32 * j + 4 * g]);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(&sm.lam[32 * j + 16 + 4 * g]);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&sm.dts[32 * j + 4 * g]);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&sm.dts[32 * j + 16 + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] *= hw_exp2(lam_end - l0[r]) * d0[r];
          v[4 + r] *= hw_exp2(lam_end - l1[r]) * d1[r];
        }
        split8(v, xh[j], xl[j]);
      }
      const float decay = hw_exp2(lam_end);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        f32x4 acc = hacc[ni] * decay;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x4 bop = ld_op(sm.bt, 16 * ni + c16, j, g);
          acc = mfma(bop, xh[j], acc);
          acc = mfma(bop, xl[j], acc);
        }
        hacc[ni] = acc;
      }
    }
  }
}

}  // namespace

int launch_ssd_fwd(const ss_ssd_desc_t& d, const void* x, const void* dt, const float* A,
                   const void* Bm, const void* Cm, const float* D, const float* dt_bias, void* y,
                   void* stream) {
  SsdArgs a{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(dt), A,
            static_cast<const uint16_t*>(Bm), static_cast<const uint16_t*>(Cm), D, dt_bias, y,
            d.seqlen, int(d.nheads), int(d.ngroups)};
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(unsigned(d.batch * d.nheads)), block(kThreads);
  const bool f32 = d.out_dtype == SS_F32, sp = d.dt_softplus != 0;
  if (f32 && sp) hipLaunchKernelGGL((ssd_fwd_kernel<float, true>), grid, block, 0, st, a);
  else if (f32) hipLaunchKernelGGL((ssd_fwd_kernel<float, false>), grid, block, 0, st, a);
  else if (sp) hipLaunchKernelGGL((ssd_fwd_kernel<uint16_t, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((ssd_fwd_kernel<uint16_t, false>), grid, block, 0, st, a);
  return int(hipGetLastError());
}

}  // namespace ss
