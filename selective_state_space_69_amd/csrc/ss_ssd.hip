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
//
// The state may start from a given H (else zero) and its value after the last
// step may be stored; both in the accumulator's own layout, straight from and
// to global memory, once per workgroup.
//
// Per chunk: the next chunk's x, B, C rows are fetched into registers (buffer
// loads; rows past the end read as zero) while this one is computed, then
// written to LDS as B and C rows and as B^T and x^T (4 x 4 transposes in
// registers).  Three barriers: tiles written, C H exchanged, tiles free again.
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

// LDS operand tiles: 64 rows x 8 units of 16 bytes.  Unit q = 4j + g of a row
// holds the 8 k slots lane group g supplies for k block j (columns 32j + 4g .. +3
// and 32j + 16 + 4g .. +3), so an operand is one 16-byte read; the unit sits at
// q ^ ((row >> 1) & 7): the 16 rows one read touches (16 lanes per pass) then
// cover all 64 banks exactly once (row parity picks the bank half, the XOR the
// unit inside it).
constexpr int kTileBytes = kDim * 128;
__device__ __forceinline__ int op_off(int row, int q) {
  return row * 128 + ((q ^ ((row >> 1) & 7)) << 4);
}
// columns 4 cb .. 4 cb + 3 of a row (8 bytes): unit 4 (cb >> 3) + (cb & 3), half (cb >> 2) & 1
__device__ __forceinline__ int col_off(int row, int cb) {
  return op_off(row, 4 * (cb >> 3) + (cb & 3)) + (((cb >> 2) & 1) << 3);
}

// LDS map (bytes)
constexpr int kOffBs = 0;                        // B rows   [s][n]
constexpr int kOffCs = kOffBs + kTileBytes;      // C rows   [t][n]
constexpr int kOffBt = kOffCs + kTileBytes;      // B^T      [n][s]
constexpr int kOffXt = kOffBt + kTileBytes;      // x^T      [p][s]
constexpr int kOffYo = kOffXt + kTileBytes;      // exp(l_t) C H as [t-tile][p-tile][lane] x 16 B
constexpr int kOffLam = kOffYo + 16 * kWave * 16;   // l_t, log2 units, inclusive from the chunk start
constexpr int kOffElam = kOffLam + kQ * 4;       // exp2(l_t)
constexpr int kOffWts = kOffElam + kQ * 4;       // exp2(l_end - l_s) dt_s
constexpr int kOffDts = kOffWts + kQ * 4;        // dt_s
constexpr int kSmemBytes = kOffDts + kQ * 4;

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

__device__ __forceinline__ uint2 buf_load8(Rsrc r, uint32_t voff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
  return make_uint2(v[0], v[1]);
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
  const float* h0;         // (B, H, N, P) state before the first step, or null (zero)
  float* h_last;           // (B, H, N, P) state after the last step, or null
  int64_t L;
  int H, G;
};

template <typename Out>
__device__ __forceinline__ void store_y4(Rsrc r, uint32_t voff, f32x4 v);
template <>
__device__ __forceinline__ void store_y4<float>(Rsrc r, uint32_t voff, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, 0, 0);
}
template <>
__device__ __forceinline__ void store_y4<uint16_t>(Rsrc r, uint32_t voff, f32x4 v) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  u32x2 p;
  p.x = pack_bf16(v[0], v[1]);
  p.y = pack_bf16(v[2], v[3]);
  __builtin_amdgcn_raw_buffer_store_b64(p, r, voff, 0, 0);
}

// STATE: a start state is read (zero where h0 is null) and the final state is
// stored where h_last is not null.
template <typename Out, bool SOFTPLUS, bool STATE>
__global__ __launch_bounds__(kThreads, 3) void ssd_fwd_kernel(SsdArgs a) {
  __shared__ __align__(16) char sm[kSmemBytes];
  const int tid = int(threadIdx.x);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int c16 = lane & 15, g = lane >> 4;
  // the heads of one batch row read the same B and C rows: with each XCD on a
  // contiguous range of (b, h) those rows are fetched once per batch row
  const int64_t bid = xcd_contiguous(blockIdx.x, gridDim.x);
  const int h = int(bid % a.H);
  const int64_t b = bid / a.H;
  const int grp = h / (a.H / a.G);
  const int64_t L = a.L;
  const int nc = int((L + kQ - 1) / kQ);
  const float Dh = a.D ? a.D[h] : 0.0f;
  const float biash = a.dt_bias ? a.dt_bias[h] : 0.0f;
  const float Ah = a.A[h];

  // operand reads: row 16 tile + c16, unit 4j + g -> byte offset tile * 2048 + opj[j]
  // (the swizzle depends on the row only through c16)
  const int opj0 = op_off(c16, g), opj1 = op_off(c16, 4 + g);
  auto ld_op = [&](int base, int tile, int j) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(sm + base + tile * (16 * 128) + (j ? opj1 : opj0));
  };
  auto ldf4 = [&](int off) -> f32x4 { return *reinterpret_cast<const f32x4*>(sm + off); };

  // staging: thread = 4 x 4 block (rows 4 rb .. +3, columns 4 cb .. +3) of each chunk tile
  const int rb = tid >> 4, cb = tid & 15;
  const uint32_t xrow_b = uint32_t(a.H) * kDim * 2, brow_b = uint32_t(a.G) * kDim * 2;
  const uint16_t* xbase = a.x + (b * L * a.H + h) * kDim;
  const uint16_t* bbase = a.Bm + (b * L * a.G + grp) * kDim;
  const uint16_t* cbase = a.Cm + (b * L * a.G + grp) * kDim;
  const uint16_t* dtbase = a.dt + b * L * a.H + h;
  Out* ybase = static_cast<Out*>(a.y) + (b * L * a.H + h) * kDim;
  // register set the next chunk is fetched into while this one is computed
  struct Stage {
    uint2 xr[4], br[4], cr[4];
    uint32_t dtr;
  };
  Stage st0;
  // The next chunk is fetched in three parts (x and the step sizes, B, C) at
  // three points of the current one, B and C while matrix products are in
  // flight: the workgroups' waves leave each barrier together, and one burst
  // of all their loads would hold every wave at the load issue until it
  // drained.
  // part 0: x and dt; part 1: B rows; part 2: C rows
  auto load_part = [&](int part, int c, Stage& sg) __attribute__((always_inline)) {
    const int64_t t0 = int64_t(c) * kQ;
    const int64_t rows = L - t0;                       // valid rows of this chunk (> 0)
    if (part == 0) {
      const Rsrc rx = make_rsrc(xbase + t0 * a.H * kDim);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = 4 * rb + i < rows;
        sg.xr[i] = buf_load8(rx, ok ? uint32_t(4 * rb + i) * xrow_b + 8 * cb : kOutOfRange);
      }
      // every wave loads the step sizes (only wave 0 uses them) so that all
      // waves have the same memory operations in flight
      const Rsrc rd = make_rsrc(dtbase + t0 * a.H);
      sg.dtr = __builtin_amdgcn_raw_buffer_load_b16(
          rd, lane < rows ? uint32_t(lane) * uint32_t(a.H) * 2 : kOutOfRange, 0, 0);
    } else {
      const Rsrc r = make_rsrc((part == 1 ? bbase : cbase) + t0 * a.G * kDim);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = 4 * rb + i < rows;
        const uint2 v = buf_load8(r, ok ? uint32_t(4 * rb + i) * brow_b + 8 * cb : kOutOfRange);
        if (part == 1) sg.br[i] = v;
        else sg.cr[i] = v;
      }
    }
  };
  auto load_chunk = [&](int c, Stage& sg) __attribute__((always_inline)) {
    load_part(0, c, sg);
    load_part(1, c, sg);
    load_part(2, c, sg);
  };
  // output rows 16 w + 4 g + r, columns 16 pi + c16
  const uint32_t yrow_b = uint32_t(a.H) * kDim * uint32_t(sizeof(Out));

  // state H[n][p]: tile ni holds rows 16 ni + 4g + r, column 16 w + c16
  f32x4 hacc[4];
  if constexpr (STATE) {
    // element (n, p) of this head's state: (b H + h) N P + n P + p; a null h0
    // gets a buffer of no records, whose loads return zero
    const Rsrc rh = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.h0) + (b * a.H + h) * int64_t(kDim * kDim), short(0),
        a.h0 ? 0x7fffffff : 0, 0x00020000);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        hacc[i][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rh, uint32_t((16 * i + 4 * g + r) * kDim + 16 * w + c16) * 4u, 0, 0));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) hacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One chunk, from register set sg.  Without a start state the first chunk
  // is peeled off the loop below: every path into the loop head then has the
  // previous chunk's output stores issued after its prefetch loads, so the
  // wait at the head covers the loads only.  With a start state the peeled
  // copy (whose state is no longer known to be zero) would not fit the
  // register budget, and the loop runs from the first chunk.
  auto chunk = [&](int c, Stage& sg) __attribute__((always_inline)) {
    const int64_t t0 = int64_t(c) * kQ;
    const int64_t rows = L - t0;
    __syncthreads();   // the previous chunk's tiles are no longer read
    {
      uint2 tr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * rb + i;
        *reinterpret_cast<uint2*>(sm + kOffBs + col_off(r, cb)) = sg.br[i];
        *reinterpret_cast<uint2*>(sm + kOffCs + col_off(r, cb)) = sg.cr[i];
      }
      transpose4(sg.br, tr);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint2*>(sm + kOffBt + col_off(4 * cb + j, rb)) = tr[j];
      transpose4(sg.xr, tr);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint2*>(sm + kOffXt + col_off(4 * cb + j, rb)) = tr[j];
      if (w == 0) {
        // step sizes, the running log2 decay of the chunk (zero past the end) and
        // the per-step factors every wave needs
        const float v = __uint_as_float(sg.dtr << 16) + biash;
        float dt2;   // dt * log2(e)
        if constexpr (SOFTPLUS) dt2 = softplus_log2(v * kLog2e);
        else dt2 = v * kLog2e;
        if (lane >= rows) dt2 = 0.0f;
        const float lam = wave_inclusive_sum(dt2 * Ah);
        const float lend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam), kQ - 1));
        const float dtn = dt2 * kLn2;
        reinterpret_cast<float*>(sm + kOffLam)[lane] = lam;
        reinterpret_cast<float*>(sm + kOffElam)[lane] = hw_exp2(lam);
        reinterpret_cast<float*>(sm + kOffWts)[lane] = hw_exp2(lend - lam) * dtn;
        reinterpret_cast<float*>(sm + kOffDts)[lane] = dtn;
      }
    }
    __syncthreads();
    if (c + 1 < nc) load_part(0, c + 1, sg);
    const float lam_end = reinterpret_cast<const float*>(sm + kOffLam)[kQ - 1];

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
      // every operand read is issued before the first product, and the four
      // row tiles' accumulation chains are interleaved
      u32x4 cop[4][2];
      f32x4 el[4], acc[4];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        cop[ti][0] = ld_op(kOffCs, ti, 0);
        cop[ti][1] = ld_op(kOffCs, ti, 1);
        el[ti] = ldf4(kOffElam + (16 * ti + 4 * g) * 4);
        acc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) acc[ti] = mfma(cop[ti][j], hh[j], acc[ti]);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) acc[ti] = mfma(cop[ti][j], hl[j], acc[ti]);
      }
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
        *reinterpret_cast<f32x4*>(sm + kOffYo + ((ti * 4 + w) * kWave + lane) * 16) =
            acc[ti] * el[ti];
    }

    // t-role: M^T tiles of t-tile w (s-tiles 0..w), masked and split
    u32x4 mh[2], ml[2];
    {
      const int t = 16 * w + c16;
      const float lamt = reinterpret_cast<const float*>(sm + kOffLam)[t];
      const u32x4 ct0 = ld_op(kOffCs, w, 0), ct1 = ld_op(kOffCs, w, 1);
      // operands of all four column tiles first (in-bounds for every wave; the
      // tiles past the diagonal are not used)
      u32x4 bop[4][2];
      f32x4 lsv[4], dsv[4], gacc[4];
#pragma unroll
      for (int si = 0; si < 4; ++si) {
        bop[si][0] = ld_op(kOffBs, si, 0);
        bop[si][1] = ld_op(kOffBs, si, 1);
        gacc[si] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int si = 0; si < 4; ++si)
        if (si <= w) gacc[si] = mfma(bop[si][0], ct0, gacc[si]);
#pragma unroll
      for (int si = 0; si < 4; ++si)
        if (si <= w) gacc[si] = mfma(bop[si][1], ct1, gacc[si]);
      if (c + 1 < nc) load_part(1, c + 1, sg);   // while the products run
      // the decay factors are read while the products run
#pragma unroll
      for (int si = 0; si < 4; ++si) {
        lsv[si] = ldf4(kOffLam + (16 * si + 4 * g) * 4);
        dsv[si] = ldf4(kOffDts + (16 * si + 4 * g) * 4);
      }
      float m[4][4];
#pragma unroll
      for (int si = 0; si < 4; ++si) {
        if (si > w) {
#pragma unroll
          for (int r = 0; r < 4; ++r) m[si][r] = 0.0f;
          continue;
        }
        const f32x4 ls = lsv[si], ds = dsv[si];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = 16 * si + 4 * g + r;
          float v = gacc[si][r] * (hw_exp2(lamt - ls[r]) * ds[r]);
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

    // t-role: Y = yo + M X for t-tile w, every p-tile.  The wave's 16 x 64
    // outputs go through its own 4 KB of the exchange area (its yo tiles, read
    // first) so that every lane stores 16 contiguous bytes and each store
    // instruction writes 4 whole output rows.
    {
      const int nkb = (w >> 1) + 1;
      char* ybuf = sm + kOffYo + w * 4 * kWave * 16;
      f32x4 acc[4];
      u32x4 xop[4][2];
#pragma unroll
      for (int pi = 0; pi < 4; ++pi) {
        acc[pi] = *reinterpret_cast<const f32x4*>(ybuf + (pi * kWave + lane) * 16);
        xop[pi][0] = ld_op(kOffXt, pi, 0);
        xop[pi][1] = ld_op(kOffXt, pi, 1);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (j >= nkb) continue;
#pragma unroll
        for (int pi = 0; pi < 4; ++pi) acc[pi] = mfma(mh[j], xop[pi][j], acc[pi]);
#pragma unroll
        for (int pi = 0; pi < 4; ++pi) acc[pi] = mfma(ml[j], xop[pi][j], acc[pi]);
      }
      if (c + 1 < nc) load_part(2, c + 1, sg);   // while the products run
      __builtin_amdgcn_wave_barrier();
      // row t (0..15) of 64 floats = 16 units of 16 bytes; unit u at u ^ (4 (t >> 2))
#pragma unroll
      for (int pi = 0; pi < 4; ++pi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 4 * g + r, u = 4 * pi + (c16 >> 2);
          *reinterpret_cast<float*>(ybuf + t * 256 + ((u ^ (4 * g)) << 4) + (c16 & 3) * 4) =
              acc[pi][r];
        }
      __builtin_amdgcn_wave_barrier();
      const Rsrc ry = make_rsrc(ybase + t0 * a.H * kDim);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int t = 4 * k + (lane >> 4), u = lane & 15;
        const f32x4 v = *reinterpret_cast<const f32x4*>(ybuf + t * 256 + ((u ^ (4 * k)) << 4));
        const int row = 16 * w + t;
        const uint32_t off = row < rows ? uint32_t(row) * yrow_b + uint32_t(4 * u * sizeof(Out))
                                        : kOutOfRange;
        store_y4<Out>(ry, off, v);
      }
    }

    // p-role: H <- exp(l_end) H + B^T X', X' = exp(l_end - l_s) dt_s x_s (p-tile w)
    {
      u32x4 xh[2], xl[2], bop[4][2], xvv[2];
      f32x4 wv[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        xvv[j] = ld_op(kOffXt, w, j);
        wv[j][0] = ldf4(kOffWts + (32 * j + 4 * g) * 4);
        wv[j][1] = ldf4(kOffWts + (32 * j + 16 + 4 * g) * 4);
      }
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        bop[ni][0] = ld_op(kOffBt, ni, 0);
        bop[ni][1] = ld_op(kOffBt, ni, 1);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 xv = xvv[j];
        const f32x4 w0 = wv[j][0], w1 = wv[j][1];
        float v[8];
        v[0] = __uint_as_float(xv.x << 16) * w0[0];
        v[1] = __uint_as_float(xv.x & 0xffff0000u) * w0[1];
        v[2] = __uint_as_float(xv.y << 16) * w0[2];
        v[3] = __uint_as_float(xv.y & 0xffff0000u) * w0[3];
        v[4] = __uint_as_float(xv.z << 16) * w1[0];
        v[5] = __uint_as_float(xv.z & 0xffff0000u) * w1[1];
        v[6] = __uint_as_float(xv.w << 16) * w1[2];
        v[7] = __uint_as_float(xv.w & 0xffff0000u) * w1[3];
        split8(v, xh[j], xl[j]);
      }
      const float decay = hw_exp2(lam_end);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) hacc[ni] *= decay;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) hacc[ni] = mfma(bop[ni][j], xh[j], hacc[ni]);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) hacc[ni] = mfma(bop[ni][j], xl[j], hacc[ni]);
      }
    }
  };
  load_chunk(0, st0);
  if constexpr (STATE) {
    for (int c = 0; c < nc; ++c) chunk(c, st0);
  } else {
    chunk(0, st0);
    for (int c = 1; c < nc; ++c) chunk(c, st0);
  }
  if (STATE && a.h_last) {
    // lane index and its parts formed afresh: nothing of the prologue's
    // addressing stays live through the chunk loop
    const int ln = int(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
    const uint32_t col = uint32_t(16 * w + (ln & 15)), row = uint32_t(4 * (ln >> 4));
    const Rsrc rh = make_rsrc(a.h_last + (b * a.H + h) * int64_t(kDim * kDim));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(hacc[i][r]), rh,
                                              ((row + 16 * i + r) * kDim + col) * 4u, 0, 0);
  }
}

// One step of the recurrence on the state of one (batch row, head):
//     H <- exp(dt A) H + dt B x^T,   y = H^T C + D x
// 256 threads; thread (wave w, lane l) owns columns p = 4 (l & 15) .. +3 of
// rows n = 4 w + (l >> 4) + 16 k, k = 0..3, so every state row is read and
// written as 16-byte pieces, a wave's four rows of one k being 1 KB in a row.
// C^T H is summed over a wave's rows with lane exchanges and over the four
// waves in LDS, in a fixed order.  The step sizes, decay and B weight are
// formed as in the chunked kernel above, so a step continues its state.
struct SsdStepArgs {
  float* h;                // (B, H, N, P) fp32, in place
  const uint16_t* x;       // (B, H, P) bf16
  const uint16_t* dt;      // (B, H) bf16
  const float* A;          // (H)
  const uint16_t* Bm;      // (B, G, N) bf16
  const uint16_t* Cm;      // (B, G, N) bf16
  const float* D;          // (H) or null
  const float* dt_bias;    // (H) or null
  void* y;                 // (B, H, P)
  int H, G;
};

template <typename Out>
__device__ __forceinline__ void store_y4_ptr(Out* p, float4 v);
template <>
__device__ __forceinline__ void store_y4_ptr<float>(float* p, float4 v) {
  *reinterpret_cast<float4*>(p) = v;
}
template <>
__device__ __forceinline__ void store_y4_ptr<uint16_t>(uint16_t* p, float4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16(v.x, v.y), pack_bf16(v.z, v.w));
}

template <typename Out, bool SOFTPLUS>
__global__ __launch_bounds__(kThreads) void ssd_step_kernel(SsdStepArgs a) {
  __shared__ float4 part[kNW][16];
  const int tid = int(threadIdx.x);
  const int w = tid / kWave, lane = tid % kWave;
  const int q = lane & 15, r = 4 * w + (lane >> 4);
  const int h = int(blockIdx.x % unsigned(a.H));
  const int64_t b = int64_t(blockIdx.x / unsigned(a.H));
  const int grp = h / (a.H / a.G);
  const int64_t bh = b * a.H + h;

  const float v = to_f32<uint16_t>(a.dt[bh]) + (a.dt_bias ? a.dt_bias[h] : 0.0f);
  float dt2;   // dt * log2(e)
  if constexpr (SOFTPLUS) dt2 = softplus_log2(v * kLog2e);
  else dt2 = v * kLog2e;
  const float decay = hw_exp2(dt2 * a.A[h]);
  const float dtn = dt2 * kLn2;
  const float4 xv = unpack4(*reinterpret_cast<const uint2*>(a.x + bh * kDim + 4 * q));
  const uint16_t* Bg = a.Bm + (b * a.G + grp) * kDim;
  const uint16_t* Cg = a.Cm + (b * a.G + grp) * kDim;
  float* hp = a.h + bh * (kDim * kDim) + 4 * q;

  float4 hv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) hv[k] = *reinterpret_cast<const float4*>(hp + (r + 16 * k) * kDim);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int n = r + 16 * k;
    const float bw = dtn * to_f32<uint16_t>(Bg[n]), cn = to_f32<uint16_t>(Cg[n]);
    float4 s = hv[k];
    s.x = fmaf(decay, s.x, bw * xv.x);
    s.y = fmaf(decay, s.y, bw * xv.y);
    s.z = fmaf(decay, s.z, bw * xv.z);
    s.w = fmaf(decay, s.w, bw * xv.w);
    *reinterpret_cast<float4*>(hp + n * kDim) = s;
    acc.x = fmaf(cn, s.x, acc.x);
    acc.y = fmaf(cn, s.y, acc.y);
    acc.z = fmaf(cn, s.z, acc.z);
    acc.w = fmaf(cn, s.w, acc.w);
  }
#pragma unroll
  for (int m = 16; m < kWave; m *= 2) {
    acc.x += __shfl_xor(acc.x, m);
    acc.y += __shfl_xor(acc.y, m);
    acc.z += __shfl_xor(acc.z, m);
    acc.w += __shfl_xor(acc.w, m);
  }
  if (lane < 16) part[w][q] = acc;
  __syncthreads();
  if (tid < 16) {
    float4 s = part[0][tid];
#pragma unroll
    for (int i = 1; i < kNW; ++i) {
      const float4 o = part[i][tid];
      s.x += o.x; s.y += o.y; s.z += o.z; s.w += o.w;
    }
    if (a.D) {
      const float Dh = a.D[h];
      const float4 xq = unpack4(*reinterpret_cast<const uint2*>(a.x + bh * kDim + 4 * tid));
      s.x = fmaf(Dh, xq.x, s.x);
      s.y = fmaf(Dh, xq.y, s.y);
      s.z = fmaf(Dh, xq.z, s.z);
      s.w = fmaf(Dh, xq.w, s.w);
    }
    store_y4_ptr<Out>(static_cast<Out*>(a.y) + bh * kDim + 4 * tid, s);
  }
}

}  // namespace

int launch_ssd_step(const ss_ssd_desc_t& d, float* h, const void* x, const void* dt,
                    const float* A, const void* Bm, const void* Cm, const float* D,
                    const float* dt_bias, void* y, void* stream) {
  SsdStepArgs a{h, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(dt), A,
                static_cast<const uint16_t*>(Bm), static_cast<const uint16_t*>(Cm), D, dt_bias, y,
                int(d.nheads), int(d.ngroups)};
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(unsigned(d.batch * d.nheads)), block(kThreads);
  const bool f32 = d.out_dtype == SS_F32, sp = d.dt_softplus != 0;
  if (f32 && sp) hipLaunchKernelGGL((ssd_step_kernel<float, true>), grid, block, 0, st, a);
  else if (f32) hipLaunchKernelGGL((ssd_step_kernel<float, false>), grid, block, 0, st, a);
  else if (sp) hipLaunchKernelGGL((ssd_step_kernel<uint16_t, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((ssd_step_kernel<uint16_t, false>), grid, block, 0, st, a);
  return int(hipGetLastError());
}

int launch_ssd_fwd(const ss_ssd_desc_t& d, const void* x, const void* dt, const float* A,
                   const void* Bm, const void* Cm, const float* D, const float* dt_bias,
                   const float* h0, void* y, float* h_last, void* stream) {
  SsdArgs a{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(dt), A,
            static_cast<const uint16_t*>(Bm), static_cast<const uint16_t*>(Cm), D, dt_bias, y,
            h0, h_last, d.seqlen, int(d.nheads), int(d.ngroups)};
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(unsigned(d.batch * d.nheads)), block(kThreads);
  const bool f32 = d.out_dtype == SS_F32, sp = d.dt_softplus != 0;
  if (h0 || h_last) {
    if (f32 && sp) hipLaunchKernelGGL((ssd_fwd_kernel<float, true, true>), grid, block, 0, st, a);
    else if (f32) hipLaunchKernelGGL((ssd_fwd_kernel<float, false, true>), grid, block, 0, st, a);
    else if (sp) hipLaunchKernelGGL((ssd_fwd_kernel<uint16_t, true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((ssd_fwd_kernel<uint16_t, false, true>), grid, block, 0, st, a);
  } else {
    if (f32 && sp) hipLaunchKernelGGL((ssd_fwd_kernel<float, true, false>), grid, block, 0, st, a);
    else if (f32) hipLaunchKernelGGL((ssd_fwd_kernel<float, false, false>), grid, block, 0, st, a);
    else if (sp) hipLaunchKernelGGL((ssd_fwd_kernel<uint16_t, true, false>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((ssd_fwd_kernel<uint16_t, false, false>), grid, block, 0, st, a);
  }
  return int(hipGetLastError());
}

}  // namespace ss
