// Chunk carries of the two-level scan, as an associative scan across the lanes
// of a wave.
//
// A chunk c of a (b, n, d) sequence acts on the state as the affine map
// h -> a_c h + s_c, with a_c = exp2(A[d,n] * sum over the chunk of dt log2 e)
// and s_c the chunk's end state from a zero start (the summary pass).  Maps
// compose associatively, (a1, s1) then (a2, s2) = (a1 a2, a2 s1 + s2) ("A Visual
// Guide to Mamba" summary, The Scan Operation: segments combined associatively;
// "A Survey of Mamba" summary, hardware-aware computation: parallel scan), so
// the start states of all chunks are an inclusive scan of the maps applied to
// the initial state.  The decay is carried as e = a - 1 (precise_expm1): a
// chunk that barely decays its state keeps it for many chunks, and a rounded
// near 1 would compound its rounding over all of them.  In that form the
// composition is (e1, s1) then (e2, s2) = (e1 + e2 + e1 e2, s1 + e2 s1 + s2).
//
// Two kernels, chosen by the number of chunks:
//  - few chunks (< 256): one lane per (b, n, d) walks the chunks in order.
//    The chain is short and every load is coalesced; nothing beats it.
//  - many chunks (the million-step case): a workgroup (4 waves) takes one
//    (b, n) and 16 channels and walks the chunks in tiles of 64.  The tile's
//    maps are read into LDS with the channels on the lanes, then each wave
//    scans 4 channels, one at a time with the chunk index on the 64 lanes, in
//    6 steps: DPP row_shr 1, 2, 4, 8 inside each row of 16 lanes, row_bcast:15
//    into the odd rows and row_bcast:31 into the upper half.  The tile's last
//    lane carries into the next tile; the results go back through LDS.  This
//    replaces a 2048-long dependent chain per lane by 32 tiles of 6 steps and
//    spreads a narrow problem over 4x more workgroups.
// Both run the adjoint carries of the backward too, in reverse chunk order (the
// adjoint recurrence runs backwards in time).
#include "ss_device.hpp"

namespace ss {
namespace {

constexpr int kTile = 64;            // chunks per tile (one per lane in the scan)
constexpr int kCh = 16;              // channels per workgroup (scan kernel)
constexpr int kWaves = 4;
constexpr int kChPerWave = kCh / kWaves;
constexpr int kRows = kWaves * kWave / kCh;   // chunk rows a workgroup moves per load pass
constexpr int kPad = kCh + 1;        // LDS row stride: the scan's column reads hit distinct banks
constexpr int kScanMinChunks = 256;  // below this the in-order walk is faster

constexpr int kRowShr = 0x110;       // DPP row_shr:n = kRowShr + n
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL,
                                                    ROW_MASK, 0xf, false));
}

// (e, s) of a lane becomes the composition of the maps of lanes 0..lane (lane 0
// first).  Lanes without a predecessor at a step receive the identity (0, 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void scan_step(float& e, float& s) {
  const float ep = dpp_or<CTRL, ROW_MASK>(0.0f, e);
  const float sp = dpp_or<CTRL, ROW_MASK>(0.0f, s);
  s = __builtin_fmaf(e, sp, s) + sp;      // earlier (ep, sp) then (e, s)
  e = __builtin_fmaf(e, ep, e) + ep;
}

__device__ __forceinline__ void wave_scan(float& e, float& s) {
  scan_step<kRowShr + 1, 0xf>(e, s);
  scan_step<kRowShr + 2, 0xf>(e, s);
  scan_step<kRowShr + 4, 0xf>(e, s);
  scan_step<kRowShr + 8, 0xf>(e, s);
  scan_step<kRowBcast15, 0xa>(e, s);
  scan_step<kRowBcast31, 0xc>(e, s);
}

// Forward (REVERSE = false): states[b][c] holds chunk c's zero-start end state
// for c <= nc - 2; afterwards slot c (1 <= c <= nc - 1) holds the true start
// state of chunk c (slot 0 is left alone: chunk 0 starts from h0).
// Reverse: states[b][c] holds chunk c's local adjoint for 1 <= c <= nc - 1;
// afterwards slot c holds the adjoint entering chunk c from its end (slot
// nc - 1 gets 0, as nothing follows the last chunk).
// dsum[b][c][d] = sum over chunk c of dt log2 e (c <= nc - 2).
template <bool REVERSE>
__global__ __launch_bounds__(kWave * kWaves) void chunk_carry_kernel(float* __restrict__ states,
                                                                   const float* __restrict__ dsum,
                                                                   const float* __restrict__ A,
                                                                   const float* __restrict__ h0,
                                                                   int64_t D, int N, int nc,
                                                                   int ndblk) {
  __shared__ float ta[kTile][kPad], ts[kTile][kPad];   // decays e = a - 1, states
  __shared__ float lastv[2][kCh];   // a tile's last result, stored after the next tile's
                                    // loads (double-buffered by tile parity)
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const int lane = int(threadIdx.x) % kWave;
  const int tch = int(threadIdx.x) % kCh, trow = int(threadIdx.x) / kCh;   // load/store layout
  int64_t bid = blockIdx.x;
  const int dblk = int(bid % ndblk);
  bid /= ndblk;
  const int n = int(bid % N);
  const int64_t b = bid / N;
  const int64_t d = int64_t(dblk) * kCh + tch;        // channel of this thread in load/store
  const bool active = d < D;
  const int64_t dc = active ? d : D - 1;
  const float An = A[dc * N + n];
  const int64_t sstride = int64_t(N) * D;              // between chunk slots
  float* st = states + (b * nc) * sstride + int64_t(n) * D + dc;
  const float* ds = dsum + (b * nc) * D + dc;
  const int npairs = nc - 1;                           // maps that produce a stored state

  // running state entering the current tile, per channel of this wave's scans
  float carry[kChPerWave];
#pragma unroll
  for (int i = 0; i < kChPerWave; ++i) {
    const int64_t dd = int64_t(dblk) * kCh + wave * kChPerWave + i;
    const int64_t ddc = dd < D ? dd : D - 1;
    carry[i] = (!REVERSE && h0) ? h0[(b * D + ddc) * N + n] : 0.0f;
  }
  // slot written with the state after pair j; it is also the input slot of pair j + 1,
  // so the last result of a tile waits until the next tile has read its inputs
  auto out_slot = [&](int j) { return REVERSE ? nc - 2 - j : j + 1; };

  for (int j0 = 0; j0 < npairs; j0 += kTile) {
    // 1. maps of pairs j0 .. j0 + 63 (pair j = chunk j forward, chunk nc-1-j reverse)
#pragma unroll
    for (int i = 0; i < kTile / kRows; ++i) {
      const int jl = i * kRows + trow, j = j0 + jl;
      float e = 0.0f, s = 0.0f;
      if (j < npairs) {
        const int c = REVERSE ? nc - 1 - j : j;
        s = st[int64_t(c) * sstride];
        // the last chunk's step sum is never formed: its map multiplies a zero
        // adjoint, so any finite decay will do
        e = (REVERSE && j == 0) ? 0.0f : precise_expm1(An * ds[int64_t(c) * D]);
      }
      ta[jl][tch] = e;
      ts[jl][tch] = s;
    }
    __syncthreads();
    // 2. scan each channel's 64 maps with the chunk on the lanes
#pragma unroll
    for (int i = 0; i < kChPerWave; ++i) {
      const int ch = wave * kChPerWave + i;
      float e = ta[lane][ch], s = ts[lane][ch];
      wave_scan(e, s);
      const float h = carry[i] + __builtin_fmaf(e, carry[i], s);   // state after pair j0 + lane
      ts[lane][ch] = h;
      carry[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h), kTile - 1));
    }
    __syncthreads();
    // 3. store: the state after pair j is the start of chunk j + 1 (forward) or
    //    the adjoint entering chunk nc - 2 - j from its end (reverse)
    const int par = (j0 / kTile) & 1;
    if (j0 > 0 && trow == 0 && active) st[int64_t(out_slot(j0 - 1)) * sstride] = lastv[par ^ 1][tch];
#pragma unroll
    for (int i = 0; i < kTile / kRows; ++i) {
      const int jl = i * kRows + trow, j = j0 + jl;
      if (j >= npairs) continue;
      if (jl == kTile - 1 && j + 1 < npairs) lastv[par][tch] = ts[jl][tch];   // deferred
      else if (active) st[int64_t(out_slot(j)) * sstride] = ts[jl][tch];
    }
    __syncthreads();
  }
  // nothing enters the last chunk from its end (its slot was read above)
  if (REVERSE && active && trow == 0) st[int64_t(nc - 1) * sstride] = 0.0f;
}

// The in-order walk: one lane per (b, n, d), same slots and semantics.  The
// chunks are taken in groups of kWalkG; a group's inputs are all fetched before
// its chain runs, so a lane waits on memory once per group, not once per chunk.
constexpr int kWalkG = 16;

// One lane's walk over (b, n, d): REVERSE = false turns the zero-start end
// states in `states` into start states, REVERSE = true the local adjoints into
// the adjoints entering each chunk from its end.
template <bool REVERSE>
__device__ __forceinline__ void chunk_walk(float* __restrict__ states, const float* __restrict__ dsum,
                                           const float* __restrict__ A,
                                           const float* __restrict__ h0, int64_t gid, int64_t D,
                                           int N, int nc) {
  const int64_t d = gid % D;
  const int n = int((gid / D) % N);
  const int64_t b = gid / (D * N);
  const float An = A[d * N + n];
  const int64_t sstride = int64_t(N) * D;
  float* st = states + (b * nc) * sstride + int64_t(n) * D + d;
  const float* ds = dsum + (b * nc) * D + d;
  float sv[kWalkG], dv[kWalkG];
  if (!REVERSE) {
    // slot c <- start of chunk c;  h <- a_c h + s_c, c = 0 .. nc - 2
    float h = h0 ? h0[(b * D + d) * N + n] : 0.0f;
    for (int c0 = 0; c0 < nc - 1; c0 += kWalkG) {
#pragma unroll
      for (int g = 0; g < kWalkG; ++g) {
        const int c = c0 + g < nc - 1 ? c0 + g : nc - 2;
        sv[g] = st[int64_t(c) * sstride];
        dv[g] = ds[int64_t(c) * D];
      }
#pragma unroll
      for (int g = 0; g < kWalkG; ++g) {
        const int c = c0 + g;
        if (c >= nc - 1) break;
        if (c >= 1) st[int64_t(c) * sstride] = h;
        h += __builtin_fmaf(precise_expm1(An * dv[g]), h, sv[g]);
      }
    }
    st[int64_t(nc - 1) * sstride] = h;
  } else {
    // slot c <- adjoint entering chunk c from its end;  h <- a_c h + r_c, c = nc - 2 .. 1
    float h = st[int64_t(nc - 1) * sstride];
    st[int64_t(nc - 1) * sstride] = 0.0f;
    for (int c0 = nc - 2; c0 >= 1; c0 -= kWalkG) {
#pragma unroll
      for (int g = 0; g < kWalkG; ++g) {
        const int c = c0 - g >= 1 ? c0 - g : 1;
        sv[g] = st[int64_t(c) * sstride];
        dv[g] = ds[int64_t(c) * D];
      }
#pragma unroll
      for (int g = 0; g < kWalkG; ++g) {
        const int c = c0 - g;
        if (c < 1) break;
        st[int64_t(c) * sstride] = h;
        h += __builtin_fmaf(precise_expm1(An * dv[g]), h, sv[g]);
      }
    }
    st[0] = h;
  }
}

template <bool REVERSE>
__global__ __launch_bounds__(256) void chunk_walk_kernel(float* __restrict__ states,
                                                         const float* __restrict__ dsum,
                                                         const float* __restrict__ A,
                                                         const float* __restrict__ h0,
                                                         int64_t B, int64_t D, int N, int nc) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= B * N * D) return;
  chunk_walk<REVERSE>(states, dsum, A, h0, gid, D, N, nc);
}

// Both walks of the backward in one launch (they are independent): the first
// B N D lanes walk the start states forward, the next B N D the adjoints
// backward, so twice the lanes cover each other's memory waits.
__global__ __launch_bounds__(256) void chunk_walk_pair_kernel(float* __restrict__ hstates,
                                                              float* __restrict__ lstates,
                                                              const float* __restrict__ dsum,
                                                              const float* __restrict__ A,
                                                              const float* __restrict__ h0,
                                                              int64_t B, int64_t D, int N, int nc) {
  const int64_t total = B * N * D;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid < total) chunk_walk<false>(hstates, dsum, A, h0, gid, D, N, nc);
  else if (gid < 2 * total) chunk_walk<true>(lstates, dsum, A, nullptr, gid - total, D, N, nc);
}

}  // namespace

int launch_chunk_carry(float* states, const float* dsum, const float* A, const float* h0,
                       int64_t batch, int64_t D, int N, int nc, bool reverse, void* stream) {
  if (nc < 2) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (nc < kScanMinChunks) {
    const int64_t total = batch * N * D;
    const dim3 grid(unsigned((total + 255) / 256)), block(256);
    if (reverse)
      hipLaunchKernelGGL(chunk_walk_kernel<true>, grid, block, 0, st, states, dsum, A, h0, batch, D,
                         N, nc);
    else
      hipLaunchKernelGGL(chunk_walk_kernel<false>, grid, block, 0, st, states, dsum, A, h0, batch, D,
                         N, nc);
    return int(hipGetLastError());
  }
  const int ndblk = int((D + kCh - 1) / kCh);
  const dim3 grid(unsigned(batch * N * ndblk)), block(kWave * kWaves);
  if (reverse)
    hipLaunchKernelGGL(chunk_carry_kernel<true>, grid, block, 0, st, states, dsum, A, h0, D, N, nc,
                       ndblk);
  else
    hipLaunchKernelGGL(chunk_carry_kernel<false>, grid, block, 0, st, states, dsum, A, h0, D, N,
                       nc, ndblk);
  return int(hipGetLastError());
}

int launch_chunk_carry_pair(float* hstates, float* lstates, const float* dsum, const float* A,
                            const float* h0, int64_t batch, int64_t D, int N, int nc,
                            void* stream) {
  if (nc < 2) return 0;
  if (nc >= kScanMinChunks) {
    const int e = launch_chunk_carry(hstates, dsum, A, h0, batch, D, N, nc, false, stream);
    if (e != 0) return e;
    return launch_chunk_carry(lstates, dsum, A, nullptr, batch, D, N, nc, true, stream);
  }
  const int64_t total = 2 * batch * N * D;
  const dim3 grid(unsigned((total + 255) / 256)), block(256);
  hipLaunchKernelGGL(chunk_walk_pair_kernel, grid, block, 0, static_cast<hipStream_t>(stream),
                     hstates, lstates, dsum, A, h0, batch, D, N, nc);
  return int(hipGetLastError());
}

}  // namespace ss
