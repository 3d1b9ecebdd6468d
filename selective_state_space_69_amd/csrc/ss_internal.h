// Internal interface between the C-ABI layer (ss_api.cpp: validation and
// planning, pure host logic) and the HIP launchers (ss_fwd.hip, ss_bwd.hip,
// ss_step.hip).  Not installed; the public contract is include/ss_scan.h.
#pragma once

#include <cstddef>
#include <cstdint>

#include "ss_conv.h"
#include "ss_ssd.h"
#include "ss_scan.h"

namespace ss {

constexpr int kWave = 64;      // lanes per wavefront on CDNA
constexpr int kMaxState = 16;  // states held per lane
constexpr int kHalfWaveSplit = 8;
constexpr int kOneStateSplit = 16;

// How a forward (or the forward recompute inside the backward) is split.
// nsplit : waves per (b, 64-channel block), each holding 16 / nsplit states;
//          kHalfWaveSplit selects the 32-channel kernel (4 waves per
//          (b, 32-channel block), two states per lane), kOneStateSplit the
//          16-channel kernel (4 waves per (b, 16-channel block), one state per
//          lane).
// nchunks == 1: one sequential pass over time per workgroup.
// nchunks  > 1: (1) chunk summaries, (2) carry scan over chunks, (3) output pass.
struct TimePlan {
  int64_t chunk_len = 0;
  int64_t nchunks = 1;
  int nsplit = 1;
};

// Workspace layout of the forward: fp32 arrays, each 256-byte aligned.
//   brow, crow : (B, L, 16)    B and C rows padded with zeros to 16 states, in
//                              the input type (only when N < 16; else the inputs are read)
//   hend : (B, nchunks, N, D)  chunk-local end state, then (after the carry scan)
//                              the start state of the chunk
//   dsum : (B, nchunks, D)     sum over the chunk of the step, in log2 units
struct FwdPlan {
  TimePlan tp;
  bool packed_rows = false;
  size_t off_brow = 0, off_crow = 0, off_hend = 0, off_dsum = 0, bytes = 0;
};

// Backward workspace (fp32 arrays, 256-byte aligned):
//   brow, crow : (B, L, 16)   B and C rows padded to 16 states (only when N < 16)
//   hend, dsum : (B, nchunks, N, D), (B, nchunks, D)  forward chunk carries
//   lam        : (B, nchunks, N, D)  adjoint carry entering each chunk from its end
//   pB, pC     : (B, L, nblk, N)     dB, dC summed over one 64-channel block
//   pA         : (B, nchunks, N, D)  dA summed over one chunk
//   pD, pbias  : (B, nchunks, D)     dD_skip, ddelta_bias summed over one chunk
// The partial sums are added in a fixed order by reduction kernels, so the
// backward is deterministic.
struct BwdPlan {
  TimePlan tp;
  int64_t nblk = 0;
  bool packed_rows = false;
  size_t off_brow = 0, off_crow = 0, off_hend = 0, off_dsum = 0, off_lam = 0, off_pB = 0,
         off_pC = 0, off_pA = 0, off_pD = 0, off_pbias = 0, bytes = 0;
};

// SS_OK when the current device is a gfx950, SS_ERR_UNSUPPORTED for another
// architecture, SS_ERR_HIP when no device can be queried (ss_runtime.hip; the
// answer is cached per device).
int check_device();

// Size of the static scratch array of ss_scan_fwd_noalloc (ss_runtime.hip).
constexpr size_t kStaticScratchBytes = size_t(SS_SCAN_STATIC_SCRATCH_BYTES);
// This GPU's copy of that array (its device address, looked up once per
// device with the device current): SS_OK, SS_ERR_HIP or SS_ERR_UNSUPPORTED.
int static_scratch(void** out);

TimePlan plan_time(const ss_desc_t& d);
FwdPlan plan_fwd(const ss_desc_t& d);
BwdPlan plan_bwd(const ss_desc_t& d);

struct FwdArgs {
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
  void* Brow;    // B, C rows padded to 16 per (b, t), input type
  void* Crow;
  float* hend;
  float* dsum;
  int rev = 0;   // reverse time: h_t from h_{t+1}, t = L-1 .. 0
  int acc = 0;   // add the result to y instead of overwriting it
};

struct BwdArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  const float* bias;
  const void* z;
  const float* h0;
  const void* dy;
  float* du;
  float* ddelta;
  float* dA;
  float* dB;
  float* dC;
  float* dDskip;
  float* dbias;
  float* dz;
  float* dh0;
  char* ws;
};

struct StepArgs {
  float* h;
  const void* u;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  const float* bias;
  const void* z;
  void* y;
};

// Launchers: return 0 or a HIP error code (converted to SS_ERR_HIP by the caller).
int launch_fwd(const ss_desc_t& d, const FwdPlan& p, const FwdArgs& a, void* stream);
// B and C rows as (B, L, 16) in the input type, zero past N.
int launch_pack_rows(const ss_desc_t& d, const void* Bm, const void* Cm, void* Brow, void* Crow,
                     void* stream);
// Chunk start states of a chunked forward (summary pass + carry scan) into
// a.hend / a.dsum; a.Brow / a.Crow must hold the 16-wide rows.
int launch_fwd_carries(const ss_desc_t& d, const TimePlan& tp, const FwdArgs& a, void* stream);
int launch_bwd(const ss_desc_t& d, const BwdPlan& p, const BwdArgs& a, void* stream);
// Conv1d + SiLU (ss_conv.hip).  Time runs in independent segments of
// kConvSeg steps; vec = 4 channels per thread when D % 4 == 0, else 1.
// Backward workspace: per-segment partials of dw (B * nseg, D, K) and dbias
// (B * nseg, D), fp32, 256-byte aligned.
constexpr int kConvSeg = 64;
struct ConvPlan {
  int64_t nseg = 1;
  int vec = 1;
  size_t off_dw = 0, off_db = 0, bytes = 0;
};
ConvPlan plan_conv(const ss_conv_desc_t& d);
int launch_conv_fwd(const ss_conv_desc_t& d, const ConvPlan& plan, const void* x, const float* w,
                    const float* bias, void* u, void* stream);
int launch_conv_bwd(const ss_conv_desc_t& d, const ConvPlan& plan, const void* x, const float* w,
                    const float* bias, const float* du, float* dx, float* dw, float* dbias,
                    char* ws, void* stream);
int launch_conv_step(const ss_conv_desc_t& d, float* state, const void* x, const float* w,
                     const float* bias, void* u, void* stream);

// Chunk carries (ss_carry.hip), in place on states (B, nc, N, D): forward turns
// chunk summaries into chunk start states (h0 may be null), reverse turns local
// adjoints into the adjoints entering each chunk from its end.
int launch_chunk_carry(float* states, const float* dsum, const float* A, const float* h0,
                       int64_t batch, int64_t D, int N, int nc, bool reverse, void* stream);
// Both carries of the backward (forward on hstates, reverse on lstates), in
// one launch when the chunks are walked in order.
int launch_chunk_carry_pair(float* hstates, float* lstates, const float* dsum, const float* A,
                            const float* h0, int64_t batch, int64_t D, int N, int nc,
                            void* stream);
int launch_step(const ss_desc_t& d, const StepArgs& a, void* stream);
// Complex-A forward plan: 32 channels per workgroup, time cut into nchunks
// chunks of chunk_len steps (one when nchunks == 1).  Workspace (256-byte
// aligned): hend (B, nchunks, N, D) complex fp32 pairs (chunk summaries, then
// chunk start states) and dsum (B, nchunks, D) fp64 (sums of dt log2 e).
struct CplxPlan {
  int64_t chunk_len = 0;
  int64_t nchunks = 1;
  size_t off_hend = 0, off_dsum = 0, bytes = 0;
};
// allow_chunks = false: the one-pass plan (no workspace)
CplxPlan plan_fwd_complex(const ss_desc_t& d, bool allow_chunks);
// Complex-A forward (ss_complex.hip): A (D,N,2), B, C (B,L,N,2), h0 / h_last (B,D,N,2).
int launch_fwd_complex(const ss_desc_t& d, const CplxPlan& plan, const void* u, const void* delta,
                       const float* A, const void* Bm, const void* Cm, const float* Dskip,
                       const float* bias, const void* z, const float* h0, void* y, float* h_last,
                       char* ws, void* stream);
// Complex-A decode step (ss_complex.hip): h (B,D,N,2) in place, A (D,N,2), B, C (B,N,2).
int launch_step_complex(const ss_desc_t& d, const StepArgs& a, void* stream);
// SSD (Mamba-2) forward (ss_ssd.hip): one workgroup per (batch row, head);
// h0 / h_last (B, H, N, P) may be null and may be the same buffer.
int launch_ssd_fwd(const ss_ssd_desc_t& d, const void* x, const void* dt, const float* A,
                   const void* Bm, const void* Cm, const float* D, const float* dt_bias,
                   const float* h0, void* y, float* h_last, void* stream);
// SSD single step on the state h (B, H, N, P), in place (ss_ssd.hip).
int launch_ssd_step(const ss_ssd_desc_t& d, float* h, const void* x, const void* dt,
                    const float* A, const void* Bm, const void* Cm, const float* D,
                    const float* dt_bias, void* y, void* stream);

}  // namespace ss
