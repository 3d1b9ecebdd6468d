// C-ABI entry points of libssscan: argument validation, time planning and
// workspace layout.  Validation is plain host logic that runs before any HIP
// call, so every validation status can be produced (and tested) without a GPU;
// only then does an entry point ask whether the current device is a gfx950
// (check_device, cached per device) and launch.
#include <climits>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "ss_internal.h"

namespace ss {
namespace {

constexpr size_t kAlign = 256;     // workspace alignment
constexpr size_t kPtrAlign = 16;   // every tensor pointer (rows are read with 16-byte loads)
constexpr int64_t kBwdChunk = 32;   // backward time chunk (8 blocks of 4 steps)

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool valid_dtype(int32_t t) { return t == SS_F32 || t == SS_BF16; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Sizes must be positive and B*L*D, B*L*N must stay far below 2^62 bytes.
int check_desc(const ss_desc_t* d, bool need_len) {
  if (!d) return SS_ERR_INVALID_ARG;
  if (d->batch < 1 || d->dim < 1 || d->dstate < 1 || d->dstate > kMaxState) return SS_ERR_INVALID_ARG;
  if (need_len && d->seqlen < 1) return SS_ERR_INVALID_ARG;
  const int64_t lim = int64_t(1) << 40;
  // time indices are 32-bit in the kernels; a channel block's row stride in
  // bytes must fit a 32-bit buffer offset
  if (d->batch > lim || d->dim > (int64_t(1) << 24) || (need_len && d->seqlen > INT32_MAX - 64))
    return SS_ERR_INVALID_ARG;
  const int64_t L = need_len ? d->seqlen : 1;
  if (d->batch > lim / L || d->batch * L > lim / d->dim) return SS_ERR_INVALID_ARG;
  if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype)) return SS_ERR_UNSUPPORTED;
  if (d->disc != SS_ZOH && d->disc != SS_EULER) return SS_ERR_UNSUPPORTED;
  if (d->bc_stride != 0 && (d->bc_stride < d->dstate || d->bc_stride > (int64_t(1) << 20)))
    return SS_ERR_INVALID_ARG;
  return SS_OK;
}

// Alignment asked of Bm and Cm: rows read in place take 16-byte loads, rows
// with a stride are only read element by element (copied, or by the step).
size_t bc_align(const ss_desc_t& d) {
  return d.bc_stride == 0 ? kPtrAlign : (d.in_dtype == SS_BF16 ? 2 : 4);
}

bool bc_aligned(const ss_desc_t& d, const void* Bm, const void* Cm) {
  return aligned(Bm, bc_align(d)) && aligned(Cm, bc_align(d));
}

int64_t env_int(const char* name) {
  const char* s = std::getenv(name);
  if (!s || !*s) return 0;
  long long v = std::atoll(s);
  return v > 0 ? int64_t(v) : 0;
}

}  // namespace

// Work decomposition.  The scan is bound by the vector ALU (one v_exp_f32 and
// 4-6 FMA-class ops per element), and a SIMD running a single wave stalls on
// transcendental and LDS latency, so the plan aims for several waves per SIMD
// (the MI355X has 1024 SIMDs in 256 CUs) with the least redundant work.  With
// cols = B * ceil(D / 64) channel blocks (cols32, cols16: the same for 32 and
// 16 channels):
//  - cols >= 2048: one wave per block (16 states per lane), one pass;
//  - cols >= 512: one pass, either 64-channel groups with the states split
//    over 4 waves, or 32-channel groups with two states per lane (twice the
//    groups, 5% more instructions per element).  The second is taken when it
//    spreads the groups over the 256 CUs clearly more evenly: a CU holds at
//    most 4 of the first kind at a time and 5 of the second, and the time is
//    set by the most loaded CU (B = 8, D = 5120: 3 vs 2.5 groups' worth);
//  - cols32 >= 512: one pass on 32-channel groups (two or more waves per
//    SIMD; B = 8, D = 2560: 0.26 ms against 0.32 chunked);
//  - cols16 >= 384: one pass on 16-channel groups with one state per lane
//    (the same vector work per element, 1.5x the LDS instructions, three
//    groups per CU; Mamba-130M, B = 8, D = 1536: 0.142 ms against 0.180
//    chunked, 0.141 against 0.204 with exact ZOH; B = 4: 0.107 against 0.111;
//    at 192 groups, 0.090 against 0.068 chunked);
//  - fewer: 4 waves per 64-channel group and time cut into chunks of >= 128
//    steps, about 8192 waves in all; a chunked forward costs about 1.8x the
//    arithmetic (summary pass + output pass) but keeps every SIMD busy.
// Measured on MI355X for the Mamba-130M/2.8B shapes, B = 2 at L = 8192, the
// 1M-step case and a few widths between.  SS_SCAN_NSPLIT (1, 2, 4, 8 for the
// 32-channel kernel, 16 for the 16-channel one) and SS_SCAN_CHUNK override
// the choice.
TimePlan plan_time(const ss_desc_t& d) {
  TimePlan tp;
  const int64_t L = d.seqlen;
  const int64_t cols = d.batch * ((d.dim + kWave - 1) / kWave);
  const int64_t cols32 = d.batch * ((d.dim + 31) / 32);
  const int64_t cols16 = d.batch * ((d.dim + 15) / 16);
  constexpr int64_t kWide = 2048, kMid = 512, kNarrow16 = 384, kChunkWaves = 8192,
                    kMinChunk = 128, kCUs = 256;
  int nsplit = int(env_int("SS_SCAN_NSPLIT"));
  const bool forced_split = nsplit == 1 || nsplit == 2 || nsplit == 4 || nsplit == kHalfWaveSplit ||
                            nsplit == kOneStateSplit;
  bool one_pass = false;
  if (!forced_split) {
    one_pass = true;
    if (cols >= kWide) {
      nsplit = 1;
    } else if (cols >= kMid) {
      // most loaded CU, in units of one 64-channel group's work
      const double t4 = double((cols + kCUs - 1) / kCUs);
      const double t8 = 0.5 * 1.05 * double((cols32 + kCUs - 1) / kCUs);
      nsplit = t8 < 0.9 * t4 ? kHalfWaveSplit : 4;
    } else if (cols32 >= kMid) {
      nsplit = kHalfWaveSplit;
    } else if (cols16 >= kNarrow16) {
      nsplit = kOneStateSplit;
    } else {
      nsplit = 4;
      one_pass = false;
    }
  }
  int64_t chunk = env_int("SS_SCAN_CHUNK");
  if (chunk <= 0) {
    if (one_pass || cols >= kMid || L < 2 * kMinChunk) {
      chunk = L;
    } else {
      const int64_t waves = nsplit == kHalfWaveSplit   ? cols32 * 4
                            : nsplit == kOneStateSplit ? cols16 * 4
                                                       : cols * nsplit;
      const int64_t want = (kChunkWaves + waves - 1) / waves;
      chunk = (L + want - 1) / want;
      if (chunk < kMinChunk) chunk = kMinChunk;
      chunk = (chunk + 15) / 16 * 16;
    }
  }
  if (chunk > L) chunk = L;
  tp.chunk_len = chunk;
  tp.nchunks = (L + chunk - 1) / chunk;
  tp.nsplit = nsplit;
  return tp;
}

FwdPlan plan_fwd(const ss_desc_t& d) {
  FwdPlan p;
  p.tp = plan_time(d);
  const size_t B = size_t(d.batch), L = size_t(d.seqlen), C = size_t(p.tp.nchunks),
               D = size_t(d.dim), N = size_t(d.dstate);
  size_t off = 0;
  p.packed_rows = d.dstate != kMaxState || d.bc_stride != 0;
  const size_t es = d.in_dtype == SS_BF16 ? 2 : 4;
  if (p.packed_rows) {
    p.off_brow = off; off += align_up(B * L * kMaxState * es);
    p.off_crow = off; off += align_up(B * L * kMaxState * es);
  }
  if (p.tp.nchunks > 1) {
    p.off_hend = off; off += align_up(B * C * N * D * sizeof(float));
    p.off_dsum = off; off += align_up(B * C * D * sizeof(float));
  }
  p.bytes = off;
  return p;
}

// The backward always splits the states over 4 waves and cuts time into chunks
// of 32 steps: a chunk's 8 block checkpoints then fit in registers.
BwdPlan plan_bwd(const ss_desc_t& d) {
  BwdPlan p;
  p.tp.nsplit = 4;
  p.tp.chunk_len = d.seqlen < kBwdChunk ? d.seqlen : kBwdChunk;
  p.tp.nchunks = (d.seqlen + p.tp.chunk_len - 1) / p.tp.chunk_len;
  const size_t B = size_t(d.batch), L = size_t(d.seqlen), C = size_t(p.tp.nchunks),
               D = size_t(d.dim), N = size_t(d.dstate);
  p.nblk = (d.dim + kWave - 1) / kWave;
  const size_t nb = size_t(p.nblk);
  p.packed_rows = d.dstate != kMaxState || d.bc_stride != 0;
  const size_t es = d.in_dtype == SS_BF16 ? 2 : 4;
  size_t off = 0;
  if (p.packed_rows) {
    p.off_brow = off; off += align_up(B * L * kMaxState * es);
    p.off_crow = off; off += align_up(B * L * kMaxState * es);
  }
  p.off_hend = off; off += align_up(B * C * N * D * sizeof(float));
  p.off_dsum = off; off += align_up(B * C * D * sizeof(float));
  p.off_lam = off;  off += align_up(B * C * N * D * sizeof(float));
  p.off_pB = off;   off += align_up(B * L * nb * N * sizeof(float));
  p.off_pC = off;   off += align_up(B * L * nb * N * sizeof(float));
  p.off_pA = off;   off += align_up(B * C * N * D * sizeof(float));
  p.off_pD = off;   off += align_up(B * C * D * sizeof(float));
  p.off_pbias = off; off += align_up(B * C * D * sizeof(float));
  p.bytes = off;
  return p;
}

// Complex-A forward: 32-channel workgroups, five per compute unit when the
// problem is wide enough (B * ceil(D / 32) >= 640 groups, or short sequences:
// one pass); otherwise time chunks of >= 128 steps so that about 1280
// workgroups run, at the cost of the summary pass (the real scan's plan, with
// the complex kernel's group size).  SS_SCAN_CHUNK overrides the chunk length.
CplxPlan plan_fwd_complex(const ss_desc_t& d, bool allow_chunks) {
  CplxPlan p;
  const int64_t L = d.seqlen;
  const int64_t cols = d.batch * ((d.dim + 31) / 32);
  constexpr int64_t kWide = 640, kWant = 1280, kMinChunk = 128;
  int64_t chunk = L;
  if (allow_chunks) {
    const int64_t forced = env_int("SS_SCAN_CHUNK");
    if (forced > 0) {
      chunk = forced;
    } else if (cols < kWide && L >= 2 * kMinChunk) {
      const int64_t want = (kWant + cols - 1) / cols;
      chunk = (L + want - 1) / want;
      if (chunk < kMinChunk) chunk = kMinChunk;
      chunk = (chunk + 15) / 16 * 16;
    }
  }
  if (chunk > L) chunk = L;
  p.chunk_len = chunk;
  p.nchunks = (L + chunk - 1) / chunk;
  if (p.nchunks > 1) {
    const size_t B = size_t(d.batch), C = size_t(p.nchunks), D = size_t(d.dim),
                 N = size_t(d.dstate);
    size_t off = 0;
    p.off_hend = off; off += align_up(B * C * N * D * 2 * sizeof(float));
    p.off_dsum = off; off += align_up(B * C * D * sizeof(double));
    p.bytes = off;
  }
  return p;
}

namespace {

// Conv1d descriptions: positive sizes, width 1..4, 32-bit segment count.
int check_conv(const ss_conv_desc_t* d, bool need_len) {
  if (!d) return SS_ERR_INVALID_ARG;
  if (d->batch < 1 || d->dim < 1 || d->width < 1 || d->width > 4) return SS_ERR_INVALID_ARG;
  if (need_len && d->seqlen < 1) return SS_ERR_INVALID_ARG;
  const int64_t lim = int64_t(1) << 40;
  const int64_t L = need_len ? d->seqlen : 1;
  if (d->batch > lim || d->dim > lim || L > (int64_t(INT32_MAX) - 64) ||
      d->batch > lim / L || d->batch * L > lim / d->dim)
    return SS_ERR_INVALID_ARG;
  if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype)) return SS_ERR_UNSUPPORTED;
  return SS_OK;
}

// SSD descriptions: positive sizes, heads divisible into groups, 32-bit grid
// (seqlen checked only where the call reads it).
int check_ssd(const ss_ssd_desc_t* d, bool need_len = true) {
  if (!d || d->reserved != 0) return SS_ERR_INVALID_ARG;
  if (d->batch < 1 || (need_len && d->seqlen < 1) || d->nheads < 1 || d->headdim < 1 ||
      d->dstate < 1 ||
      d->ngroups < 1 || d->nheads % d->ngroups != 0)
    return SS_ERR_INVALID_ARG;
  const int64_t lim = int64_t(1) << 40;
  const int64_t L = need_len ? d->seqlen : 1;
  if (d->batch > lim || L > lim || d->nheads > lim || d->ngroups > lim ||
      d->batch > (int64_t(INT32_MAX) / d->nheads) || d->batch * L > lim / d->nheads)
    return SS_ERR_INVALID_ARG;
  if (d->headdim != 64 || d->dstate != 64) return SS_ERR_UNSUPPORTED;
  if (d->in_dtype != SS_BF16 || !valid_dtype(d->out_dtype)) return SS_ERR_UNSUPPORTED;
  return SS_OK;
}

}  // namespace

ConvPlan plan_conv(const ss_conv_desc_t& d) {
  ConvPlan p;
  p.nseg = (d.seqlen + kConvSeg - 1) / kConvSeg;
  p.vec = d.dim % 4 == 0 ? 4 : 1;
  const size_t parts = size_t(d.batch) * size_t(p.nseg), D = size_t(d.dim);
  p.off_dw = 0;
  p.off_db = align_up(parts * D * size_t(d.width) * sizeof(float));
  p.bytes = p.off_db + align_up(parts * D * sizeof(float));
  return p;
}

}  // namespace ss

using namespace ss;

namespace {

// The forward in either direction.  static_ws: the scratch is the library's
// static array (ss_scan_fwd_noalloc) instead of the caller's workspace.
int fwd_call(const ss_desc_t* desc, int direction, int accumulate, const void* u,
             const void* delta, const float* A, const void* Bm, const void* Cm,
             const float* D_skip, const float* delta_bias, const void* z, const float* h0,
             void* y, float* h_last, void* workspace, size_t ws_bytes, bool static_ws,
             void* stream) {
  int rc = check_desc(desc, true);
  if (rc != SS_OK) return rc;
  if (direction != SS_DIR_FORWARD && direction != SS_DIR_REVERSE) return SS_ERR_INVALID_ARG;
  if (!u || !delta || !A || !Bm || !Cm || !y) return SS_ERR_INVALID_ARG;
  if (h_last && h0 && static_cast<const void*>(h_last) == static_cast<const void*>(h0))
    return SS_ERR_INVALID_ARG;
  const void* ptrs[] = {u, delta, z, A, D_skip, delta_bias, h0, h_last, y};
  for (const void* p : ptrs)
    if (p && !aligned(p, kPtrAlign)) return SS_ERR_INVALID_ARG;
  if (!bc_aligned(*desc, Bm, Cm)) return SS_ERR_INVALID_ARG;
  const FwdPlan plan = plan_fwd(*desc);
  if (static_ws) {
    if (plan.bytes > kStaticScratchBytes) return SS_ERR_SCRATCH_LIMIT;
  } else if (plan.bytes > 0 &&
             (!workspace || ws_bytes < plan.bytes || !aligned(workspace, kAlign))) {
    return SS_ERR_WORKSPACE;
  }
  if ((rc = check_device()) != SS_OK) return rc;
  if (static_ws && plan.bytes > 0 && (rc = static_scratch(&workspace)) != SS_OK) return rc;
  FwdArgs a{u, delta, A, Bm, Cm, D_skip, delta_bias, z, h0, y, h_last,
            nullptr, nullptr, nullptr, nullptr};
  a.rev = direction == SS_DIR_REVERSE;
  a.acc = accumulate != 0;
  char* ws = static_cast<char*>(workspace);
  if (plan.packed_rows) {
    a.Brow = ws + plan.off_brow;
    a.Crow = ws + plan.off_crow;
  }
  if (plan.tp.nchunks > 1) {
    a.hend = reinterpret_cast<float*>(ws + plan.off_hend);
    a.dsum = reinterpret_cast<float*>(ws + plan.off_dsum);
  }
  return launch_fwd(*desc, plan, a, stream) == 0 ? SS_OK : SS_ERR_HIP;
}

}  // namespace

extern "C" {

int ss_scan_version(void) { return 20000; }

int ss_scan_arch_supported(const char* arch_name) {
  if (!arch_name) return SS_ERR_INVALID_ARG;
  // "gfx950" alone or followed by target features ("gfx950:sramecc+:xnack-")
  static const char kArch[] = "gfx950";
  if (std::strncmp(arch_name, kArch, sizeof(kArch) - 1) != 0) return SS_ERR_UNSUPPORTED;
  const char next = arch_name[sizeof(kArch) - 1];
  return (next == '\0' || next == ':') ? SS_OK : SS_ERR_UNSUPPORTED;
}

const char* ss_scan_strerror(int status) {
  switch (status) {
    case SS_OK: return "ok";
    case SS_ERR_INVALID_ARG: return "invalid argument (null required pointer, size out of range, misaligned pointer or aliasing)";
    case SS_ERR_UNSUPPORTED: return "unsupported dtype, discretisation or option combination, or the current device is not a gfx950";
    case SS_ERR_WORKSPACE: return "workspace missing or smaller than ss_scan_workspace_bytes()";
    case SS_ERR_HIP: return "HIP kernel launch failed";
    case SS_ERR_SCRATCH_LIMIT: return "the plan needs more scratch than the static array of ss_scan_fwd_noalloc (SS_SCAN_STATIC_SCRATCH_BYTES); use ss_scan_fwd with a workspace";
    default: return "unknown status";
  }
}

size_t ss_scan_workspace_bytes(const ss_desc_t* desc, int op) {
  if (check_desc(desc, true) != SS_OK) return 0;
  if (op == SS_OP_FWD) return plan_fwd(*desc).bytes;
  if (op == SS_OP_BWD) return plan_bwd(*desc).bytes;
  if (op == SS_OP_FWD_COMPLEX) return desc->bc_stride ? 0 : plan_fwd_complex(*desc, true).bytes;
  return 0;
}

int ss_scan_fwd(const ss_desc_t* desc, const void* u, const void* delta, const float* A,
                const void* Bm, const void* Cm, const float* D_skip, const float* delta_bias,
                const void* z, const float* h0, void* y, float* h_last, void* workspace,
                size_t ws_bytes, void* stream) {
  return ss_scan_fwd_dir(desc, SS_DIR_FORWARD, 0, u, delta, A, Bm, Cm, D_skip, delta_bias, z, h0,
                         y, h_last, workspace, ws_bytes, stream);
}

int ss_scan_fwd_dir(const ss_desc_t* desc, int direction, int accumulate, const void* u,
                    const void* delta, const float* A, const void* Bm, const void* Cm,
                    const float* D_skip, const float* delta_bias, const void* z, const float* h0,
                    void* y, float* h_last, void* workspace, size_t ws_bytes, void* stream) {
  return fwd_call(desc, direction, accumulate, u, delta, A, Bm, Cm, D_skip, delta_bias, z, h0, y,
                  h_last, workspace, ws_bytes, false, stream);
}

int ss_scan_fwd_noalloc(const ss_desc_t* desc, const void* u, const void* delta, const float* A,
                        const void* Bm, const void* Cm, const float* D_skip,
                        const float* delta_bias, const void* z, const float* h0, void* y,
                        float* h_last, void* stream) {
  return fwd_call(desc, SS_DIR_FORWARD, 0, u, delta, A, Bm, Cm, D_skip, delta_bias, z, h0, y,
                  h_last, nullptr, 0, true, stream);
}

int ss_scan_fwd_complex_ws(const ss_desc_t* desc, const void* u, const void* delta,
                           const float* A, const void* Bm, const void* Cm, const float* D_skip,
                           const float* delta_bias, const void* z, const float* h0, void* y,
                           float* h_last, void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc, true);
  if (rc != SS_OK) return rc;
  if (desc->bc_stride != 0) return SS_ERR_UNSUPPORTED;
  if (!u || !delta || !A || !Bm || !Cm || !y) return SS_ERR_INVALID_ARG;
  if (h_last && h0 && static_cast<const void*>(h_last) == static_cast<const void*>(h0))
    return SS_ERR_INVALID_ARG;
  const void* ptrs[] = {u, delta, Bm, Cm, z, A, D_skip, delta_bias, h0, h_last, y};
  for (const void* p : ptrs)
    if (p && !aligned(p, kPtrAlign)) return SS_ERR_INVALID_ARG;
  // the one-pass plan when the caller brings no workspace at all
  const CplxPlan plan = plan_fwd_complex(*desc, workspace != nullptr || ws_bytes != 0);
  if (plan.bytes > 0 && (!workspace || ws_bytes < plan.bytes || !aligned(workspace, kAlign)))
    return SS_ERR_WORKSPACE;
  if ((rc = check_device()) != SS_OK) return rc;
  return launch_fwd_complex(*desc, plan, u, delta, A, Bm, Cm, D_skip, delta_bias, z, h0, y,
                            h_last, static_cast<char*>(workspace), stream) == 0
             ? SS_OK
             : SS_ERR_HIP;
}

int ss_scan_fwd_complex(const ss_desc_t* desc, const void* u, const void* delta, const float* A,
                        const void* Bm, const void* Cm, const float* D_skip,
                        const float* delta_bias, const void* z, const float* h0, void* y,
                        float* h_last, void* stream) {
  return ss_scan_fwd_complex_ws(desc, u, delta, A, Bm, Cm, D_skip, delta_bias, z, h0, y, h_last,
                                nullptr, 0, stream);
}

int ss_scan_bwd(const ss_desc_t* desc, const void* u, const void* delta, const float* A,
                const void* Bm, const void* Cm, const float* D_skip, const float* delta_bias,
                const void* z, const float* h0, const void* dy, void* du, void* ddelta,
                float* dA, float* dB, float* dC, float* dD_skip, float* ddelta_bias, void* dz,
                float* dh0, void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc, true);
  if (rc != SS_OK) return rc;
  if (desc->out_dtype != SS_F32) return SS_ERR_UNSUPPORTED;
  if (!u || !delta || !A || !Bm || !Cm || !dy || !du || !ddelta || !dA || !dB || !dC)
    return SS_ERR_INVALID_ARG;
  if ((D_skip != nullptr) != (dD_skip != nullptr)) return SS_ERR_INVALID_ARG;
  if ((delta_bias != nullptr) != (ddelta_bias != nullptr)) return SS_ERR_INVALID_ARG;
  if ((z != nullptr) != (dz != nullptr)) return SS_ERR_INVALID_ARG;
  const void* ptrs[] = {u, delta, z, dy, A, D_skip, delta_bias, h0, du, ddelta,
                        dA, dB, dC, dD_skip, ddelta_bias, dz, dh0};
  for (const void* p : ptrs)
    if (p && !aligned(p, kPtrAlign)) return SS_ERR_INVALID_ARG;
  if (!bc_aligned(*desc, Bm, Cm)) return SS_ERR_INVALID_ARG;
  const BwdPlan plan = plan_bwd(*desc);
  if (plan.bytes > 0 && (!workspace || ws_bytes < plan.bytes || !aligned(workspace, kAlign)))
    return SS_ERR_WORKSPACE;
  BwdArgs a{u, delta, A, Bm, Cm, D_skip, delta_bias, z, h0, dy,
            static_cast<float*>(du), static_cast<float*>(ddelta), dA, dB, dC, dD_skip,
            ddelta_bias, static_cast<float*>(dz), dh0, static_cast<char*>(workspace)};
  if ((rc = check_device()) != SS_OK) return rc;
  return launch_bwd(*desc, plan, a, stream) == 0 ? SS_OK : SS_ERR_HIP;
}

int ss_scan_step(const ss_desc_t* desc, float* h, const void* u, const void* delta,
                 const float* A, const void* Bm, const void* Cm, const float* D_skip,
                 const float* delta_bias, const void* z, void* y, void* stream) {
  int rc = check_desc(desc, false);
  if (rc != SS_OK) return rc;
  if (!h || !u || !delta || !A || !Bm || !Cm || !y) return SS_ERR_INVALID_ARG;
  if (desc->batch * desc->dim > (int64_t(1) << 33)) return SS_ERR_INVALID_ARG;   // 32-bit grid
  // y is written while other lanes still read the state and the inputs
  const void* hv = h;
  if (y == hv || y == u || y == delta || y == Bm || y == Cm || y == z) return SS_ERR_INVALID_ARG;
  const void* ptrs[] = {h, u, delta, A, D_skip, delta_bias, z, y};
  for (const void* p : ptrs)
    if (p && !aligned(p, kPtrAlign)) return SS_ERR_INVALID_ARG;
  if (!bc_aligned(*desc, Bm, Cm)) return SS_ERR_INVALID_ARG;
  StepArgs a{h, u, delta, A, Bm, Cm, D_skip, delta_bias, z, y};
  if ((rc = check_device()) != SS_OK) return rc;
  return launch_step(*desc, a, stream) == 0 ? SS_OK : SS_ERR_HIP;
}

int ss_scan_step_complex(const ss_desc_t* desc, float* h, const void* u, const void* delta,
                         const float* A, const void* Bm, const void* Cm, const float* D_skip,
                         const float* delta_bias, const void* z, void* y, void* stream) {
  int rc = check_desc(desc, false);
  if (rc != SS_OK) return rc;
  if (desc->bc_stride != 0) return SS_ERR_UNSUPPORTED;
  if (!h || !u || !delta || !A || !Bm || !Cm || !y) return SS_ERR_INVALID_ARG;
  if (desc->batch * desc->dim > (int64_t(1) << 33)) return SS_ERR_INVALID_ARG;   // 32-bit grid
  const void* hv = h;
  if (y == hv || y == u || y == delta || y == Bm || y == Cm || y == z) return SS_ERR_INVALID_ARG;
  const void* ptrs[] = {h, u, delta, A, Bm, Cm, D_skip, delta_bias, z, y};
  for (const void* p : ptrs)
    if (p && !aligned(p, kPtrAlign)) return SS_ERR_INVALID_ARG;
  StepArgs a{h, u, delta, A, Bm, Cm, D_skip, delta_bias, z, y};
  if ((rc = check_device()) != SS_OK) return rc;
  return launch_step_complex(*desc, a, stream) == 0 ? SS_OK : SS_ERR_HIP;
}

size_t ss_conv1d_workspace_bytes(const ss_conv_desc_t* desc) {
  if (check_conv(desc, true) != SS_OK) return 0;
  return plan_conv(*desc).bytes;
}

int ss_conv1d_fwd(const ss_conv_desc_t* desc, const void* x, const float* w, const float* bias,
                  void* u, void* stream) {
  int rc = check_conv(desc, true);
  if (rc != SS_OK) return rc;
  if (!x || !w || !u || x == u) return SS_ERR_INVALID_ARG;
  const void* ptrs[] = {x, w, bias, u};
  for (const void* p : ptrs)
    if (p && !aligned(p, kPtrAlign)) return SS_ERR_INVALID_ARG;
  if ((rc = check_device()) != SS_OK) return rc;
  return launch_conv_fwd(*desc, plan_conv(*desc), x, w, bias, u, stream) == 0 ? SS_OK : SS_ERR_HIP;
}

int ss_conv1d_bwd(const ss_conv_desc_t* desc, const void* x, const float* w, const float* bias,
                  const float* du, float* dx, float* dw, float* dbias, void* workspace,
                  size_t ws_bytes, void* stream) {
  int rc = check_conv(desc, true);
  if (rc != SS_OK) return rc;
  if (!x || !w || !du || !dx || !dw) return SS_ERR_INVALID_ARG;
  if ((bias != nullptr) != (dbias != nullptr)) return SS_ERR_INVALID_ARG;
  if (static_cast<const void*>(dx) == x || dx == du) return SS_ERR_INVALID_ARG;
  const void* ptrs[] = {x, w, bias, du, dx, dw, dbias};
  for (const void* p : ptrs)
    if (p && !aligned(p, kPtrAlign)) return SS_ERR_INVALID_ARG;
  const ConvPlan plan = plan_conv(*desc);
  if (!workspace || ws_bytes < plan.bytes || !aligned(workspace, kAlign)) return SS_ERR_WORKSPACE;
  if ((rc = check_device()) != SS_OK) return rc;
  return launch_conv_bwd(*desc, plan, x, w, bias, du, dx, dw, dbias,
                         static_cast<char*>(workspace), stream) == 0
             ? SS_OK
             : SS_ERR_HIP;
}

int ss_conv1d_step(const ss_conv_desc_t* desc, float* state, const void* x, const float* w,
                   const float* bias, void* u, void* stream) {
  int rc = check_conv(desc, false);
  if (rc != SS_OK) return rc;
  if (!x || !w || !u || (!state && desc->width > 1)) return SS_ERR_INVALID_ARG;
  const void* ptrs[] = {state, x, w, bias, u};
  for (const void* p : ptrs)
    if (p && !aligned(p, kPtrAlign)) return SS_ERR_INVALID_ARG;
  if ((rc = check_device()) != SS_OK) return rc;
  return launch_conv_step(*desc, state, x, w, bias, u, stream) == 0 ? SS_OK : SS_ERR_HIP;
}

int ss_ssd_fwd_state(const ss_ssd_desc_t* desc, const void* x, const void* dt, const float* A,
                     const void* Bm, const void* Cm, const float* D, const float* dt_bias,
                     const float* h0, void* y, float* h_last, void* stream) {
  int rc = check_ssd(desc);
  if (rc != SS_OK) return rc;
  if (!x || !dt || !A || !Bm || !Cm || !y) return SS_ERR_INVALID_ARG;
  if (y == x || y == dt || y == Bm || y == Cm) return SS_ERR_INVALID_ARG;
  if (h0 && (static_cast<const void*>(h0) == y)) return SS_ERR_INVALID_ARG;
  if (h_last) {
    const void* hl = h_last;
    if (hl == x || hl == dt || hl == Bm || hl == Cm || hl == y || h_last == A || h_last == D ||
        h_last == dt_bias)
      return SS_ERR_INVALID_ARG;
  }
  const void* ptrs[] = {x, dt, A, Bm, Cm, D, dt_bias, h0, y, h_last};
  for (const void* p : ptrs)
    if (p && !aligned(p, kPtrAlign)) return SS_ERR_INVALID_ARG;
  if ((rc = check_device()) != SS_OK) return rc;
  return launch_ssd_fwd(*desc, x, dt, A, Bm, Cm, D, dt_bias, h0, y, h_last, stream) == 0
             ? SS_OK
             : SS_ERR_HIP;
}

int ss_ssd_fwd(const ss_ssd_desc_t* desc, const void* x, const void* dt, const float* A,
               const void* Bm, const void* Cm, const float* D, const float* dt_bias, void* y,
               void* stream) {
  return ss_ssd_fwd_state(desc, x, dt, A, Bm, Cm, D, dt_bias, nullptr, y, nullptr, stream);
}

int ss_ssd_step(const ss_ssd_desc_t* desc, float* h, const void* x, const void* dt,
                const float* A, const void* Bm, const void* Cm, const float* D,
                const float* dt_bias, void* y, void* stream) {
  int rc = check_ssd(desc, false);
  if (rc != SS_OK) return rc;
  if (!h || !x || !dt || !A || !Bm || !Cm || !y) return SS_ERR_INVALID_ARG;
  const void* hv = h;
  if (y == x || y == dt || y == Bm || y == Cm || y == hv) return SS_ERR_INVALID_ARG;
  if (hv == x || hv == dt || hv == Bm || hv == Cm || h == A || h == D || h == dt_bias)
    return SS_ERR_INVALID_ARG;
  const void* ptrs[] = {h, x, dt, A, Bm, Cm, D, dt_bias, y};
  for (const void* p : ptrs)
    if (p && !aligned(p, kPtrAlign)) return SS_ERR_INVALID_ARG;
  if ((rc = check_device()) != SS_OK) return rc;
  return launch_ssd_step(*desc, h, x, dt, A, Bm, Cm, D, dt_bias, y, stream) == 0 ? SS_OK
                                                                                  : SS_ERR_HIP;
}

}  // extern "C"
