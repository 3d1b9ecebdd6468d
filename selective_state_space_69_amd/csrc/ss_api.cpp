// C-ABI entry points of libssscan: argument validation, time planning and
// workspace layout.  Everything here is plain host logic that runs before any
// HIP call, so every status code can be produced (and tested) without a GPU.
#include <climits>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "ss_internal.h"

namespace ss {
namespace {

constexpr size_t kAlign = 256;     // workspace alignment
constexpr size_t kPtrAlign = 16;   // every tensor pointer (rows are read with 16-byte loads)

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
  return SS_OK;
}

int64_t env_chunk() {
  const char* s = std::getenv("SS_SCAN_CHUNK");
  if (!s || !*s) return 0;
  long long v = std::atoll(s);
  return v > 0 ? int64_t(v) : 0;
}

}  // namespace

// Split the sequence into chunks when one pass per (b, 64-channel block) would
// leave most of the GPU idle.  A chunked forward costs about 1.8x the arithmetic
// (summary pass + output pass), so chunking is only chosen when the sequential
// plan would fill less than half of the 1024 SIMDs of a 256-CU MI355X.
TimePlan plan_time(const ss_desc_t& d) {
  TimePlan tp;
  const int64_t L = d.seqlen;
  const int64_t cols = d.batch * ((d.dim + kWave - 1) / kWave);
  int64_t chunk = env_chunk();
  if (chunk <= 0) {
    constexpr int64_t kSimds = 1024, kTargetWaves = 2048, kMinChunk = 64;
    if (cols >= kSimds / 2 || L <= 2 * kMinChunk) {
      chunk = L;
    } else {
      int64_t want = (kTargetWaves + cols - 1) / cols;
      chunk = (L + want - 1) / want;
      if (chunk < kMinChunk) chunk = kMinChunk;
      chunk = (chunk + 15) / 16 * 16;
    }
  }
  if (chunk > L) chunk = L;
  tp.chunk_len = chunk;
  tp.nchunks = (L + chunk - 1) / chunk;
  return tp;
}

FwdPlan plan_fwd(const ss_desc_t& d) {
  FwdPlan p;
  p.tp = plan_time(d);
  if (p.tp.nchunks > 1) {
    const size_t B = size_t(d.batch), C = size_t(p.tp.nchunks), D = size_t(d.dim), N = size_t(d.dstate);
    p.off_hend = 0;
    p.off_dsum = align_up(B * C * N * D * sizeof(float));
    p.bytes = p.off_dsum + align_up(B * C * D * sizeof(float));
  }
  return p;
}

BwdPlan plan_bwd(const ss_desc_t& d) {
  BwdPlan p;
  p.tp = plan_time(d);
  const size_t B = size_t(d.batch), L = size_t(d.seqlen), C = size_t(p.tp.nchunks),
               D = size_t(d.dim), N = size_t(d.dstate);
  p.nblk = (d.dim + kWave - 1) / kWave;
  const size_t nb = size_t(p.nblk);
  size_t off = 0;
  p.off_hend = off; off += align_up(B * C * N * D * sizeof(float));
  p.off_dsum = off; off += align_up(B * C * D * sizeof(float));
  p.off_lam = off;  off += align_up(B * C * N * D * sizeof(float));
  p.off_lsum = off; off += align_up(B * C * D * sizeof(float));
  p.off_pB = off;   off += align_up(B * L * nb * N * sizeof(float));
  p.off_pC = off;   off += align_up(B * L * nb * N * sizeof(float));
  p.off_pA = off;   off += align_up(B * C * N * D * sizeof(float));
  p.off_pD = off;   off += align_up(B * C * D * sizeof(float));
  p.off_pbias = off; off += align_up(B * C * D * sizeof(float));
  p.bytes = off;
  return p;
}

}  // namespace ss

using namespace ss;

extern "C" {

int ss_scan_version(void) { return 10000; }

const char* ss_scan_strerror(int status) {
  switch (status) {
    case SS_OK: return "ok";
    case SS_ERR_INVALID_ARG: return "invalid argument (null required pointer, size out of range, misaligned pointer or aliasing)";
    case SS_ERR_UNSUPPORTED: return "unsupported dtype, discretisation or option combination";
    case SS_ERR_WORKSPACE: return "workspace missing or smaller than ss_scan_workspace_bytes()";
    case SS_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

size_t ss_scan_workspace_bytes(const ss_desc_t* desc, int op) {
  if (check_desc(desc, true) != SS_OK) return 0;
  if (op == SS_OP_FWD) return plan_fwd(*desc).bytes;
  if (op == SS_OP_BWD) return plan_bwd(*desc).bytes;
  return 0;
}

int ss_scan_fwd(const ss_desc_t* desc, const void* u, const void* delta, const float* A,
                const void* Bm, const void* Cm, const float* D_skip, const float* delta_bias,
                const void* z, const float* h0, void* y, float* h_last, void* workspace,
                size_t ws_bytes, void* stream) {
  int rc = check_desc(desc, true);
  if (rc != SS_OK) return rc;
  if (!u || !delta || !A || !Bm || !Cm || !y) return SS_ERR_INVALID_ARG;
  if (h_last && h0 && static_cast<const void*>(h_last) == static_cast<const void*>(h0))
    return SS_ERR_INVALID_ARG;
  const void* ptrs[] = {u, delta, Bm, Cm, z, A, D_skip, delta_bias, h0, h_last, y};
  for (const void* p : ptrs)
    if (p && !aligned(p, kPtrAlign)) return SS_ERR_INVALID_ARG;
  const FwdPlan plan = plan_fwd(*desc);
  if (plan.bytes > 0 && (!workspace || ws_bytes < plan.bytes || !aligned(workspace, kAlign)))
    return SS_ERR_WORKSPACE;
  FwdArgs a{u, delta, A, Bm, Cm, D_skip, delta_bias, z, h0, y, h_last, nullptr, nullptr};
  if (plan.bytes > 0) {
    char* ws = static_cast<char*>(workspace);
    a.hend = reinterpret_cast<float*>(ws + plan.off_hend);
    a.dsum = reinterpret_cast<float*>(ws + plan.off_dsum);
  }
  return launch_fwd(*desc, plan, a, stream) == 0 ? SS_OK : SS_ERR_HIP;
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
  const void* ptrs[] = {u, delta, Bm, Cm, z, dy, A, D_skip, delta_bias, h0, du, ddelta,
                        dA, dB, dC, dD_skip, ddelta_bias, dz, dh0};
  for (const void* p : ptrs)
    if (p && !aligned(p, kPtrAlign)) return SS_ERR_INVALID_ARG;
  const BwdPlan plan = plan_bwd(*desc);
  if (plan.bytes > 0 && (!workspace || ws_bytes < plan.bytes || !aligned(workspace, kAlign)))
    return SS_ERR_WORKSPACE;
  BwdArgs a{u, delta, A, Bm, Cm, D_skip, delta_bias, z, h0, dy,
            static_cast<float*>(du), static_cast<float*>(ddelta), dA, dB, dC, dD_skip,
            ddelta_bias, static_cast<float*>(dz), dh0, static_cast<char*>(workspace)};
  return launch_bwd(*desc, plan, a, stream) == 0 ? SS_OK : SS_ERR_HIP;
}

int ss_scan_step(const ss_desc_t* desc, float* h, const void* u, const void* delta,
                 const float* A, const void* Bm, const void* Cm, const float* D_skip,
                 const float* delta_bias, const void* z, void* y, void* stream) {
  int rc = check_desc(desc, false);
  if (rc != SS_OK) return rc;
  if (!h || !u || !delta || !A || !Bm || !Cm || !y) return SS_ERR_INVALID_ARG;
  const void* ptrs[] = {h, u, delta, A, Bm, Cm, D_skip, delta_bias, z, y};
  for (const void* p : ptrs)
    if (p && !aligned(p, kPtrAlign)) return SS_ERR_INVALID_ARG;
  StepArgs a{h, u, delta, A, Bm, Cm, D_skip, delta_bias, z, y};
  return launch_step(*desc, a, stream) == 0 ? SS_OK : SS_ERR_HIP;
}

}  // extern "C"
