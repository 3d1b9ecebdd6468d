// Parameters shared by the forward scan kernels (ss_fwd_kernels.hpp: one wave
// per 64 channels and a slice of the states; ss_fwd_hw.hpp: 32 or 16 channels
// per workgroup with two states or one per lane) and by their launchers.
#pragma once

#include "ss_device.hpp"

namespace ss {

constexpr int kZoh = SS_ZOH;
constexpr int kEuler = SS_EULER;
constexpr int kBlk = 8;   // time steps per block: prefetch ring, B/C staging, partial sums

struct FwdParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* Brow;    // (B, L, 16) rows of B in the input type (zero past N)
  const void* Crow;    // (B, L, 16) rows of C
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
  // Time direction.  Logical step t of a batch row is physical step t
  // (forward) or L - 1 - t (reverse); the recurrence always runs over logical
  // steps.  Buffer offsets cannot be negative, so in reverse a block of BLK
  // steps is addressed from its last logical step (its lowest address) and
  // logical step t + k sits at position BLK - 1 - k.
  int32_t rev;
  int32_t acc;   // nonzero: y += result (the old y is read in the output type)
};

// Address helpers of the time direction for blocks of BLK steps (compile
// time; forward code is the plain t * D addressing).
template <bool REV, int BLK = kBlk>
struct TimeDir {
  int64_t ts;     // elements from logical step t to t + 1 (+D or -D)
  __device__ __forceinline__ int32_t blk(int32_t t) const { return REV ? t + (BLK - 1) : t; }
  __device__ __forceinline__ uint32_t pos(int32_t k) const {
    return uint32_t(REV ? (BLK - 1) - k : k);
  }
  // row index (b * L + physical step) of the block base of logical step t
  __device__ __forceinline__ int64_t row(int64_t b, int64_t L, int32_t t) const {
    return REV ? b * L + (L - 1) - blk(t) : b * L + t;
  }
};

// Launch of the 64-channel kernels for one element-type pair (input, output):
// every discretisation, flag combination, layout (nsplit 1, 2, 4) and direction.
hipError_t fwd_dispatch_bf16_f32(const FwdParams& p, int disc, int nsplit, bool has_z,
                                 bool softplus, bool summary, int64_t nblocks, hipStream_t st);
hipError_t fwd_dispatch_bf16_bf16(const FwdParams& p, int disc, int nsplit, bool has_z,
                                  bool softplus, bool summary, int64_t nblocks, hipStream_t st);
hipError_t fwd_dispatch_f32_f32(const FwdParams& p, int disc, int nsplit, bool has_z,
                                bool softplus, bool summary, int64_t nblocks, hipStream_t st);
hipError_t fwd_dispatch_f32_bf16(const FwdParams& p, int disc, int nsplit, bool has_z,
                                 bool softplus, bool summary, int64_t nblocks, hipStream_t st);

// Launch of the 32-channel kernel (two states per lane) over
// B * ndblk * grid_chunks workgroups (ndblk = ceil(D / 32)); summary = chunk
// summaries instead of outputs.
hipError_t launch_fwd_hw(const ss_desc_t& d, const FwdParams& p, bool summary, int64_t nblocks,
                         hipStream_t st);
// The same with 16-channel workgroups, one state per lane (ndblk = ceil(D / 16)).
hipError_t launch_fwd_hw1(const ss_desc_t& d, const FwdParams& p, bool summary, int64_t nblocks,
                          hipStream_t st);

}  // namespace ss
