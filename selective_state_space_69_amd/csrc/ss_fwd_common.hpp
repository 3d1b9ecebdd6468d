// Parameters shared by the two forward scan kernels (ss_fwd.hip: one wave per
// 64 channels and a slice of the states; ss_fwd_hw.hip: 32 channels per wave
// and two states per lane) and by their launchers.
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
};

// Launch of the 32-channel kernel over B * ndblk * grid_chunks workgroups
// (ndblk = ceil(D / 32)); summary = chunk summaries instead of outputs.
hipError_t launch_fwd_hw(const ss_desc_t& d, const FwdParams& p, bool summary, int64_t nblocks,
                         hipStream_t st);

}  // namespace ss
