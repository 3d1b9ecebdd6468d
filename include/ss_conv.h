/*
 * ss_conv.h -- C ABI of the causal depthwise Conv1d + SiLU that produces the
 * selective scan's input u (same library, libssscan.so).
 *
 * The operation: in a Mamba block the expanded input passes a convolution along
 * time and a SiLU before the selective SSM (Gu & Dao wiki note, git.lyz.one,
 * section "Mamba architecture": Linear(expand) -> Conv1d -> SiLU -> SSM(S6);
 * "A Visual Guide to Mamba" summary, wenxiaobai, section "Mamba block": the
 * convolution keeps tokens from being processed independently).  One filter per
 * channel, causal, width K:
 *     pre[b,t,d] = bias[d] + sum_{k=0}^{K-1} w[d,k] * x[b, t-K+1+k, d]   (x = 0 before t = 0)
 *     u[b,t,d]   = pre * sigmoid(pre)      (silu = 1)   or   pre   (silu = 0)
 *
 * Conventions (as in ss_scan.h):
 *   - Dense row-major tensors, last index fastest: x, u, du, dx : (B, L, D);
 *     w, dw : (D, K); bias, dbias : (D); decode state : (B, D, K-1), oldest first.
 *   - DEVICE pointers owned by the caller, 16-byte aligned, valid until the stream
 *     reaches the work.  x and the decode-step x use in_dtype; u uses out_dtype;
 *     du, dx, w, dw, bias, dbias and the decode state are float32.  bf16 values
 *     are raw bfloat16 bit patterns (uint16).
 *   - Asynchronous on `stream` (a hipStream_t; NULL = the null stream).  All
 *     validation happens before any HIP call.  The library never allocates.
 *   - Status codes are those of ss_scan.h (SS_OK, SS_ERR_*).  All three entry
 *     points are deterministic (the backward reduces dw and dbias in a fixed order).
 */
#ifndef SS_CONV_H
#define SS_CONV_H

#include <stddef.h>
#include <stdint.h>

#include "ss_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Problem description.  batch, seqlen, dim >= 1; 1 <= width <= 4. */
typedef struct ss_conv_desc {
  int64_t batch;      /* B */
  int64_t seqlen;     /* L (ignored by ss_conv1d_step) */
  int64_t dim;        /* D, channels */
  int32_t width;      /* K, taps per channel */
  int32_t in_dtype;   /* ss_dtype_t of x */
  int32_t out_dtype;  /* ss_dtype_t of u (ss_conv1d_fwd, ss_conv1d_step) */
  int32_t silu;       /* nonzero: u = silu(pre); zero: u = pre */
} ss_conv_desc_t;

/*
 * Forward: u = silu(causal depthwise conv(x) + bias).
 *   x, w, u required; bias optional (NULL = 0).  u must not alias x.
 */
int ss_conv1d_fwd(const ss_conv_desc_t* desc, const void* x, const float* w, const float* bias,
                  void* u, void* stream);

/* Bytes of device workspace ss_conv1d_bwd needs (per-segment dw / dbias partials). */
size_t ss_conv1d_workspace_bytes(const ss_conv_desc_t* desc);

/*
 * Backward of ss_conv1d_fwd.  du = d(loss)/d(u), float32.  Outputs, all
 * overwritten: dx (float32, required), dw (required), dbias (required iff bias
 * given).  dx must not alias x or du.
 *   workspace, ws_bytes : at least ss_conv1d_workspace_bytes(desc).
 */
int ss_conv1d_bwd(const ss_conv_desc_t* desc, const void* x, const float* w, const float* bias,
                  const float* du, float* dx, float* dw, float* dbias,
                  void* workspace, size_t ws_bytes, void* stream);

/*
 * One decode step for every (b, d): the window is [state (K-1 values), x];
 * u = silu(bias + w . window); the state then drops its oldest value and
 * appends x (read and overwritten in place; NULL allowed only when K == 1).
 * x, u : (B, D).  desc->seqlen is ignored.
 */
int ss_conv1d_step(const ss_conv_desc_t* desc, float* state, const void* x, const float* w,
                   const float* bias, void* u, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SS_CONV_H */
