/*
 * ss_ssd.h -- C ABI of the structured state-space duality (SSD, "Mamba-2")
 * layer forward (same library, libssscan.so).
 *
 * The operation ("A Survey of Mamba" summary, csdn, section "Mamba-2: state
 * space duality"): the selective SSM written as a semiseparable matrix,
 * y = M x with M_ji = C_j^T A_{j:i} B_i, evaluated by block decomposition --
 * diagonal blocks inside time chunks as matrix products, off-diagonal blocks
 * through the hidden state carried from chunk to chunk.  Per batch row b and
 * head h (P channels) the state is an N x P matrix and A is a per-head scalar:
 *     dt_t = softplus(dt[b,t,h] + dt_bias[h])    (or without softplus)
 *     a_t  = exp(dt_t * A[h])
 *     H_t  = a_t H_{t-1} + dt_t B_t x_t^T        B_t, C_t: (N) of group h / (H/G)
 *     y_t  = H_t^T C_t + D[h] x_t
 *
 * Conventions (as in ss_scan.h): dense row-major tensors, last index fastest:
 *   x, y : (B, L, H, P);  dt : (B, L, H);  Bm, Cm : (B, L, G, N);
 *   A, D, dt_bias : (H).  DEVICE pointers owned by the caller, 16-byte aligned.
 *   x, dt, Bm, Cm use in_dtype; y uses out_dtype; A, D, dt_bias are float32.
 *   Asynchronous on `stream`; validation before any HIP call; no allocation,
 *   no workspace (each (b, h) carries its state on chip from chunk to chunk);
 *   deterministic.  Status codes of ss_scan.h.
 * Supported: headdim P = 64, dstate N = 64, in_dtype SS_BF16, out_dtype SS_F32
 * or SS_BF16; other values return SS_ERR_UNSUPPORTED.
 */
#ifndef SS_SSD_H
#define SS_SSD_H

#include <stddef.h>
#include <stdint.h>

#include "ss_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ss_ssd_desc {
  int64_t batch;        /* B */
  int64_t seqlen;       /* L */
  int64_t nheads;       /* H */
  int64_t headdim;      /* P, channels per head */
  int64_t dstate;       /* N */
  int64_t ngroups;      /* G, divides H: heads h share B, C of group h / (H / G) */
  int32_t in_dtype;     /* ss_dtype_t of x, dt, Bm, Cm */
  int32_t out_dtype;    /* ss_dtype_t of y */
  int32_t dt_softplus;  /* nonzero: dt = softplus(dt + dt_bias); zero: dt + dt_bias */
  int32_t reserved;     /* must be 0 */
} ss_ssd_desc_t;

/*
 * SSD forward.  x, dt, A, Bm, Cm, y required; D and dt_bias optional (NULL = 0).
 * y must not alias an input.  The state starts at zero.
 */
int ss_ssd_fwd(const ss_ssd_desc_t* desc, const void* x, const void* dt, const float* A,
               const void* Bm, const void* Cm, const float* D, const float* dt_bias, void* y,
               void* stream);

/*
 * SSD forward from a given state, keeping the state after the last step, so
 * that a sequence may be processed in pieces (prefill) and continued by
 * ss_ssd_step: the recurrence above with H_0 = h0 instead of zero, and
 * h_last = H_L.
 *   h0     : (B, H, N, P) float32, the state before step 1; NULL = zero.
 *   h_last : (B, H, N, P) float32 output; NULL = not stored.  It may be the
 *            same buffer as h0 (the state is then advanced in place), and must
 *            not alias any other argument.
 * Element [b][h][n][p] of a state is H[n][p] of head h of batch row b.
 * Other arguments, validation and status codes as ss_ssd_fwd.
 */
int ss_ssd_fwd_state(const ss_ssd_desc_t* desc, const void* x, const void* dt, const float* A,
                     const void* Bm, const void* Cm, const float* D, const float* dt_bias,
                     const float* h0, void* y, float* h_last, void* stream);

/*
 * One SSD step (decoding): desc->seqlen is not read.
 *   h      : (B, H, N, P) float32, state in / out, advanced in place;
 *   x      : (B, H, P) in_dtype;  dt : (B, H) in_dtype;
 *   Bm, Cm : (B, G, N) in_dtype;  A, D, dt_bias : (H) float32 (D, dt_bias
 *            optional);  y : (B, H, P) out_dtype.
 * Computes H <- a H + dt B x^T and y = H^T C + D x with dt and a as in the
 * recurrence above.  y and h must not alias any other argument.  Device
 * pointers, 16-byte aligned; asynchronous on `stream`; no allocation;
 * deterministic.
 */
int ss_ssd_step(const ss_ssd_desc_t* desc, float* h, const void* x, const void* dt,
                const float* A, const void* Bm, const void* Cm, const float* D,
                const float* dt_bias, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SS_SSD_H */
