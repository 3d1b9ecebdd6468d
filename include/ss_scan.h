/*
 * ss_scan.h -- C ABI of the MI355X (gfx950) selective-scan (S6) library.
 *
 * The operation (pages and sections it follows):
 *   For every batch row b and channel d an independent single-input
 *   single-output state-space system with N real diagonal states ("Mamba: S4
 *   epic upgrade", hk.pswp.cn, sections "S4 intro" and "parameter-efficient data
 *   dependence": one SISO system per input channel, A diagonal with N entries
 *   per channel, A_bar = exp(delta A)).  Per time step t, with the selective,
 *   input-dependent delta_t, B_t, C_t (Gu & Dao wiki note, git.lyz.one, section
 *   "From S4 to S6": delta_t = tau(Delta + s_Delta(x_t)), here tau = softplus and
 *   Delta = delta_bias):
 *     step   dt     = softplus(delta[b,t,d] + delta_bias[d])   (or without softplus)
 *     decay  abar_n = exp(dt * A[d,n])
 *     input  bbar_n = (exp(dt*A[d,n]) - 1) / A[d,n] * B[b,t,n]   exact zero-order hold,
 *                     dt * B[b,t,n] when A[d,n] == 0 or in Euler mode
 *                     (computed as (abar - 1) / A from the rounded abar, relative error
 *                     about 2^-24 / |dt A|, where every |A| of a wave is >= 0.25; otherwise
 *                     dt (1 + x/2 + x^2/6 + x^3/24), x = dt A, wherever |x| < 0.05)
 *            (ZOH and its first-order form: "Mamba explained", hackbyte.io,
 *             discretization section; "A Survey of Mamba" summary, csdn, SSM section)
 *     state  h_n    = abar_n * h_n + bbar_n * u[b,t,d]
 *            ("A Visual Guide to Mamba" summary, wenxiaobai, The Scan Operation)
 *     output y      = sum_n C[b,t,n] h_n + D_skip[d] * u[b,t,d]     (Eq 1b, hackbyte.io)
 *     gate   out    = y * silu(z[b,t,d])            (Gu & Dao note, Mamba architecture)
 *   The discretised abar, bbar are never stored; the states are kept on chip
 *   (wenxiaobai summary, Hardware-aware Algorithm; hk.pswp.cn, IO-aware Parallel Scan).
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major, with the last index fastest:
 *       u, delta, z, y, dy, du, ddelta, dz : (B, L, D)
 *       Bm, Cm, dB, dC                     : (B, L, N)
 *       A, dA : (D, N)   D_skip, delta_bias, dD_skip, ddelta_bias : (D)
 *       h0, h_last, dh0, step state h      : (B, D, N)
 *     except that Bm and Cm may be read with a row stride (desc->bc_stride):
 *     in the Mamba block B and C are column ranges of the input projection's
 *     output (x_proj, (B, L, R + 2N): the low-rank step input, then B, then C;
 *     Gu & Dao note, Mamba architecture; "Mamba: S4 epic upgrade",
 *     parameter-efficient data dependence), and the scan reads them in place.
 *   - Pointers are DEVICE pointers owned by the caller, 16-byte aligned (Bm and
 *     Cm read with a row stride: aligned to their element size), and valid until
 *     the stream reaches the queued work.  Element types: in_dtype for u, delta,
 *     z, Bm, Cm and dy; out_dtype for y, du, ddelta and dz; float32 for everything
 *     else.  bf16 values are raw IEEE bfloat16 bit patterns (uint16).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  Kernel faults surface at the next synchronisation.
 *   - Argument validation happens before any HIP call, so every validation
 *     error can be produced without a GPU.  After it, each entry point checks
 *     that the current device is a gfx950 (SS_ERR_UNSUPPORTED otherwise; the
 *     answer is cached per device, see ss_scan_arch_supported) and launches.
 *     No exception crosses the ABI.  The library never allocates device
 *     memory: scratch comes from the caller's workspace.
 *   - NaN / Inf inputs propagate unchecked.
 *   - The forward, backward and step are deterministic (bitwise repeatable): the
 *     backward's reductions add their partial sums in a fixed order, without atomics.
 */
#ifndef SS_SCAN_H
#define SS_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SS_OK 0
#define SS_ERR_INVALID_ARG (-1)  /* NULL required pointer, size out of range, aliasing */
#define SS_ERR_UNSUPPORTED (-2)  /* dtype / discretisation / flag combination not provided,
                                    or the current device is not a gfx950 */
#define SS_ERR_WORKSPACE (-3)    /* workspace NULL or smaller than ss_scan_workspace_bytes */
#define SS_ERR_HIP (-4)          /* a HIP launch reported an error */
#define SS_ERR_SCRATCH_LIMIT (-5) /* ss_scan_fwd_noalloc: the plan needs more scratch than
                                     SS_SCAN_STATIC_SCRATCH_BYTES */

typedef enum { SS_F32 = 0, SS_BF16 = 1 } ss_dtype_t;
typedef enum { SS_ZOH = 0, SS_EULER = 1 } ss_disc_t;

/* Problem description.  1 <= dstate <= 16; batch, seqlen, dim >= 1. */
typedef struct ss_desc {
  int64_t batch;          /* B */
  int64_t seqlen;         /* L (ignored by ss_scan_step) */
  int64_t dim;            /* D, channels */
  int64_t dstate;         /* N, states per channel */
  int32_t in_dtype;       /* ss_dtype_t of u, delta, z, Bm, Cm, dy */
  int32_t out_dtype;      /* ss_dtype_t of y (fwd, step) and of du, ddelta, dz (bwd; must be SS_F32) */
  int32_t disc;           /* ss_disc_t: exact zero-order hold or Euler input coefficient */
  int32_t delta_softplus; /* nonzero: dt = softplus(delta + delta_bias); zero: dt = delta + delta_bias */
  /* Elements from one (b, t) row of Bm and Cm to the next ((b) row for the
   * step); 0 means dense (dstate).  Otherwise dstate <= bc_stride <= 2^20;
   * Bm and Cm then need only be aligned to their element size (the forward and
   * backward copy the rows into their workspace first, the step reads them
   * element by element).  The complex-A entry points take 0 only.  The
   * gradients dB, dC stay dense (B, L, N). */
  int64_t bc_stride;
} ss_desc_t;

/* Operations for ss_scan_workspace_bytes. */
#define SS_OP_FWD 0
#define SS_OP_BWD 1
#define SS_OP_FWD_COMPLEX 2   /* ss_scan_fwd_complex_ws */

/*
 * Bytes of device workspace that ss_scan_fwd (op = SS_OP_FWD), ss_scan_bwd
 * (op = SS_OP_BWD) or ss_scan_fwd_complex_ws (op = SS_OP_FWD_COMPLEX) needs for
 * this description (0 when none).  The size depends
 * only on the description (and the SS_SCAN_CHUNK tuning variable, if set).
 * Returns 0 for an invalid description.  Workspace contents are scratch: they
 * need not be initialised and are clobbered.
 */
size_t ss_scan_workspace_bytes(const ss_desc_t* desc, int op);

/*
 * Forward selective scan.
 *   u, delta, Bm, Cm, A, y     required.
 *   D_skip, delta_bias, z, h0  optional (NULL = zero skip, zero bias, no gate,
 *                              zero initial state).
 *   h_last                     optional output: the state after the last step;
 *                              must not alias h0.
 *   workspace, ws_bytes        at least ss_scan_workspace_bytes(desc, SS_OP_FWD).
 * Long or narrow problems are split into time chunks whose start states are
 * found by a scan over per-chunk (decay, end state) summaries under
 * (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2) ("A Visual Guide to Mamba" summary,
 * The Scan Operation: compute in segments and combine them associatively).
 */
int ss_scan_fwd(const ss_desc_t* desc,
                const void* u, const void* delta, const float* A,
                const void* Bm, const void* Cm,
                const float* D_skip, const float* delta_bias, const void* z,
                const float* h0,
                void* y, float* h_last,
                void* workspace, size_t ws_bytes, void* stream);

/* Bytes of the static scratch array ss_scan_fwd_noalloc uses on each GPU. */
#define SS_SCAN_STATIC_SCRATCH_BYTES (32u << 20)

/*
 * ss_scan_fwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The scratch a plan needs (chunk start states and
 * step sums, padded B/C rows; ss_scan_workspace_bytes(desc, SS_OP_FWD) bytes,
 * at most about 9 MB for chunk carries at any shape) comes from a static
 * device array of SS_SCAN_STATIC_SCRATCH_BYTES (32 MiB) that each GPU the
 * library runs on holds from load until the process ends.  The call makes no
 * allocation of any kind.
 *   Arguments, results and other status codes: exactly ss_scan_fwd (the same
 *   kernels and plan, so the output is bitwise that of ss_scan_fwd).
 *   Returns SS_ERR_SCRATCH_LIMIT, before any HIP call, when the plan needs
 *   more than SS_SCAN_STATIC_SCRATCH_BYTES (e.g. dstate < 16 or a nonzero
 *   bc_stride with a very long batch * seqlen, whose padded rows scale with
 *   it); use ss_scan_fwd then.
 * All calls on one GPU share its array, which keeps the last call's contents
 * (every value a call reads from it, that call has written first): calls that
 * overlap on one GPU (different streams, or threads without ordering) race.
 * Serialise them on one stream or with events.
 */
int ss_scan_fwd_noalloc(const ss_desc_t* desc,
                        const void* u, const void* delta, const float* A,
                        const void* Bm, const void* Cm,
                        const float* D_skip, const float* delta_bias, const void* z,
                        const float* h0,
                        void* y, float* h_last, void* stream);

/* Time directions of ss_scan_fwd_dir. */
#define SS_DIR_FORWARD 0
#define SS_DIR_REVERSE 1

/*
 * Forward selective scan in either time direction, optionally added to y.
 * Scan modes: a scan that runs only forward in time sees no later tokens,
 * which suits text but not images or video; flat scan modes therefore also
 * scan the token sequence the other way and combine the results ("A Survey of
 * Mamba" summary, section on scan modes).
 *   direction = SS_DIR_FORWARD: exactly ss_scan_fwd.
 *   direction = SS_DIR_REVERSE: the same system run from t = L-1 down to 0,
 *       h_t = abar_t h_{t+1} + bbar_t u_t,  y_t = C_t h_t + D_skip u_t (gated),
 *       i.e. ss_scan_fwd on the time-reversed sequence, reversed back.  h0 is
 *       the state entering at t = L-1, h_last the state after t = 0.
 *   accumulate != 0: y += result (y must hold valid values of out_dtype;
 *       the addition is done in fp32).  A bidirectional scan is a forward call
 *       followed by a reverse call with accumulate = 1 (each direction may use
 *       its own A, D_skip, delta_bias).
 * Other arguments, workspace size and status codes as ss_scan_fwd.
 * Returns SS_ERR_INVALID_ARG for any other direction.
 */
int ss_scan_fwd_dir(const ss_desc_t* desc, int direction, int accumulate,
                    const void* u, const void* delta, const float* A,
                    const void* Bm, const void* Cm,
                    const float* D_skip, const float* delta_bias, const void* z,
                    const float* h0,
                    void* y, float* h_last,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * Forward selective scan with a complex diagonal A (the S4D-Lin kind of
 * system; "A Survey of Mamba" summary, HiPPO-based memory initialisation:
 * complex and real diagonal initialisations; "Mamba: S4 epic upgrade",
 * ablation on A: real and complex decay compared).  Per channel and complex
 * state n:
 *     abar  = exp(dt a)                   a = A[d,n] complex
 *     bcoef = (abar - 1) / a              exact ZOH (dt when a == 0 or Euler)
 *     h_n   = abar h_n + bcoef B_n u      B_n, C_n complex per (b, t)
 *     y     = 2 Re(sum_n C_n h_n) + D_skip u      (each state stands for itself
 *                                                  and its conjugate)
 *     out   = y * silu(z)
 * Complex tensors are stored as (re, im) pairs in a last axis of 2:
 *     A : (D, N, 2) float32;  Bm, Cm : (B, L, N, 2) in in_dtype;
 *     h0, h_last : (B, D, N, 2) float32.
 * Everything else as ss_scan_fwd.  dstate = N complex states (1..16).  No
 * workspace: one workgroup walks the whole sequence of its 32 channels, so a
 * long sequence with few channels runs on few workgroups; use
 * ss_scan_fwd_complex_ws there.
 */
int ss_scan_fwd_complex(const ss_desc_t* desc,
                        const void* u, const void* delta, const float* A,
                        const void* Bm, const void* Cm,
                        const float* D_skip, const float* delta_bias, const void* z,
                        const float* h0,
                        void* y, float* h_last, void* stream);

/*
 * ss_scan_fwd_complex with a workspace of ss_scan_workspace_bytes(desc,
 * SS_OP_FWD_COMPLEX) bytes (256-byte aligned), which lets long, narrow
 * problems be cut into time chunks: a summary pass gives each chunk's end state
 * from a zero start and its sum of step sizes, an in-order walk over the
 * chunks turns them into start states (the chunk maps h -> abar_c h + s_c,
 * abar_c = exp(a sum dt), composed associatively: "A Visual Guide to Mamba"
 * summary, The Scan Operation), and the output pass runs every chunk from its
 * true start.  The step sums are kept in fp64, since a chunk's rotation angle
 * Im(a) sum dt can reach hundreds of radians.  With workspace == NULL and
 * ws_bytes == 0 this is exactly ss_scan_fwd_complex (one pass).  Returns
 * SS_ERR_WORKSPACE when a workspace is given but is too small or misaligned.
 * Other arguments and status codes as ss_scan_fwd_complex.
 */
int ss_scan_fwd_complex_ws(const ss_desc_t* desc,
                           const void* u, const void* delta, const float* A,
                           const void* Bm, const void* Cm,
                           const float* D_skip, const float* delta_bias, const void* z,
                           const float* h0,
                           void* y, float* h_last,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * One recurrent step with complex diagonal A (decoding), the single-token form
 * of ss_scan_fwd_complex: desc->seqlen is not read; desc->dstate = N <= 16
 * complex states.
 *   h      : (B, D, N, 2) float32 (re, im), state in / out, advanced in place
 *   u, delta, z : (B, D) in_dtype (z optional);  A : (D, N, 2) float32
 *   Bm, Cm : (B, N, 2) in_dtype;  D_skip, delta_bias : (D) float32, optional
 *   y      : (B, D) out_dtype, 2 Re(sum_n C_n h_n) + D u, gated by silu(z)
 * The discretisation and its guarded series near dt A = 0 are those of
 * ss_scan_fwd_complex, so a step continues a scan's h_last.  y must not alias
 * an input.  Device pointers, 16-byte aligned; asynchronous on `stream`; no
 * allocation; deterministic.
 */
int ss_scan_step_complex(const ss_desc_t* desc, float* h, const void* u, const void* delta,
                         const float* A, const void* Bm, const void* Cm, const float* D_skip,
                         const float* delta_bias, const void* z, void* y, void* stream);

/*
 * Backward of ss_scan_fwd with recomputation: the states are rebuilt from the
 * inputs (chunk start states in the workspace, the rest on chip), never read
 * from a stored (B,L,D,N) tensor ("A Visual Guide to Mamba" summary,
 * Hardware-aware Algorithm: recomputation; "A Survey of Mamba" summary,
 * hardware-aware computation).
 *   Inputs: as ss_scan_fwd (h0 optional) plus dy = d(loss)/d(out), in_dtype.
 *   Outputs, all overwritten (never accumulated into):
 *     du, ddelta (w.r.t. the raw delta input, through softplus)   required
 *     dA, dB, dC                                                    required
 *     dD_skip (required iff D_skip given), ddelta_bias (required iff
 *     delta_bias given), dz (required iff z given), dh0 (optional).
 *   out_dtype must be SS_F32.  dA, dB, dC, dD_skip, ddelta_bias are reduced in
 *   fp32 in a fixed order (deterministic).
 */
int ss_scan_bwd(const ss_desc_t* desc,
                const void* u, const void* delta, const float* A,
                const void* Bm, const void* Cm,
                const float* D_skip, const float* delta_bias, const void* z,
                const float* h0, const void* dy,
                void* du, void* ddelta, float* dA, float* dB, float* dC,
                float* dD_skip, float* ddelta_bias, void* dz, float* dh0,
                void* workspace, size_t ws_bytes, void* stream);

/*
 * One recurrent (inference) step for every (b, d): the state h (B,D,N) fp32 is
 * read and overwritten in place; u, delta, z, y are (B,D); Bm, Cm are (B,N)
 * (rows desc->bc_stride elements apart when it is nonzero).
 * desc->seqlen is ignored.  Optional pointers as in ss_scan_fwd.  y must not
 * alias h, u, delta, Bm, Cm or z (SS_ERR_INVALID_ARG): it is written while other
 * lanes still read them.  batch * dim <= 2^33.  The state is O(1) per token,
 * unlike a growing attention cache ("Mamba explained", hackbyte.io,
 * quadratic-bottleneck section).
 */
int ss_scan_step(const ss_desc_t* desc, float* h,
                 const void* u, const void* delta, const float* A,
                 const void* Bm, const void* Cm,
                 const float* D_skip, const float* delta_bias, const void* z,
                 void* y, void* stream);

/*
 * Whether the library's kernels run on a device of this architecture:
 * arch_name is a HIP gcnArchName such as "gfx950:sramecc+:xnack-".  Returns
 * SS_OK for "gfx950" (with or without ":feature" suffixes), SS_ERR_UNSUPPORTED
 * for any other name, SS_ERR_INVALID_ARG for NULL.  Pure host function (no
 * HIP call); every launching entry point applies it to the current device
 * after its argument checks.
 */
int ss_scan_arch_supported(const char* arch_name);

/* Static, human-readable text for a status code. */
const char* ss_scan_strerror(int status);

/* Library ABI version (major * 10000 + minor * 100 + patch).  2.0 added the
 * trailing bc_stride field of ss_desc_t (the struct grew by 8 bytes). */
int ss_scan_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SS_SCAN_H */
