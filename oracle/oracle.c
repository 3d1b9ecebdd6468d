/*
 * oracle.c -- plain, slow, sequential fp64 reference of the selective scan (S6).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header, table or constant with the HIP library.
 *
 * Every routine takes its inputs as fp64 arrays (the caller converts the exact
 * bf16 / fp32 bits the GPU receives) and computes in fp64, one independent
 * single-input single-output channel (b, d) at a time, stepping t = 0 .. L-1.
 *
 * Sources (pages, sections):
 *  - "Mamba explained" translation (hackbyte.io), section on the state: Eq 1a
 *    h'(t) = A h(t) + B x(t) and Eq 1b y(t) = C h(t) + D x(t); section on
 *    discretization: the first-order (Euler) step h_{t+1} ~ (I + dA) h_t + (dB) x_t.
 *  - "Mamba: S4 epic upgrade" (hk.pswp.cn), sections "TL;DR" (shapes u, delta:
 *    (B,L,D); B, C: (B,L,N); A: (D,N)), "S4 intro" (zero-order hold, one SISO
 *    system per input channel) and "parameter-efficient data dependence"
 *    (A_bar = exp(delta A), A diagonal and real).
 *  - Gu & Dao wiki note (git.lyz.one), section "From S4 to S6": B_t = s_B(x_t),
 *    C_t = s_C(x_t), delta_t = tau(Delta + s_Delta(x_t)); section "Mamba
 *    architecture": SiLU gating branch.
 *  - "A Visual Guide to Mamba" summary (wenxiaobai), section "The Scan Operation":
 *    each state is the previous state times A plus the current input times B;
 *    section "Hardware-aware Algorithm": states are recomputed for the backward.
 *  - "A Survey of Mamba" summary (csdn), sections "SSM" (ZOH discretised form,
 *    D x(t) is the skip connection) and "Selection" (Broadcast_D of delta terms).
 *
 * Readings taken where the pages are silent or garbled:
 *  - tau_Delta is softplus; the per-channel parameter Delta enters as a bias added
 *    to the raw per-token delta before softplus.
 *  - exact ZOH input matrix: B_bar = (exp(dA) - 1) / A * B, with the limit d*B at
 *    A = 0.  "Euler" switches only B_bar to d*B; A_bar stays exp(dA).
 *  - h_t = A_bar_t h_{t-1} + B_bar_t u_t, y_t uses h_t (current input included).
 *  - initial state 0 unless h0 is given; out = y * silu(z) with the D skip inside
 *    the gate.
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_ZOH 0
#define ORACLE_EULER 1

/* softplus(x) = log(1 + e^x), evaluated without overflow. */
double oracle_softplus(double x) {
  if (x > 0.0) return x + log1p(exp(-x));
  return log1p(exp(x));
}

/* logistic sigma(x) = 1 / (1 + e^-x) */
static double sigmoid(double x) {
  if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
  double e = exp(x);
  return e / (1.0 + e);
}

/* Discretise one (step dt, diagonal entry a) pair.
 * abar = exp(dt * a) (ZOH state matrix; also used in Euler mode).
 * bcoef = (exp(dt*a) - 1) / a  (exact ZOH), limit dt at a == 0;  dt for Euler.
 * The input coefficient multiplies B and u: B_bar u = bcoef * B * u. */
void oracle_discretize(double dt, double a, int disc, double* abar, double* bcoef) {
  *abar = exp(dt * a);
  if (disc == ORACLE_EULER || a == 0.0) {
    *bcoef = dt;
  } else {
    *bcoef = expm1(dt * a) / a;
  }
}

/* d(bcoef)/d(a) for the exact ZOH coefficient.  f(a) = expm1(dt a)/a, so
 * f'(a) = (dt a e^{dt a} - expm1(dt a)) / a^2.  Near dt*a = 0 the closed form
 * cancels, so the Taylor series of f'(a) = dt^2 sum_j (j+1) (dt a)^j / (j+2)!
 * is summed instead (terms to j = 6; the first dropped term is < 1e-17 relative
 * for |dt a| < 1e-2). */
static double zoh_dbcoef_da(double dt, double a) {
  double x = dt * a;
  if (fabs(x) < 1e-2) {
    double s = 0.0, p = 1.0, fact = 2.0; /* (j+2)! for j = 0 */
    for (int j = 0; j <= 6; ++j) {
      s += (double)(j + 1) * p / fact;
      p *= x;
      fact *= (double)(j + 3);
    }
    return dt * dt * s;
  }
  return (x * exp(x) - expm1(x)) / (a * a);
}

static double step_size(double delta, double bias, int softplus) {
  double x = delta + bias;
  return softplus ? oracle_softplus(x) : x;
}

/*
 * Forward scan.  Shapes (row-major, contiguous):
 *   u, delta, z, out : (Bt, L, D)      A : (D, N)        Bm, Cm : (Bt, L, N)
 *   Dskip, bias : (D) or NULL           h0, h_last : (Bt, D, N) or NULL
 * out receives y * silu(z) when z != NULL, else y.
 * nthreads > 1 splits the independent channels over OpenMP threads.
 */
int oracle_fwd(int64_t Bt, int64_t L, int64_t D, int64_t N, int disc, int softplus,
               const double* u, const double* delta, const double* A,
               const double* Bm, const double* Cm, const double* Dskip,
               const double* bias, const double* z, const double* h0,
               double* out, double* h_last, int nthreads) {
  if (Bt < 0 || L < 0 || D < 0 || N < 1 || N > 64) return -1;
  int64_t nch = Bt * D;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
#endif
  for (int64_t ch = 0; ch < nch; ++ch) {
    int64_t b = ch / D, d = ch % D;
    double h[64];
    for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
    double dsk = Dskip ? Dskip[d] : 0.0;
    double bi = bias ? bias[d] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
      int64_t i = (b * L + t) * D + d;
      double dt = step_size(delta[i], bi, softplus);
      double ut = u[i];
      double y = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        double abar, bcoef;
        oracle_discretize(dt, A[d * N + n], disc, &abar, &bcoef);
        int64_t j = (b * L + t) * N + n;
        h[n] = abar * h[n] + bcoef * Bm[j] * ut;   /* recurrence */
        y += Cm[j] * h[n];                          /* output contraction */
      }
      y += dsk * ut;                                /* skip connection D u */
      if (z) y *= z[i] * sigmoid(z[i]);             /* silu(z) gate */
      out[i] = y;
    }
    if (h_last)
      for (int64_t n = 0; n < N; ++n) h_last[(b * D + d) * N + n] = h[n];
  }
  (void)nthreads;
  return 0;
}

/*
 * Backward of oracle_fwd by the chain rule, with every intermediate state of a
 * channel kept (the GPU recomputes them instead).  g = d(loss)/d(out), (Bt,L,D).
 * Outputs (all overwritten, never accumulated into):
 *   du, ddelta (w.r.t. the raw delta, through softplus), dz : (Bt,L,D)
 *   dA : (D,N)   dB, dC : (Bt,L,N)   dDskip, dbias : (D)   dh0 : (Bt,D,N)
 * Any output pointer may be NULL (dz is ignored when z is NULL).
 */
int oracle_bwd(int64_t Bt, int64_t L, int64_t D, int64_t N, int disc, int softplus,
               const double* u, const double* delta, const double* A,
               const double* Bm, const double* Cm, const double* Dskip,
               const double* bias, const double* z, const double* h0,
               const double* g,
               double* du, double* ddelta, double* dA, double* dB, double* dC,
               double* dDskip, double* dbias, double* dz, double* dh0) {
  if (Bt < 0 || L < 0 || D < 0 || N < 1 || N > 64) return -1;
  double* hs = (double*)malloc(sizeof(double) * (size_t)(L + 1) * (size_t)N);
  double* dts = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  double* gys = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  if (!hs || !dts || !gys) { free(hs); free(dts); free(gys); return -2; }
  if (dA) memset(dA, 0, sizeof(double) * (size_t)(D * N));
  if (dB) memset(dB, 0, sizeof(double) * (size_t)(Bt * L * N));
  if (dC) memset(dC, 0, sizeof(double) * (size_t)(Bt * L * N));
  if (dDskip) memset(dDskip, 0, sizeof(double) * (size_t)D);
  if (dbias) memset(dbias, 0, sizeof(double) * (size_t)D);

  for (int64_t b = 0; b < Bt; ++b) {
    for (int64_t d = 0; d < D; ++d) {
      double dsk = Dskip ? Dskip[d] : 0.0;
      double bi = bias ? bias[d] : 0.0;
      /* forward, keeping h_{-1} .. h_{L-1} in hs[0 .. L] */
      for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        int64_t i = (b * L + t) * D + d;
        double dt = step_size(delta[i], bi, softplus);
        dts[t] = dt;
        double y = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          double abar, bcoef;
          oracle_discretize(dt, A[d * N + n], disc, &abar, &bcoef);
          int64_t j = (b * L + t) * N + n;
          double hn = abar * hs[t * N + n] + bcoef * Bm[j] * u[i];
          hs[(t + 1) * N + n] = hn;
          y += Cm[j] * hn;
        }
        y += dsk * u[i];
        double gy = g[i];
        if (z) {
          double s = sigmoid(z[i]);
          if (dz) dz[i] = g[i] * y * s * (1.0 + z[i] * (1.0 - s));
          gy = g[i] * z[i] * s;
        }
        gys[t] = gy;   /* d(loss)/dy_t */
        if (dDskip) dDskip[d] += gy * u[i];
      }
      /* reverse sweep; mu[n] = A_bar_{t+1} * lambda_{t+1} carried backwards */
      double mu[64];
      for (int64_t n = 0; n < N; ++n) mu[n] = 0.0;
      for (int64_t t = L - 1; t >= 0; --t) {
        int64_t i = (b * L + t) * D + d;
        double dt = dts[t], gy = gys[t], ut = u[i];
        double ddt = 0.0, dut = gy * dsk;
        for (int64_t n = 0; n < N; ++n) {
          double a = A[d * N + n];
          double abar, bcoef;
          oracle_discretize(dt, a, disc, &abar, &bcoef);
          int64_t j = (b * L + t) * N + n;
          double lam = gy * Cm[j] + mu[n];          /* d(loss)/dh_t */
          double hprev = hs[t * N + n];
          if (dC) dC[j] += gy * hs[(t + 1) * N + n];
          double dabar = lam * hprev;
          double dbb = lam * ut;                    /* d(loss)/d(B_bar) */
          dut += lam * bcoef * Bm[j];
          if (dB) dB[j] += dbb * bcoef;
          /* d(bcoef)/d(dt) and d(bcoef)/d(a) */
          double dc_ddt, dc_da;
          if (disc == ORACLE_EULER) { dc_ddt = 1.0; dc_da = 0.0; }
          else if (a == 0.0) { dc_ddt = 1.0; dc_da = 0.5 * dt * dt; }
          else { dc_ddt = abar; dc_da = zoh_dbcoef_da(dt, a); }
          ddt += dabar * abar * a + dbb * Bm[j] * dc_ddt;
          if (dA) dA[d * N + n] += dabar * abar * dt + dbb * Bm[j] * dc_da;
          mu[n] = abar * lam;
        }
        if (du) du[i] = dut;
        double dx = softplus ? ddt * sigmoid(delta[i] + bi) : ddt;
        if (ddelta) ddelta[i] = dx;
        if (dbias) dbias[d] += dx;
      }
      if (dh0)
        for (int64_t n = 0; n < N; ++n) dh0[(b * D + d) * N + n] = mu[n];
    }
  }
  free(hs); free(dts); free(gys);
  return 0;
}

/*
 * One recurrent step (inference mode): h (Bt,D,N) is read and overwritten;
 * u, delta, z, out are (Bt,D); Bm, Cm are (Bt,N).
 */
int oracle_step(int64_t Bt, int64_t D, int64_t N, int disc, int softplus,
                double* h, const double* u, const double* delta, const double* A,
                const double* Bm, const double* Cm, const double* Dskip,
                const double* bias, const double* z, double* out) {
  if (Bt < 0 || D < 0 || N < 1 || N > 64) return -1;
  for (int64_t b = 0; b < Bt; ++b) {
    for (int64_t d = 0; d < D; ++d) {
      int64_t i = b * D + d;
      double dt = step_size(delta[i], bias ? bias[d] : 0.0, softplus);
      double y = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        double abar, bcoef;
        oracle_discretize(dt, A[d * N + n], disc, &abar, &bcoef);
        double* hn = &h[i * N + n];
        *hn = abar * *hn + bcoef * Bm[b * N + n] * u[i];
        y += Cm[b * N + n] * *hn;
      }
      y += (Dskip ? Dskip[d] : 0.0) * u[i];
      if (z) y *= z[i] * sigmoid(z[i]);
      out[i] = y;
    }
  }
  return 0;
}

/*
 * Causal depthwise convolution of width K along time, then SiLU: the step that
 * turns the expanded input x into the scan's u (Gu & Dao wiki note, "Mamba
 * architecture": Linear(expand) -> Conv1d -> SiLU -> SSM; "A Visual Guide to
 * Mamba" summary, "Mamba block": a convolution before the selective SSM so
 * that tokens are not processed independently).
 * Readings: one filter per channel (depthwise: the scan is per channel), causal
 * (output t sees inputs t-K+1 .. t, zero before t = 0), width 1 <= K <= 4, an
 * optional per-channel bias; silu = 0 leaves the activation out.
 *   pre[b,t,d] = bias[d] + sum_k w[d,k] x[b, t-K+1+k, d]
 *   u[b,t,d]   = pre * sigma(pre)   (or pre)
 * x, u: (Bt, L, D); w: (D, K); bias: (D) or NULL.
 */
static double conv_pre(const double* x, const double* w, const double* bias, int64_t L, int64_t D,
                       int64_t K, int64_t b, int64_t t, int64_t d) {
  double s = bias ? bias[d] : 0.0;
  for (int64_t k = 0; k < K; ++k) {
    int64_t tt = t - K + 1 + k;
    if (tt >= 0) s += w[d * K + k] * x[(b * L + tt) * D + d];
  }
  return s;
}

int oracle_conv1d_fwd(int64_t Bt, int64_t L, int64_t D, int64_t K, int silu, const double* x,
                      const double* w, const double* bias, double* u) {
  if (Bt < 0 || L < 0 || D < 0 || K < 1) return -1;
  for (int64_t b = 0; b < Bt; ++b)
    for (int64_t t = 0; t < L; ++t)
      for (int64_t d = 0; d < D; ++d) {
        double p = conv_pre(x, w, bias, L, D, K, b, t, d);
        u[(b * L + t) * D + d] = silu ? p * sigmoid(p) : p;
      }
  return 0;
}

/*
 * Backward of the above by the chain rule.  Given g = dLoss/du:
 *   gp[b,t,d] = g * d silu(p)/dp = g * s (1 + p (1 - s)),  s = sigma(p)  (or g)
 *   dx[b,t,d] = sum_k w[d,k] gp[b, t+K-1-k, d]   (terms past L - 1 are 0)
 *   dw[d,k]   = sum_{b,t} gp[b,t,d] x[b, t-K+1+k, d]
 *   dbias[d]  = sum_{b,t} gp[b,t,d]
 * dw and dbias are written (not accumulated into); dbias may be NULL.
 */
int oracle_conv1d_bwd(int64_t Bt, int64_t L, int64_t D, int64_t K, int silu, const double* x,
                      const double* w, const double* bias, const double* g, double* dx,
                      double* dw, double* dbias) {
  if (Bt < 0 || L < 0 || D < 0 || K < 1) return -1;
  double* gp = (double*)malloc(sizeof(double) * (size_t)(Bt * L * D > 0 ? Bt * L * D : 1));
  if (!gp) return -2;
  for (int64_t b = 0; b < Bt; ++b)
    for (int64_t t = 0; t < L; ++t)
      for (int64_t d = 0; d < D; ++d) {
        int64_t i = (b * L + t) * D + d;
        double p = conv_pre(x, w, bias, L, D, K, b, t, d);
        double s = sigmoid(p);
        gp[i] = silu ? g[i] * s * (1.0 + p * (1.0 - s)) : g[i];
      }
  for (int64_t d = 0; d < D; ++d) {
    for (int64_t k = 0; k < K; ++k) dw[d * K + k] = 0.0;
    if (dbias) dbias[d] = 0.0;
  }
  for (int64_t b = 0; b < Bt; ++b)
    for (int64_t t = 0; t < L; ++t)
      for (int64_t d = 0; d < D; ++d) {
        int64_t i = (b * L + t) * D + d;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
          int64_t to = t + K - 1 - k;     /* output step that read x[t] through tap k */
          if (to < L) acc += w[d * K + k] * gp[(b * L + to) * D + d];
          int64_t ti = t - K + 1 + k;     /* input step that tap k of output t read */
          if (ti >= 0) dw[d * K + k] += gp[i] * x[(b * L + ti) * D + d];
        }
        dx[i] = acc;
        if (dbias) dbias[d] += gp[i];
      }
  free(gp);
  return 0;
}

/*
 * One decode step of the convolution: state (Bt, D, K-1) holds the last K-1
 * inputs of each channel, oldest first; x, u: (Bt, D).  The window is
 * [state, x]; afterwards the state holds its last K-1 entries.
 */
int oracle_conv1d_step(int64_t Bt, int64_t D, int64_t K, int silu, double* state,
                       const double* x, const double* w, const double* bias, double* u) {
  if (Bt < 0 || D < 0 || K < 1) return -1;
  for (int64_t b = 0; b < Bt; ++b)
    for (int64_t d = 0; d < D; ++d) {
      double* st = state + (b * D + d) * (K - 1);
      double p = bias ? bias[d] : 0.0;
      for (int64_t k = 0; k < K - 1; ++k) p += w[d * K + k] * st[k];
      p += w[d * K + K - 1] * x[b * D + d];
      for (int64_t k = 0; k + 1 < K - 1; ++k) st[k] = st[k + 1];
      if (K > 1) st[K - 2] = x[b * D + d];
      u[b * D + d] = silu ? p * sigmoid(p) : p;
    }
  return 0;
}

/*
 * Structured state-space duality (SSD) layer, sequential reference ("A Survey
 * of Mamba" summary, section "Mamba-2: state space duality": the SSM as a
 * semiseparable matrix M_ji = C_j^T A_{j:i} B_i, computed by block
 * decomposition with diagonal blocks inside chunks and off-diagonal blocks
 * through hidden states).  Per batch row b and head h the state is an N x P
 * matrix and A_t is a scalar (times the identity), shared by the head's P
 * channels; B and C are shared by the heads of a group.
 * Readings: A_h is a per-head scalar (it is what makes M a matrix shared by the
 * head's channels); dt_t = softplus(dt_raw[b,t,h] + dt_bias[h]) as in the
 * selective scan; the input coefficient is dt (B_bar = dt B); D_h is a per-head
 * skip; no gate (the gate is applied outside the layer).
 *   a_t  = exp(dt_t A_h)
 *   H_t  = a_t H_{t-1} + dt_t B_t x_t^T              (N x P)
 *   y_t  = H_t^T C_t + D_h x_t                       (P)
 * x, y: (Bt, L, Hh, P); dt: (Bt, L, Hh); A, D, dt_bias: (Hh);
 * Bm, Cm: (Bt, L, G, N), head h uses group h / (Hh / G).
 * h0 (state before the first step, zero when NULL) and h_last (state after the
 * last step, written when not NULL): (Bt, Hh, N, P).
 */
int oracle_ssd_fwd(int64_t Bt, int64_t L, int64_t Hh, int64_t P, int64_t N, int64_t G,
                   int softplus, const double* x, const double* dt_raw, const double* A,
                   const double* Bm, const double* Cm, const double* Dh, const double* dt_bias,
                   const double* h0, double* y, double* h_last, int nthreads) {
  if (Bt < 0 || L < 0 || Hh < 1 || P < 1 || N < 1 || G < 1 || Hh % G) return -1;
  const int64_t hpg = Hh / G;
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
  for (int64_t b = 0; b < Bt; ++b) {
    for (int64_t h = 0; h < Hh; ++h) {
      double* H = (double*)calloc((size_t)(N * P), sizeof(double));
      if (h0)
        for (int64_t k = 0; k < N * P; ++k) H[k] = h0[(b * Hh + h) * N * P + k];
      const int64_t g = h / hpg;
      for (int64_t t = 0; t < L; ++t) {
        double dt = step_size(dt_raw[(b * L + t) * Hh + h], dt_bias ? dt_bias[h] : 0.0, softplus);
        double a = exp(dt * A[h]);
        const double* Bt_ = Bm + ((b * L + t) * G + g) * N;
        const double* Ct = Cm + ((b * L + t) * G + g) * N;
        const double* xt = x + ((b * L + t) * Hh + h) * P;
        double* yt = y + ((b * L + t) * Hh + h) * P;
        for (int64_t n = 0; n < N; ++n)
          for (int64_t p = 0; p < P; ++p)
            H[n * P + p] = a * H[n * P + p] + dt * Bt_[n] * xt[p];
        for (int64_t p = 0; p < P; ++p) {
          double s = 0.0;
          for (int64_t n = 0; n < N; ++n) s += Ct[n] * H[n * P + p];
          yt[p] = s + (Dh ? Dh[h] : 0.0) * xt[p];
        }
      }
      if (h_last)
        for (int64_t k = 0; k < N * P; ++k) h_last[(b * Hh + h) * N * P + k] = H[k];
      free(H);
    }
  }
  return 0;
}

/*
 * Complex diagonal A.  The pages name a complex diagonal initialisation
 * (S4D-Lin) beside the real one (S4D-Real) ("A Survey of Mamba" summary,
 * HiPPO-based memory initialisation) and compare complex with real decay in an
 * ablation ("Mamba: S4 epic upgrade", ablation on A).  A (D,N), B, C (Bt,L,N),
 * h0 and h_last (Bt,D,N) are complex, stored as (re, im) pairs in a last axis
 * of 2.  Per channel and step, with the same step size as oracle_fwd:
 *   abar  = exp(dt a)                                     complex exponential
 *   bcoef = (exp(dt a) - 1) / a  (exact ZOH; dt when a == 0 or in Euler mode)
 *   h_n   = abar h_n + bcoef B_n u
 *   y     = 2 Re(sum_n C_n h_n) + D u      each complex state stands for itself
 *                                          and its conjugate; the real output
 *                                          adds both, i.e. twice the real part
 *   out   = y * silu(z)
 */
int oracle_fwd_complex(int64_t Bt, int64_t L, int64_t D, int64_t N, int disc, int softplus,
                       const double* u, const double* delta, const double* A,
                       const double* Bm, const double* Cm, const double* Dskip,
                       const double* bias, const double* z, const double* h0,
                       double* out, double* h_last, int nthreads) {
  if (Bt < 0 || L < 0 || D < 0 || N < 1 || N > 64) return -1;
  int64_t nch = Bt * D;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
#endif
  for (int64_t ch = 0; ch < nch; ++ch) {
    int64_t b = ch / D, d = ch % D;
    double complex h[64];
    for (int64_t n = 0; n < N; ++n) {
      int64_t k = ((b * D + d) * N + n) * 2;
      h[n] = h0 ? h0[k] + I * h0[k + 1] : 0.0;
    }
    double dsk = Dskip ? Dskip[d] : 0.0;
    double bi = bias ? bias[d] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
      int64_t i = (b * L + t) * D + d;
      double dt = step_size(delta[i], bi, softplus);
      double ut = u[i];
      double complex acc = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        double complex a = A[(d * N + n) * 2] + I * A[(d * N + n) * 2 + 1];
        double complex abar = cexp(dt * a);
        double complex bcoef = (disc == ORACLE_EULER || a == 0.0) ? (double complex)dt
                                                                  : (abar - 1.0) / a;
        int64_t j = ((b * L + t) * N + n) * 2;
        double complex Bn = Bm[j] + I * Bm[j + 1];
        double complex Cn = Cm[j] + I * Cm[j + 1];
        h[n] = abar * h[n] + bcoef * Bn * ut;     /* recurrence */
        acc += Cn * h[n];                          /* output contraction */
      }
      double y = 2.0 * creal(acc) + dsk * ut;      /* conjugate pairs, skip D u */
      if (z) y *= z[i] * sigmoid(z[i]);            /* silu(z) gate */
      out[i] = y;
    }
    if (h_last)
      for (int64_t n = 0; n < N; ++n) {
        int64_t k = ((b * D + d) * N + n) * 2;
        h_last[k] = creal(h[n]);
        h_last[k + 1] = cimag(h[n]);
      }
  }
  (void)nthreads;
  return 0;
}
