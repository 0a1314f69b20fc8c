/*
 * ssm_oracle.c -- plain fp64 CPU oracle for the Mamba-1 selective scan and its
 * single-token state update.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The GPU product path
 * never calls it, and it shares no code, header or constant with the HIP
 * sources.
 *
 * What it computes (sources are the five pages on Mamba; cited by page title
 * and section):
 *   - "Mamba模型笔记" (Mamba model notes), section 2.2: discrete SSM
 *     h_t = Abar h_{t-1} + Bbar x_t,  y_t = C h_t + D x_t.
 *   - same page, section 4.4: one independent SSM per channel, so the state
 *     of channel d is a vector over the state index n and A is diagonal per
 *     channel (A[d,n]); exp is elementwise.
 *   - same page, section 4.1: B, C and the step size Delta depend on the
 *     input token; here they are given per (batch, n, t) and per (batch, d, t).
 *   - Mamba paper notes (0539edu.com), section 2.3: zero-order-hold
 *     discretisation as used in practice: Abar = exp(Delta*A), Bbar = Delta*B,
 *     Cbar = C, with Delta kept positive by a softplus.
 *   - Mamba training/inference guide (zhouruolin.cn), FAQ item 2: the
 *     projection bias places Delta in a target range -> Delta =
 *     softplus(dt + bias[d]).
 *   - Mamba model notes, section 4.3: the gate branch multiplies the SSM
 *     output; gate = silu(z) applied after the D skip term.
 *   - Mamba paper notes, section 4.3: recurrent inference keeps only a
 *     fixed-size state per (batch, channel) and updates it once per token
 *     (the decode form below).
 *   - Mamba paper notes, section 5.5: the state starts at zero.
 *
 * Readings where the pages are silent:
 *   softplus is exact (max(x,0) + log1p(exp(-|x|))), no threshold; the
 *   initial state is h0 when given, else zero; out = (sum_n C h + D u) * silu(z).
 *
 * Parity pins live in tests/test_oracle_pins.py (LTI convolution, Delta -> 0,
 * L = 1 closed form, split sequence, decode == scan, reset, A = 0 prefix sum,
 * linearity, unrolled-sum brute force in fp64 and 40-digit decimal) and, for
 * the backward, in tests/test_oracle_bwd_pins.py (exact Jacobian-vector
 * products of the forward for the inputs it is linear in, central
 * differences of the forward for the others).
 *
 * Layouts (all contiguous, row-major):
 *   u, delta, z, out : (batch, dim, seqlen)
 *   Bm, Cm           : (batch, ngroups, dstate, seqlen); channel d reads
 *                      group d / (dim / ngroups) (ngroups = 1: one B_t, C_t
 *                      per token shared by every channel, as in the pages)
 *   A                : (dim, dstate)
 *   Dv, bias         : (dim)
 *   h0, last_state   : (batch, dim, dstate)
 * Decode: state (batch, dim, dstate); x, dt, z, out (batch, dim);
 *         Bm, Cm (batch, ngroups, dstate).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

double oracle_softplus(double x) {
  /* log(1 + e^x) written so that neither branch overflows or cancels */
  return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

static double step_size(double dt, const double* bias, int64_t d, int softplus) {
  double x = dt + (bias ? bias[d] : 0.0);
  return softplus ? oracle_softplus(x) : x;
}

/* One (batch, channel) row of the prefill scan, strictly sequential in t. */
static void scan_row(int64_t b, int64_t d, int64_t dim, int64_t L, int64_t N, int64_t G,
                     const double* u, const double* delta, const double* z,
                     const double* Bm, const double* Cm, const double* A,
                     const double* Dv, const double* bias, int softplus,
                     const double* h0, double* out, double* last_state, double* h) {
  const int64_t row = (b * dim + d) * L;
  const int64_t grp = b * G + d / (dim / G);           /* this channel's B/C group */
  const double* Bb = Bm + grp * N * L;
  const double* Cb = Cm + grp * N * L;
  for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[(b * dim + d) * N + n] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    const double ut = u[row + t];
    const double dl = step_size(delta[row + t], bias, d, softplus);
    double y = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double abar = exp(dl * A[d * N + n]);      /* Abar = exp(Delta*A)   */
      const double bbar_u = dl * Bb[n * L + t] * ut;    /* Bbar*u = Delta*B*u    */
      h[n] = abar * h[n] + bbar_u;
      y += Cb[n * L + t] * h[n];                        /* C_t . h_t             */
    }
    if (Dv) y += Dv[d] * ut;                            /* skip term D*u         */
    if (z) y *= oracle_silu(z[row + t]);                /* gate, after the skip  */
    out[row + t] = y;
  }
  if (last_state)
    for (int64_t n = 0; n < N; ++n) last_state[(b * dim + d) * N + n] = h[n];
}

/* Prefill: runs every (batch, channel) row; rows are independent, so they are
 * spread over OpenMP threads (nthreads <= 0 means the runtime default). The
 * recurrence over t inside a row stays sequential. Returns the thread count. */
int oracle_selective_scan_f64(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate,
                              int64_t ngroups, const double* u, const double* delta, const double* z,
                              const double* Bm, const double* Cm, const double* A,
                              const double* Dv, const double* bias, int softplus,
                              const double* h0, double* out, double* last_state,
                              int nthreads) {
  int used = 1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
  {
#pragma omp single
    used = omp_get_num_threads();
    double h[1024];
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < batch * dim; ++r)
      scan_row(r / dim, r % dim, dim, seqlen, dstate, ngroups, u, delta, z, Bm, Cm, A, Dv, bias,
               softplus, h0, out, last_state, h);
  }
#else
  (void)nthreads;
  double h[1024];
  for (int64_t r = 0; r < batch * dim; ++r)
    scan_row(r / dim, r % dim, dim, seqlen, dstate, ngroups, u, delta, z, Bm, Cm, A, Dv, bias,
             softplus, h0, out, last_state, h);
#endif
  return used;
}

/* Decode: one token per (batch, channel); state updated in place.  Written as
 * its own loop body (not a call into scan_row) so that "decode equals scan" is
 * a real check between two pieces of code. */
static void update_row(int64_t r, int64_t dim, int64_t N, int64_t G, double* state,
                       const double* x, const double* dt, const double* z,
                       const double* Bm, const double* Cm, const double* A,
                       const double* Dv, const double* bias, int softplus, double* out) {
  const int64_t b = r / dim, d = r % dim;
  const double* Bt = Bm + (b * G + d / (dim / G)) * N;  /* this channel's group */
  const double* Ct = Cm + (b * G + d / (dim / G)) * N;
  const double xt = x[r];
  double dl = dt[r] + (bias ? bias[d] : 0.0);
  if (softplus) dl = oracle_softplus(dl);
  double* s = state + r * N;
  double y = 0.0;
  for (int64_t n = 0; n < N; ++n) {
    s[n] = exp(dl * A[d * N + n]) * s[n] + dl * Bt[n] * xt;
    y += Ct[n] * s[n];
  }
  if (Dv) y += Dv[d] * xt;
  if (z) y *= oracle_silu(z[r]);
  out[r] = y;
}

int oracle_state_update_f64(int64_t batch, int64_t dim, int64_t dstate, int64_t ngroups,
                            double* state,
                            const double* x, const double* dt, const double* z,
                            const double* Bm, const double* Cm, const double* A,
                            const double* Dv, const double* bias, int softplus,
                            double* out, int nthreads) {
  int used = 1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
  {
#pragma omp single
    used = omp_get_num_threads();
#pragma omp for schedule(static)
    for (int64_t r = 0; r < batch * dim; ++r)
      update_row(r, dim, dstate, ngroups, state, x, dt, z, Bm, Cm, A, Dv, bias, softplus, out);
  }
#else
  (void)nthreads;
  for (int64_t r = 0; r < batch * dim; ++r)
    update_row(r, dim, dstate, ngroups, state, x, dt, z, Bm, Cm, A, Dv, bias, softplus, out);
#endif
  return used;
}

/* ------------------------------------------------------------------------ *
 * Backward of the prefill scan (reverse-mode derivative of the loop in
 * scan_row), for one upstream gradient dout on out and, optionally, dlast on
 * last_state.  Chain rule through each step, in fp64:
 *   gate     out = y s(z) z,  s = logistic:  dy = dout * silu(z),
 *            dz = dout * y * s (1 + z (1 - s))
 *   readout  y = sum_n C h_t + D u:  dC += dy h_t,  dD += dy u,  du += dy D,
 *            adjoint of h_t gains dy C
 *   step     h_t = e_t h_{t-1} + Delta B u,  e_t = exp(Delta A):
 *            with g the adjoint of h_t,
 *            dB += g Delta u,  du += g Delta B,
 *            dDelta += g (B u + A e_t h_{t-1}),  dA += g Delta e_t h_{t-1},
 *            adjoint of h_{t-1} = e_t g
 *   Delta    Delta = softplus(x), x = delta + bias:  dx = dDelta s(x)
 *            (dx = dDelta without softplus);  ddelta = dx,  dbias += dx
 *   h0       dh0 = adjoint of h_{-1}
 * Rows (b, d) run on OpenMP threads into per-row slots; the sums over rows
 * (dB and dC over d, dA/dD/dbias over b and t) are then added in a fixed
 * order, so the result does not depend on the thread count.
 * ------------------------------------------------------------------------ */
static double logistic(double x) { return 1.0 / (1.0 + exp(-x)); }

static void scan_row_bwd(int64_t b, int64_t d, int64_t dim, int64_t L, int64_t N, int64_t G,
                         const double* u, const double* delta, const double* z,
                         const double* Bm, const double* Cm, const double* A,
                         const double* Dv, const double* bias, int softplus,
                         const double* h0, const double* dout, const double* dlast,
                         double* du, double* ddelta, double* dz,
                         double* dBrow, double* dCrow, double* dArow, double* dDrow,
                         double* dbrow, double* dh0, double* hs, double* es, double* g) {
  const int64_t row = (b * dim + d) * L;
  const int64_t grp = b * G + d / (dim / G);
  const double* Bb = Bm + grp * N * L;
  const double* Cb = Cm + grp * N * L;
  /* forward again, keeping every h_t and e_t (hs[(t+1)*N + n] = h_t, hs[n] = h_{-1}) */
  for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[(b * dim + d) * N + n] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    const double xt = delta[row + t] + (bias ? bias[d] : 0.0);
    const double step = softplus ? oracle_softplus(xt) : xt;
    for (int64_t n = 0; n < N; ++n) {
      const double decay = exp(step * A[d * N + n]);
      es[t * N + n] = decay;
      hs[(t + 1) * N + n] = decay * hs[t * N + n] + step * Bb[n * L + t] * u[row + t];
    }
  }
  for (int64_t n = 0; n < N; ++n) {
    g[n] = dlast ? dlast[(b * dim + d) * N + n] : 0.0;
    dArow[n] = 0.0;
  }
  double sumD = 0.0, sumbias = 0.0;
  for (int64_t t = L - 1; t >= 0; --t) {
    const double ut = u[row + t];
    const double xt = delta[row + t] + (bias ? bias[d] : 0.0);
    const double step = softplus ? oracle_softplus(xt) : xt;
    /* y_t again (before the gate), for dz */
    double yt = 0.0;
    for (int64_t n = 0; n < N; ++n) yt += Cb[n * L + t] * hs[(t + 1) * N + n];
    if (Dv) yt += Dv[d] * ut;
    double dy = dout[row + t];
    if (z) {
      const double zt = z[row + t], sg = logistic(zt);
      dz[row + t] = dy * yt * sg * (1.0 + zt * (1.0 - sg));
      dy *= zt * sg;
    }
    double dut = Dv ? dy * Dv[d] : 0.0;
    sumD += dy * ut;
    double dstep = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double ht = hs[(t + 1) * N + n], hp = hs[t * N + n], et = es[t * N + n];
      dCrow[n * L + t] = dy * ht;
      const double adj = g[n] + dy * Cb[n * L + t];      /* adjoint of h_t */
      dBrow[n * L + t] = adj * step * ut;
      dut += adj * step * Bb[n * L + t];
      dstep += adj * (Bb[n * L + t] * ut + A[d * N + n] * et * hp);
      dArow[n] += adj * step * et * hp;
      g[n] = et * adj;                                    /* adjoint of h_{t-1} */
    }
    const double dx = softplus ? dstep * logistic(xt) : dstep;
    du[row + t] = dut;
    ddelta[row + t] = dx;
    sumbias += dx;
  }
  *dDrow = sumD;
  *dbrow = sumbias;
  if (dh0)
    for (int64_t n = 0; n < N; ++n) dh0[(b * dim + d) * N + n] = g[n];
}

/* Gradients of the prefill scan.  Outputs: du, ddelta (batch, dim, L); dz
 * (when z is given); dB, dC (batch, ngroups, N, L), each summed over the
 * channels of its group; dA (dim, N); dD, dbias (dim; when
 * D / bias are given); dh0 (batch, dim, N; when h0 is given).  dlast may be
 * NULL (no gradient on last_state).  Returns the thread count used. */
int oracle_selective_scan_bwd_f64(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate,
                                  int64_t ngroups, const double* u, const double* delta, const double* z,
                                  const double* Bm, const double* Cm, const double* A,
                                  const double* Dv, const double* bias, int softplus,
                                  const double* h0, const double* dout, const double* dlast,
                                  double* du, double* ddelta, double* dz, double* dB,
                                  double* dC, double* dA, double* dD, double* dbias,
                                  double* dh0, int nthreads) {
  const int64_t L = seqlen, N = dstate, G = ngroups, rows = batch * dim;
  double* dBrows = (double*)calloc((size_t)(rows * N * L > 0 ? rows * N * L : 1), sizeof(double));
  double* dCrows = (double*)calloc((size_t)(rows * N * L > 0 ? rows * N * L : 1), sizeof(double));
  double* dArows = (double*)calloc((size_t)(rows * N > 0 ? rows * N : 1), sizeof(double));
  double* dDrows = (double*)calloc((size_t)(rows > 0 ? rows : 1), sizeof(double));
  double* dbrows = (double*)calloc((size_t)(rows > 0 ? rows : 1), sizeof(double));
  int used = 1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
  {
#pragma omp single
    used = omp_get_num_threads();
    double* hs = (double*)malloc(sizeof(double) * (size_t)((L + 1) * N));
    double* es = (double*)malloc(sizeof(double) * (size_t)(L * N + 1));
    double* g = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r)
      scan_row_bwd(r / dim, r % dim, dim, L, N, G, u, delta, z, Bm, Cm, A, Dv, bias, softplus, h0,
                   dout, dlast, du, ddelta, dz, dBrows + r * N * L, dCrows + r * N * L,
                   dArows + r * N, dDrows + r, dbrows + r, dh0, hs, es, g);
    free(hs); free(es); free(g);
  }
#else
  (void)nthreads;
  {
    double* hs = (double*)malloc(sizeof(double) * (size_t)((L + 1) * N));
    double* es = (double*)malloc(sizeof(double) * (size_t)(L * N + 1));
    double* g = (double*)malloc(sizeof(double) * (size_t)N);
    for (int64_t r = 0; r < rows; ++r)
      scan_row_bwd(r / dim, r % dim, dim, L, N, G, u, delta, z, Bm, Cm, A, Dv, bias, softplus, h0,
                   dout, dlast, du, ddelta, dz, dBrows + r * N * L, dCrows + r * N * L,
                   dArows + r * N, dDrows + r, dbrows + r, dh0, hs, es, g);
    free(hs); free(es); free(g);
  }
#endif
  /* sums over rows, in a fixed order: dB, dC over the channels of each group */
  const int64_t cpg = G > 0 ? dim / G : 0;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t gi = 0; gi < G; ++gi)
      for (int64_t i = 0; i < N * L; ++i) {
        double sb = 0.0, sc = 0.0;
        for (int64_t d = gi * cpg; d < (gi + 1) * cpg; ++d) {
          sb += dBrows[(b * dim + d) * N * L + i];
          sc += dCrows[(b * dim + d) * N * L + i];
        }
        dB[(b * G + gi) * N * L + i] = sb;
        dC[(b * G + gi) * N * L + i] = sc;
      }
  for (int64_t d = 0; d < dim; ++d) {
    double sD = 0.0, sb = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      double sA = 0.0;
      for (int64_t b = 0; b < batch; ++b) sA += dArows[(b * dim + d) * N + n];
      dA[d * N + n] = sA;
    }
    for (int64_t b = 0; b < batch; ++b) {
      sD += dDrows[b * dim + d];
      sb += dbrows[b * dim + d];
    }
    if (dD) dD[d] = sD;
    if (dbias) dbias[d] = sb;
  }
  free(dBrows); free(dCrows); free(dArows); free(dDrows); free(dbrows);
  return used;
}

/* ------------------------------------------------------------------------ *
 * Causal depthwise convolution of the Mamba block's conv branch (Mamba model
 * notes, section 4.3: the branch feeding the SSM passes a local convolution
 * first; the block's printed parameter count holds d_inner x d_conv weights
 * plus a bias per channel), optionally followed by SiLU:
 *   pre[b,d,t] = bias[d] + sum_{k=0}^{K-1} w[d,k] * x[b,d,t-(K-1)+k]
 *   u[b,d,t]   = silu(pre) (or pre)
 * x before t = 0 comes from the conv state: state[b,d,k] = x[b,d,k-K] for
 * k = 0..K-1 (zeros when no state is given).  state_out receives the last K
 * inputs, x[L-K .. L-1], in the same layout.
 * ------------------------------------------------------------------------ */
int oracle_causal_conv1d_f64(int64_t batch, int64_t dim, int64_t seqlen, int64_t K,
                             const double* x, const double* w, const double* bias,
                             const double* state_in, int silu, double* u, double* state_out,
                             int nthreads) {
  int used = 1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
  {
#pragma omp single
    used = omp_get_num_threads();
#pragma omp for schedule(static)
#else
  (void)nthreads;
#endif
    for (int64_t r = 0; r < batch * dim; ++r) {
      const int64_t d = r % dim;
      const double* xr = x + r * seqlen;
      for (int64_t t = 0; t < seqlen; ++t) {
        double acc = bias ? bias[d] : 0.0;
        for (int64_t k = 0; k < K; ++k) {
          const int64_t s = t - (K - 1) + k;           /* input index */
          const double xv = s >= 0 ? xr[s] : (state_in ? state_in[r * K + K + s] : 0.0);
          acc += w[d * K + k] * xv;
        }
        u[r * seqlen + t] = silu ? oracle_silu(acc) : acc;
      }
      if (state_out)
        for (int64_t k = 0; k < K; ++k) {
          const int64_t s = seqlen - K + k;
          state_out[r * K + k] = s >= 0 ? xr[s] : (state_in ? state_in[r * K + K + s] : 0.0);
        }
    }
#ifdef _OPENMP
  }
#endif
  return used;
}

/* One decode token of the conv branch: shift the state left by one, append
 * x, and form the output from the new state (written as its own loop so that
 * "decode equals prefill" is a check between two pieces of code). */
int oracle_conv_state_update_f64(int64_t batch, int64_t dim, int64_t K, double* state,
                                 const double* x, const double* w, const double* bias, int silu,
                                 double* u) {
  for (int64_t r = 0; r < batch * dim; ++r) {
    const int64_t d = r % dim;
    double* s = state + r * K;
    for (int64_t k = 0; k + 1 < K; ++k) s[k] = s[k + 1];
    s[K - 1] = x[r];
    double acc = bias ? bias[d] : 0.0;
    for (int64_t k = 0; k < K; ++k) acc += w[d * K + k] * s[k];
    u[r] = silu ? oracle_silu(acc) : acc;
  }
  return 1;
}

/* ------------------------------------------------------------------------ *
 * Mamba-2 SSM (the SSD layer), recurrent form, in fp64.
 *
 * Mamba-2 is multi-head (Mamba-2 section of the mamba_ssm notes and the
 * skill page's Mamba-2 configuration: headdim, ngroups): the inner width is
 * H heads of P channels, and the block's printed parameter count (6,468,320
 * for d_model 1024, d_state 64) has one A, one D and one step bias per head
 * and 2 * ngroups * d_state B/C numbers per token.  So for batch b, head h,
 * channel p of the head and state n, with g = h / (H / G) the head's group:
 *   Delta_t   = softplus(dt[b,t,h] + bias[h])        (one step per head)
 *   S_t[p,n]  = exp(Delta_t A[h]) S_{t-1}[p,n] + Delta_t B[b,t,g,n] x[b,t,h,p]
 *   y[b,t,h,p]= sum_n C[b,t,g,n] S_t[p,n] + D[h] x[b,t,h,p],  times silu(z)
 * starting from S_{-1} = h0[b,h] (or zero) and returning S_{L-1}.  The
 * structured-matrix (attention-like) view the pages call state space
 * duality is the same map written as y = M x; the pins check the two agree.
 *
 * Layouts (contiguous, row-major): x, z, out (batch, L, H, P); dt (batch,
 * L, H); Bm, Cm (batch, L, G, N); A, Dv, bias (H); h0, last (batch, H, P, N).
 * ------------------------------------------------------------------------ */
static void ssd_head(int64_t b, int64_t h, int64_t L, int64_t H, int64_t P, int64_t G,
                     int64_t N, const double* x, const double* dt, const double* z,
                     const double* Bm, const double* Cm, const double* A, const double* Dv,
                     const double* bias, int softplus, const double* h0, double* out,
                     double* last, double* S) {
  const int64_t g = h / (H / G);                      /* the head's B/C group */
  for (int64_t i = 0; i < P * N; ++i) S[i] = h0 ? h0[(b * H + h) * P * N + i] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    const double step = step_size(dt[(b * L + t) * H + h], bias, h, softplus);
    const double decay = exp(step * A[h]);            /* scalar decay per head */
    const double* Bt = Bm + ((b * L + t) * G + g) * N;
    const double* Ct = Cm + ((b * L + t) * G + g) * N;
    for (int64_t p = 0; p < P; ++p) {
      const int64_t xi = ((b * L + t) * H + h) * P + p;
      const double xv = x[xi];
      double y = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        S[p * N + n] = decay * S[p * N + n] + step * Bt[n] * xv;
        y += Ct[n] * S[p * N + n];
      }
      if (Dv) y += Dv[h] * xv;
      if (z) y *= oracle_silu(z[xi]);
      out[xi] = y;
    }
  }
  if (last)
    for (int64_t i = 0; i < P * N; ++i) last[(b * H + h) * P * N + i] = S[i];
}

int oracle_ssd_scan_f64(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t ngroups, int64_t dstate, const double* x, const double* dt,
                        const double* z, const double* Bm, const double* Cm, const double* A,
                        const double* Dv, const double* bias, int softplus, const double* h0,
                        double* out, double* last, int nthreads) {
  int used = 1;
  const int64_t PN = headdim * dstate > 0 ? headdim * dstate : 1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
  {
#pragma omp single
    used = omp_get_num_threads();
    double* S = (double*)malloc(sizeof(double) * (size_t)PN);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < batch * nheads; ++r)
      ssd_head(r / nheads, r % nheads, seqlen, nheads, headdim, ngroups, dstate, x, dt, z, Bm,
               Cm, A, Dv, bias, softplus, h0, out, last, S);
    free(S);
  }
#else
  (void)nthreads;
  double* S = (double*)malloc(sizeof(double) * (size_t)PN);
  for (int64_t r = 0; r < batch * nheads; ++r)
    ssd_head(r / nheads, r % nheads, seqlen, nheads, headdim, ngroups, dstate, x, dt, z, Bm, Cm,
             A, Dv, bias, softplus, h0, out, last, S);
  free(S);
#endif
  return used;
}
