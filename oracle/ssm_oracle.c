/*
 * ssm_oracle.c -- plain fp64 CPU oracle for the selective state-space scan (S6)
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * GPU path is compared against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header, table
 * or helper with the HIP library, and the HIP library never calls it.
 *
 * What it computes (one independent channel per (b, d) row):
 *
 *   Delta_t  = softplus(delta_raw[b,d,t] + bias[d])            (or without softplus)
 *   Abar_t,n = exp(Delta_t * A[d,n])                           (zero-order hold, diagonal A)
 *   Bbar_t,n = Delta_t                                         (Euler input term, default)
 *            = (exp(Delta_t * A[d,n]) - 1) / A[d,n]            (zero-order hold, flag; Delta_t at A = 0)
 *   h_t,n    = Abar_t,n * h_{t-1},n + Bbar_t,n * B[b,n,t] * u[b,d,t]
 *   y_t      = (sum_n C[b,n,t] * h_t,n + Dskip[d] * u[b,d,t]) * silu(z[b,d,t])
 *
 * Sources (web pages, cited by title and section):
 *  - "Mamba" paper review (wiki.alexanderbaur.de), section "SSM": the
 *    continuous system h' = Ah + Bx, y = Ch, its zero-order-hold
 *    discretisation Abar = exp(Delta A), and the recurrence
 *    h_t = Abar h_{t-1} + Bbar x_t read out through C; diagonal A applied
 *    per channel in SISO form.
 *  - "Paper: Mamba" course module (konke.bhala.ai/m/F12), "Math & data
 *    structures": zero-order hold Abar = exp(Delta A),
 *    Bbar = (exp(Delta A) - 1)/A B, with Euler as the alternative.  The
 *    default input term is the Euler form Bbar x = Delta * B * x; the flag
 *    `zoh` selects the zero-order-hold form, written with expm1 so it keeps
 *    its digits for small Delta*A, and equal to its limit Delta at A = 0.
 *  - "Exercises -- State-space models (Mamba, S4)" (brentwoodlivery.com):
 *    the recurrent view h_k = Abar h_{k-1} + Bbar x_k followed by
 *    y_k = C h_k (the readout comes after the update at the same step), the
 *    zero initial state of the worked impulse response, and
 *    softplus(x) = ln(1 + e^x) as the map that keeps Delta positive.
 *  - "Mamba" paper review, section "Mamba" block description: the block
 *    gates its output with a residual branch (no formula given).  Read here
 *    as the output gate y <- (C.h + Dskip*u) * silu(z), silu(z) = z/(1 + e^-z).
 *  - The same block description: before the SSM the expanded input goes
 *    through a convolution followed by a nonlinear function; NN LAB "Mamba"
 *    page, "Kernel Fusion in On-Chip SRAM": that convolution is causal, 1-D.
 *    Read here as a depthwise (per channel) causal convolution of width K
 *    along t, the last tap on the current input, plus a per-channel bias,
 *    followed by silu:  u[t] = silu(cb[d] + sum_k w[d,k] x[t-K+1+k]),
 *    with the K-1 inputs before t = 0 taken from a carried conv state (or
 *    zero).  oracle_causal_conv1d_silu computes it on its own; its output is
 *    the u of the scan.
 *
 * Backward (oracle_scan_bwd): the gradients of L = sum_t dy_t . y_t (plus
 * dlast . last_state) with respect to every input, by the chain rule through
 * the same sequential definition -- the recomputation the "Mamba" paper
 * review describes under "Optimization" (the intermediate states are
 * recomputed from the inputs, not stored).  Per channel: a forward sweep
 * keeps every h_t, then a reverse sweep carries the adjoint
 * lambda_t = dL/dh_t = ds_t C_t + Abar_{t+1} lambda_{t+1}.
 *
 * Precision: every input is widened to double before use and all arithmetic
 * is double.  No blocking, fusion or reordering beyond the sequential
 * definition: each row walks t = 0..L-1 in order, and within a step the
 * states n = 0..N-1 in order.  Rows are independent, so they may be handed
 * to worker threads; that changes nothing in any row's arithmetic.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* softplus(x) = ln(1 + e^x), written as max(x,0) + log1p(e^-|x|) so that it
 * neither overflows for large x nor loses digits for very negative x.  The
 * two forms are equal for every real x. */
static double softplus(double x) {
  double m = x > 0.0 ? x : 0.0;
  return m + log1p(exp(-fabs(x)));
}

/* Input-term coefficient: Delta (Euler), or (e^{Delta A} - 1)/A (zero-order
 * hold), whose limit at A = 0 is Delta. */
static double bbar(double dt, double a, int zoh) {
  if (!zoh || a == 0.0) return dt;
  return expm1(dt * a) / a;
}

/* silu(z) = z * sigmoid(z) = z / (1 + e^-z).  For z -> -inf, e^-z -> inf and
 * the quotient goes to -0, which is the limit. */
static double silu(double z) { return z / (1.0 + exp(-z)); }

typedef struct {
  const double *u, *delta, *A, *B, *C, *Dskip, *z, *bias, *h0;
  double *y, *last_state;
  int softplus_on, zoh;
  long batch, dim, dstate, seqlen;
  long row_begin, row_end;
} scan_job;

/* One channel (b, d), all L steps, in order. */
static void scan_row(const scan_job *j, long row, double *h) {
  const long b = row / j->dim, d = row % j->dim;
  const long N = j->dstate, L = j->seqlen;
  const double *u = j->u + row * L;
  const double *dr = j->delta + row * L;
  const double *z = j->z ? j->z + row * L : NULL;
  const double *Bb = j->B + b * N * L; /* B[b, n, t] at Bb[n*L + t] */
  const double *Cb = j->C + b * N * L;
  const double *Ad = j->A + d * N;
  const double bias = j->bias ? j->bias[d] : 0.0;
  const double Dd = j->Dskip ? j->Dskip[d] : 0.0;
  double *y = j->y + row * L;

  for (long n = 0; n < N; ++n) h[n] = j->h0 ? j->h0[row * N + n] : 0.0;

  for (long t = 0; t < L; ++t) {
    const double x = dr[t] + bias;
    const double dt = j->softplus_on ? softplus(x) : x;
    double acc = 0.0;
    for (long n = 0; n < N; ++n) {
      const double abar = exp(dt * Ad[n]);                 /* ZOH transition */
      h[n] = abar * h[n] + bbar(dt, Ad[n], j->zoh) * Bb[n * L + t] * u[t];
      acc += Cb[n * L + t] * h[n];                          /* readout after update */
    }
    acc += Dd * u[t];
    if (z) acc *= silu(z[t]);
    y[t] = acc;
  }
  if (j->last_state)
    for (long n = 0; n < N; ++n) j->last_state[row * N + n] = h[n];
}

static void *scan_worker(void *arg) {
  const scan_job *j = (const scan_job *)arg;
  double *h = (double *)malloc(sizeof(double) * (size_t)j->dstate);
  if (!h) return (void *)1;
  for (long r = j->row_begin; r < j->row_end; ++r) scan_row(j, r, h);
  free(h);
  return NULL;
}

/*
 * oracle_scan_fwd: the full forward scan.
 *   u, delta, z, y : (batch, dim, seqlen), seqlen fastest
 *   A              : (dim, dstate)
 *   B, C           : (batch, dstate, seqlen)
 *   Dskip, bias    : (dim,)            (NULL -> 0)
 *   z              : NULL -> no gate
 *   h0, last_state : (batch, dim, dstate) (NULL -> zero start / not written)
 *   softplus_on    : Delta = softplus(delta + bias), else delta + bias
 *   zoh            : zero-order-hold input term instead of Euler
 *   nthreads       : worker threads over rows (<= 1 -> run inline)
 * Returns 0 on success, -1 on bad arguments, -2 on allocation/thread failure.
 */
int oracle_scan_fwd(const double *u, const double *delta, const double *A,
                    const double *B, const double *C, const double *Dskip,
                    const double *z, const double *bias, int softplus_on, int zoh,
                    const double *h0, double *y, double *last_state, long batch,
                    long dim, long dstate, long seqlen, int nthreads) {
  if (!u || !delta || !A || !B || !C || !y) return -1;
  if (batch < 0 || dim < 0 || dstate < 1 || seqlen < 0) return -1;
  const long rows = batch * dim;
  scan_job base = {u, delta, A, B, C, Dskip, z, bias, h0, y, last_state,
                   softplus_on, zoh, batch, dim, dstate, seqlen, 0, rows};
  if (rows == 0) return 0;
  if (nthreads <= 1 || rows < 2) {
    return scan_worker(&base) ? -2 : 0;
  }
  if (nthreads > rows) nthreads = (int)rows;
  pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  scan_job *jobs = (scan_job *)malloc(sizeof(scan_job) * (size_t)nthreads);
  if (!tid || !jobs) { free(tid); free(jobs); return -2; }
  int rc = 0, started = 0;
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = base;
    jobs[i].row_begin = rows * i / nthreads;
    jobs[i].row_end = rows * (i + 1) / nthreads;
    if (pthread_create(&tid[i], NULL, scan_worker, &jobs[i]) != 0) { rc = -2; break; }
    ++started;
  }
  for (int i = 0; i < started; ++i) {
    void *ret = NULL;
    pthread_join(tid[i], &ret);
    if (ret) rc = -2;
  }
  free(tid);
  free(jobs);
  return rc;
}

/*
 * oracle_state_update: one decode step, the same recurrence with L = 1 and
 * the state carried by the caller ("Exercises -- State-space models":
 * generation runs the recurrence one token at a time with a constant-size
 * state).
 *   state : (batch, dim, dstate), updated in place
 *   u, delta, z, y : (batch, dim)
 *   B, C  : (batch, dstate)
 *   A     : (dim, dstate); Dskip, bias : (dim,) or NULL; z NULL -> no gate
 */
int oracle_state_update(double *state, const double *u, const double *delta,
                        const double *A, const double *B, const double *C,
                        const double *Dskip, const double *z, const double *bias,
                        int softplus_on, int zoh, double *y, long batch, long dim,
                        long dstate) {
  if (!state || !u || !delta || !A || !B || !C || !y) return -1;
  if (batch < 0 || dim < 0 || dstate < 1) return -1;
  for (long b = 0; b < batch; ++b) {
    for (long d = 0; d < dim; ++d) {
      const long row = b * dim + d;
      const double x = delta[row] + (bias ? bias[d] : 0.0);
      const double dt = softplus_on ? softplus(x) : x;
      double *h = state + row * dstate;
      double acc = 0.0;
      for (long n = 0; n < dstate; ++n) {
        const double abar = exp(dt * A[d * dstate + n]);
        h[n] = abar * h[n] + bbar(dt, A[d * dstate + n], zoh) * B[b * dstate + n] * u[row];
        acc += C[b * dstate + n] * h[n];
      }
      acc += (Dskip ? Dskip[d] : 0.0) * u[row];
      if (z) acc *= silu(z[row]);
      y[row] = acc;
    }
  }
  return 0;
}

/*
 * oracle_causal_conv1d_silu: u = silu(causal depthwise conv(x) + cb).
 *   x, u      : (batch, dim, seqlen)
 *   w         : (dim, K), tap K-1 multiplies the current input
 *   cb        : (dim,) or NULL
 *   state_in  : (batch, dim, K-1) or NULL: the K-1 inputs before t = 0,
 *               oldest first (NULL -> zeros)
 *   state_out : (batch, dim, K-1) or NULL: the K-1 last inputs (oldest
 *               first), taken from state_in where seqlen < K-1
 */
int oracle_causal_conv1d_silu(const double *x, const double *w, const double *cb, long K,
                              const double *state_in, double *u, double *state_out,
                              long batch, long dim, long seqlen) {
  if (!x || !w || !u || K < 1 || batch < 0 || dim < 0 || seqlen < 0) return -1;
  const long H = K - 1;
  for (long row = 0; row < batch * dim; ++row) {
    const long d = row % dim;
    const double *xr = x + row * seqlen;
    const double *si = state_in ? state_in + row * H : NULL;
    for (long t = 0; t < seqlen; ++t) {
      double acc = cb ? cb[d] : 0.0;
      for (long k = 0; k < K; ++k) {
        const long s = t - H + k;
        const double xv = s >= 0 ? xr[s] : (si ? si[H + s] : 0.0);
        acc += w[d * K + k] * xv;
      }
      u[row * seqlen + t] = silu(acc);
    }
    if (state_out)
      for (long j = 0; j < H; ++j) {
        const long s = seqlen - H + j;
        state_out[row * H + j] = s >= 0 ? xr[s] : (si ? si[H + s] : 0.0);
      }
  }
  return 0;
}

/*
 * oracle_conv_step: one token of the same convolution for decoding.
 *   conv_state : (batch, dim, K-1) inputs before this token, oldest first;
 *                shifted in place to end with x
 *   x, u       : (batch, dim)
 */
int oracle_conv_step(double *conv_state, const double *x, const double *w, const double *cb,
                     long K, double *u, long batch, long dim) {
  if ((!conv_state && K > 1) || !x || !w || !u || K < 1 || batch < 0 || dim < 0) return -1;
  const long H = K - 1;
  for (long row = 0; row < batch * dim; ++row) {
    const long d = row % dim;
    double *cs = conv_state ? conv_state + row * H : NULL;
    double acc = cb ? cb[d] : 0.0;
    for (long k = 0; k < H; ++k) acc += w[d * K + k] * cs[k];
    acc += w[d * K + H] * x[row];
    u[row] = silu(acc);
    for (long k = 0; k + 1 < H; ++k) cs[k] = cs[k + 1];
    if (H > 0) cs[H - 1] = x[row];
  }
  return 0;
}

/* silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z))) */
static double silu_grad(double z) {
  const double sg = 1.0 / (1.0 + exp(-z));
  return sg * (1.0 + z * (1.0 - sg));
}

/* d Bbar / d Delta and d Bbar / d A for the input coefficient of bbar(). */
static double bbar_d_dt(double dt, double a, int zoh) {
  if (!zoh) return 1.0;
  return exp(dt * a); /* d/dDelta (e^{Delta A} - 1)/A = e^{Delta A}, also at A = 0 */
}
static double bbar_d_a(double dt, double a, int zoh) {
  if (!zoh) return 0.0;
  if (a == 0.0) return 0.5 * dt * dt; /* limit of (Delta A e^{Delta A} - (e^{Delta A} - 1))/A^2 */
  const double e = exp(dt * a);
  return (dt * a * e - expm1(dt * a)) / (a * a);
}

typedef struct {
  const double *u, *delta, *A, *B, *C, *Dskip, *z, *bias, *h0, *dy, *dlast;
  int softplus_on, zoh;
  long batch, dim, dstate, seqlen;
  long row_begin, row_end;
  /* outputs: per-element ones written directly, reduced ones per job */
  double *du, *ddelta, *dz, *dh0;
  double *dA, *dB, *dC, *dD, *dbias; /* this job's private sums */
} bwd_job;

static void *bwd_worker(void *arg) {
  bwd_job *j = (bwd_job *)arg;
  const long N = j->dstate, L = j->seqlen, dim = j->dim;
  double *hs = (double *)malloc(sizeof(double) * (size_t)((L + 1) * N));
  double *dts = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  double *ss = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  double *lam = (double *)malloc(sizeof(double) * (size_t)N);
  if (!hs || !dts || !ss || !lam) { free(hs); free(dts); free(ss); free(lam); return (void *)1; }
  for (long row = j->row_begin; row < j->row_end; ++row) {
    const long b = row / dim, d = row % dim;
    const double *u = j->u + row * L, *dr = j->delta + row * L;
    const double *z = j->z ? j->z + row * L : NULL;
    const double *gy = j->dy + row * L;
    const double *Bb = j->B + b * N * L, *Cb = j->C + b * N * L, *Ad = j->A + d * N;
    const double bias = j->bias ? j->bias[d] : 0.0;
    const double Dd = j->Dskip ? j->Dskip[d] : 0.0;
    /* forward sweep: hs[(t+1)*N + n] = h_t, hs[n] = h_{-1} */
    for (long n = 0; n < N; ++n) hs[n] = j->h0 ? j->h0[row * N + n] : 0.0;
    for (long t = 0; t < L; ++t) {
      const double x = dr[t] + bias;
      const double dt = j->softplus_on ? softplus(x) : x;
      dts[t] = dt;
      double acc = 0.0;
      for (long n = 0; n < N; ++n) {
        const double h = exp(dt * Ad[n]) * hs[t * N + n] + bbar(dt, Ad[n], j->zoh) * Bb[n * L + t] * u[t];
        hs[(t + 1) * N + n] = h;
        acc += Cb[n * L + t] * h;
      }
      ss[t] = acc + Dd * u[t]; /* the output before the gate */
    }
    /* reverse sweep */
    for (long n = 0; n < N; ++n) lam[n] = j->dlast ? j->dlast[row * N + n] : 0.0;
    for (long t = L - 1; t >= 0; --t) {
      const double dt = dts[t];
      double ds = gy[t];
      if (z) {
        j->dz[row * L + t] = gy[t] * ss[t] * silu_grad(z[t]);
        ds = gy[t] * silu(z[t]);
      }
      j->dD[d] += ds * u[t];
      double du = ds * Dd, ddt = 0.0;
      for (long n = 0; n < N; ++n) {
        const double h = hs[(t + 1) * N + n], hp = hs[t * N + n];
        const double a = exp(dt * Ad[n]);
        const double bb = bbar(dt, Ad[n], j->zoh);
        const double bu = Bb[n * L + t] * u[t];
        lam[n] += ds * Cb[n * L + t];            /* dL/dh_t */
        j->dC[b * N * L + n * L + t] += ds * h;
        ddt += lam[n] * (hp * a * Ad[n] + bbar_d_dt(dt, Ad[n], j->zoh) * bu);
        j->dA[d * N + n] += lam[n] * (hp * a * dt + bbar_d_a(dt, Ad[n], j->zoh) * bu);
        j->dB[b * N * L + n * L + t] += lam[n] * bb * u[t];
        du += lam[n] * bb * Bb[n * L + t];
        lam[n] *= a;                             /* dL/dh_{t-1} */
      }
      j->du[row * L + t] = du;
      const double x = dr[t] + bias;
      const double dx = j->softplus_on ? ddt / (1.0 + exp(-x)) : ddt; /* softplus' = sigmoid */
      j->ddelta[row * L + t] = dx;
      j->dbias[d] += dx;
    }
    if (j->dh0)
      for (long n = 0; n < N; ++n) j->dh0[row * N + n] = lam[n];
  }
  free(hs); free(dts); free(ss); free(lam);
  return NULL;
}

/*
 * oracle_scan_bwd: gradients of L = sum(dy * y) + sum(dlast * last_state)
 * for the forward scan of oracle_scan_fwd (same arguments and layouts).
 *   dy        : (batch, dim, seqlen)           required
 *   dlast     : (batch, dim, dstate) or NULL   (NULL -> 0)
 *   du, ddelta: (batch, dim, seqlen)           written
 *   dz        : (batch, dim, seqlen)           written when z is given
 *   dA        : (dim, dstate); dB, dC: (batch, dstate, seqlen);
 *   dD, dbias : (dim,); dh0: (batch, dim, dstate) or NULL -- all written
 * Rows are split over nthreads workers; the reduced gradients are summed
 * per worker and then over workers in worker order.
 */
int oracle_scan_bwd(const double *u, const double *delta, const double *A, const double *B,
                    const double *C, const double *Dskip, const double *z, const double *bias,
                    int softplus_on, int zoh, const double *h0, const double *dy,
                    const double *dlast, double *du, double *ddelta, double *dA, double *dB,
                    double *dC, double *dD, double *dz, double *dbias, double *dh0, long batch,
                    long dim, long dstate, long seqlen, int nthreads) {
  if (!u || !delta || !A || !B || !C || !dy || !du || !ddelta || !dA || !dB || !dC || !dD ||
      !dbias || (z && !dz))
    return -1;
  if (batch < 0 || dim < 0 || dstate < 1 || seqlen < 0) return -1;
  const long rows = batch * dim, N = dstate, L = seqlen;
  const size_t nA = (size_t)(dim * N), nBC = (size_t)(batch * N * L), nd = (size_t)dim;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > rows && rows > 0) nthreads = (int)rows;
  double *priv = (double *)calloc((size_t)nthreads * (nA + 2 * nBC + 2 * nd) + 1, sizeof(double));
  bwd_job *jobs = (bwd_job *)malloc(sizeof(bwd_job) * (size_t)nthreads);
  pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!priv || !jobs || !tid) { free(priv); free(jobs); free(tid); return -2; }
  int rc = 0, started = 0;
  for (int i = 0; i < nthreads; ++i) {
    double *p = priv + (size_t)i * (nA + 2 * nBC + 2 * nd);
    bwd_job jb = {u, delta, A, B, C, Dskip, z, bias, h0, dy, dlast, softplus_on, zoh,
                  batch, dim, dstate, seqlen, rows * i / nthreads, rows * (i + 1) / nthreads,
                  du, ddelta, dz, dh0, p, p + nA, p + nA + nBC, p + nA + 2 * nBC,
                  p + nA + 2 * nBC + nd};
    jobs[i] = jb;
  }
  if (nthreads == 1) {
    rc = bwd_worker(&jobs[0]) ? -2 : 0;
  } else {
    for (int i = 0; i < nthreads; ++i) {
      if (pthread_create(&tid[i], NULL, bwd_worker, &jobs[i]) != 0) { rc = -2; break; }
      ++started;
    }
    for (int i = 0; i < started; ++i) {
      void *ret = NULL;
      pthread_join(tid[i], &ret);
      if (ret) rc = -2;
    }
  }
  for (size_t k = 0; k < nA; ++k) dA[k] = 0.0;
  for (size_t k = 0; k < nBC; ++k) dB[k] = dC[k] = 0.0;
  for (size_t k = 0; k < nd; ++k) dD[k] = dbias[k] = 0.0;
  for (int i = 0; i < nthreads; ++i) {
    const bwd_job *jb = &jobs[i];
    for (size_t k = 0; k < nA; ++k) dA[k] += jb->dA[k];
    for (size_t k = 0; k < nBC; ++k) { dB[k] += jb->dB[k]; dC[k] += jb->dC[k]; }
    for (size_t k = 0; k < nd; ++k) { dD[k] += jb->dD[k]; dbias[k] += jb->dbias[k]; }
  }
  free(priv); free(jobs); free(tid);
  return rc;
}
