/*
 * fp64 CPU oracle for the selective state space hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the HIP library is checked against.  Only the tests, the
 * package smoke check and the benchmark's CPU-baseline leg may load it; the
 * library never does, and this file shares no code with it.
 *
 * Every routine runs the sequential recurrence exactly as the pages state it,
 * one independent unit (a (batch, channel) pair, or a (batch, head) pair for
 * SSD) at a time, in double precision.  Threads only split the independent
 * units; nothing is blocked, fused or reordered inside a unit.
 *
 * Sources (page title, then section / equation):
 *  - "Mamba (deep learning)" (wiki article), state-space paragraph:
 *    discretisation of the continuous model gives the decay Abar = exp(Delta*A).
 *  - "Mamba-1/2/3 visual guide" (blog.yecov.com), section 1, SSM equation:
 *    h_t = Abar_t h_{t-1} + Bbar_t x_t,  y_t = C_t h_t.
 *  - same blog, section 2, selectivity table: Delta, B, C depend on the
 *    current input (they vary with t); block diagram: the SSM output is
 *    multiplied elementwise by a gate branch.
 *  - same blog, section 2 figure "train/prefill -> parallel scan, one-token
 *    generation -> recurrent update, same model": the decode step is one
 *    step of the same recurrence.
 *  - same blog, section 3 comparison table: Mamba-2 restricts A to a scalar
 *    times identity per head; chunk figure: chunks pass the state.
 * Readings where the pages are silent (they leave Bbar undefined, and say
 * nothing of D or of the gate's form):
 *  - Bbar_t x_t = delta_t * B_t * u_t (Euler-style input term);
 *  - y_t reads the state after the update at step t (so it includes u_t);
 *  - out = (C_t . h_t + D * u_t) * silu(z_t), silu(z) = z / (1 + exp(-z));
 *    D null -> no skip term, z null -> no gate;
 *  - the initial state is h0 when given, else zero.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* ------------------------------------------------------------------------ */
/* Selective scan.                                                           */
/* u, delta, z, y: [batch, dim, seqlen]; B, C: [batch, dstate, seqlen];      */
/* A: [dim, dstate]; D: [dim]; h0, h_last: [batch, dim, dstate].             */
/* ------------------------------------------------------------------------ */
typedef struct {
  const double *u, *delta, *A, *B, *C, *D, *z, *h0;
  double *y, *h_last;
  long batch, dim, dstate, seqlen;
  long unit_begin, unit_end;
} scan_job;

static void scan_unit(const scan_job* j, long b, long d) {
  const long N = j->dstate, L = j->seqlen;
  double* h = (double*)malloc(sizeof(double) * (size_t)N);
  for (long n = 0; n < N; ++n) h[n] = j->h0 ? j->h0[(b * j->dim + d) * N + n] : 0.0;
  const double* u = j->u + (b * j->dim + d) * L;
  const double* dl = j->delta + (b * j->dim + d) * L;
  const double* z = j->z ? j->z + (b * j->dim + d) * L : NULL;
  double* y = j->y + (b * j->dim + d) * L;
  const double* Bb = j->B + b * N * L;
  const double* Cb = j->C + b * N * L;
  const double Dd = j->D ? j->D[d] : 0.0;
  for (long t = 0; t < L; ++t) {
    double acc = 0.0;
    for (long n = 0; n < N; ++n) {
      double abar = exp(dl[t] * j->A[d * N + n]);          /* Abar_t = exp(delta_t A) */
      h[n] = abar * h[n] + dl[t] * Bb[n * L + t] * u[t];   /* + Bbar_t u_t            */
      acc += Cb[n * L + t] * h[n];                         /* C_t . h_t               */
    }
    double out = acc + Dd * u[t];
    y[t] = z ? out * silu(z[t]) : out;
  }
  if (j->h_last)
    for (long n = 0; n < N; ++n) j->h_last[(b * j->dim + d) * N + n] = h[n];
  free(h);
}

static void* scan_worker(void* arg) {
  const scan_job* j = (const scan_job*)arg;
  for (long k = j->unit_begin; k < j->unit_end; ++k) scan_unit(j, k / j->dim, k % j->dim);
  return NULL;
}

void oracle_selective_scan(const double* u, const double* delta, const double* A, const double* B,
                           const double* C, const double* D, const double* z, const double* h0,
                           double* y, double* h_last, long batch, long dim, long dstate, long seqlen,
                           int nthreads) {
  long units = batch * dim;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > units) nthreads = (int)(units > 0 ? units : 1);
  scan_job* jobs = (scan_job*)calloc((size_t)nthreads, sizeof(scan_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int i = 0; i < nthreads; ++i) {
    scan_job j = {u, delta, A, B, C, D, z, h0, y, h_last, batch, dim, dstate, seqlen,
                  units * i / nthreads, units * (i + 1) / nthreads};
    jobs[i] = j;
    pthread_create(&th[i], NULL, scan_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
}

/* ------------------------------------------------------------------------ */
/* Selective scan, backward: the gradient of a scalar loss with respect to   */
/* every input of the forward above, given dy = dloss/dy (and dh_last =      */
/* dloss/dh_last, or zero).  Training runs the same model over whole         */
/* sequences ("Mamba (deep learning)", paragraph on how it generates and     */
/* trains; visual guide section 2 figure: training/prefill use the parallel  */
/* scan); the gradient is the derivative of the forward as defined, written  */
/* out by the chain rule in reverse time, with the forward states kept.      */
/* For each (b, d), with dh the gradient of the state after step t:          */
/*   dout_t = dy_t * silu(z_t);  dz_t = dy_t * out_t * silu'(z_t)            */
/*   dh    += C_t dout_t               (then dC_t += dout_t h_t)             */
/*   h_t = a_t h_{t-1} + delta_t B_t u_t,  a_t = exp(delta_t A):             */
/*   dA += dh h_{t-1} a_t delta_t;  ddelta_t += dh (h_{t-1} a_t A + B_t u_t) */
/*   du_t += dh delta_t B_t (+ D dout_t);  dB_t += dh delta_t u_t            */
/*   dh    <- a_t dh                   (the gradient of h_{t-1})             */
/* and dh0 is dh after step 0.  dB, dC sum over d; dA, dD over b and t.      */
/* ------------------------------------------------------------------------ */
typedef struct {
  const double *u, *delta, *A, *B, *C, *D, *z, *h0, *dy, *dh_last;
  double *du, *ddelta, *dz, *dh0;
  double *dA, *dB, *dC, *dD;  /* this thread's partial sums (zeroed by the caller) */
  long batch, dim, dstate, seqlen;
  long unit_begin, unit_end;
} bwd_job;

static void bwd_unit(const bwd_job* j, long b, long d) {
  const long N = j->dstate, L = j->seqlen;
  const size_t row = (size_t)(b * j->dim + d);
  const double* u = j->u + row * L;
  const double* dl = j->delta + row * L;
  const double* z = j->z ? j->z + row * L : NULL;
  const double* dy = j->dy + row * L;
  const double* Bb = j->B + b * N * L;
  const double* Cb = j->C + b * N * L;
  const double* Ad = j->A + d * N;
  const double Dd = j->D ? j->D[d] : 0.0;
  /* forward, keeping every state (hs[t*N + n] = h after step t) and out_t */
  double* hs = (double*)malloc(sizeof(double) * (size_t)(L * N));
  double* out = (double*)malloc(sizeof(double) * (size_t)L);
  double* h0 = (double*)malloc(sizeof(double) * (size_t)N);
  double* dh = (double*)malloc(sizeof(double) * (size_t)N);
  for (long n = 0; n < N; ++n) h0[n] = j->h0 ? j->h0[row * N + n] : 0.0;
  for (long t = 0; t < L; ++t) {
    double acc = 0.0;
    for (long n = 0; n < N; ++n) {
      const double hp = t > 0 ? hs[(t - 1) * N + n] : h0[n];
      const double h = exp(dl[t] * Ad[n]) * hp + dl[t] * Bb[n * L + t] * u[t];
      hs[t * N + n] = h;
      acc += Cb[n * L + t] * h;
    }
    out[t] = acc + Dd * u[t];
  }
  /* reverse */
  for (long n = 0; n < N; ++n) dh[n] = j->dh_last ? j->dh_last[row * N + n] : 0.0;
  for (long t = L - 1; t >= 0; --t) {
    double dout = dy[t];
    if (z) {
      const double sg = 1.0 / (1.0 + exp(-z[t]));
      dout = dy[t] * z[t] * sg;                                    /* dy * silu(z)        */
      j->dz[row * L + t] = dy[t] * out[t] * sg * (1.0 + z[t] * (1.0 - sg)); /* silu'(z)  */
    }
    double du = Dd * dout, dd = 0.0;
    if (j->D) j->dD[d] += dout * u[t];
    for (long n = 0; n < N; ++n) {
      const double h = hs[t * N + n];
      const double hp = t > 0 ? hs[(t - 1) * N + n] : h0[n];
      const double a = exp(dl[t] * Ad[n]);
      dh[n] += Cb[n * L + t] * dout;
      j->dC[(b * N + n) * L + t] += dout * h;
      j->dA[d * N + n] += dh[n] * hp * a * dl[t];
      dd += dh[n] * (hp * a * Ad[n] + Bb[n * L + t] * u[t]);
      du += dh[n] * dl[t] * Bb[n * L + t];
      j->dB[(b * N + n) * L + t] += dh[n] * dl[t] * u[t];
      dh[n] *= a;
    }
    j->du[row * L + t] = du;
    j->ddelta[row * L + t] = dd;
  }
  if (j->dh0)
    for (long n = 0; n < N; ++n) j->dh0[row * N + n] = dh[n];
  free(hs);
  free(out);
  free(h0);
  free(dh);
}

static void* bwd_worker(void* arg) {
  const bwd_job* j = (const bwd_job*)arg;
  for (long k = j->unit_begin; k < j->unit_end; ++k) bwd_unit(j, k / j->dim, k % j->dim);
  return NULL;
}

/* dA [dim, dstate], dB, dC [batch, dstate, seqlen], dD [dim] are written   */
/* (not accumulated); dz is written only when z is given, dh0 when non-null. */
void oracle_selective_scan_bwd(const double* u, const double* delta, const double* A, const double* B,
                               const double* C, const double* D, const double* z, const double* h0,
                               const double* dy, const double* dh_last, double* du, double* ddelta,
                               double* dA, double* dB, double* dC, double* dD, double* dz, double* dh0,
                               long batch, long dim, long dstate, long seqlen, int nthreads) {
  long units = batch * dim;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > units) nthreads = (int)(units > 0 ? units : 1);
  const size_t nA = (size_t)(dim * dstate), nBC = (size_t)(batch * dstate * seqlen), nD = (size_t)dim;
  const size_t per = nA + 2 * nBC + nD;
  double* part = (double*)calloc((size_t)nthreads * per, sizeof(double));
  bwd_job* jobs = (bwd_job*)calloc((size_t)nthreads, sizeof(bwd_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int i = 0; i < nthreads; ++i) {
    double* p = part + (size_t)i * per;
    bwd_job j = {u, delta, A, B, C, D, z, h0, dy, dh_last, du, ddelta, dz, dh0,
                 p, p + nA, p + nA + nBC, p + nA + 2 * nBC, batch, dim, dstate, seqlen,
                 units * i / nthreads, units * (i + 1) / nthreads};
    jobs[i] = j;
    pthread_create(&th[i], NULL, bwd_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  /* partial sums added in thread order */
  memset(dA, 0, nA * sizeof(double));
  memset(dB, 0, nBC * sizeof(double));
  memset(dC, 0, nBC * sizeof(double));
  if (dD) memset(dD, 0, nD * sizeof(double));
  for (int i = 0; i < nthreads; ++i) {
    const double* p = part + (size_t)i * per;
    for (size_t k = 0; k < nA; ++k) dA[k] += p[k];
    for (size_t k = 0; k < nBC; ++k) dB[k] += p[nA + k];
    for (size_t k = 0; k < nBC; ++k) dC[k] += p[nA + nBC + k];
    if (dD)
      for (size_t k = 0; k < nD; ++k) dD[k] += p[nA + 2 * nBC + k];
  }
  free(th);
  free(jobs);
  free(part);
}

/* ------------------------------------------------------------------------ */
/* One-token state update (generation): one step of the same recurrence,     */
/* with the state read and written in place.                                 */
/* h: [batch, dim, dstate]; u, delta, z, y: [batch, dim]; B, C: [batch, dstate] */
/* ------------------------------------------------------------------------ */
typedef struct {
  double* h;
  const double *u, *delta, *A, *B, *C, *D, *z;
  double* y;
  long batch, dim, dstate;
  long unit_begin, unit_end;
} update_job;

static void* update_worker(void* arg) {
  const update_job* j = (const update_job*)arg;
  const long N = j->dstate;
  for (long bd = j->unit_begin; bd < j->unit_end; ++bd) {
    const long b = bd / j->dim, d = bd % j->dim;
    double acc = 0.0;
    for (long n = 0; n < N; ++n) {
      double abar = exp(j->delta[bd] * j->A[d * N + n]);
      j->h[bd * N + n] = abar * j->h[bd * N + n] + j->delta[bd] * j->B[b * N + n] * j->u[bd];
      acc += j->C[b * N + n] * j->h[bd * N + n];
    }
    double out = acc + (j->D ? j->D[d] : 0.0) * j->u[bd];
    j->y[bd] = j->z ? out * silu(j->z[bd]) : out;
  }
  return NULL;
}

void oracle_state_update(double* h, const double* u, const double* delta, const double* A,
                         const double* B, const double* C, const double* D, const double* z,
                         double* y, long batch, long dim, long dstate, int nthreads) {
  long units = batch * dim;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > units) nthreads = (int)(units > 0 ? units : 1);
  update_job* jobs = (update_job*)calloc((size_t)nthreads, sizeof(update_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int i = 0; i < nthreads; ++i) {
    update_job j = {h, u, delta, A, B, C, D, z, y, batch, dim, dstate,
                    units * i / nthreads, units * (i + 1) / nthreads};
    jobs[i] = j;
    pthread_create(&th[i], NULL, update_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
}

/* ------------------------------------------------------------------------ */
/* Mamba-2 (SSD) layer, computed as its plain recurrence: per head the decay */
/* is one scalar exp(delta * A_h) applied to the whole P x N state; heads of */
/* one group share B and C.  No chunking: the chunk size only decides at     */
/* which steps the state is recorded in chunk_states.                        */
/* x, z, y: [batch, seqlen, nheads, headdim]; delta: [batch, seqlen, nheads];*/
/* A, D: [nheads]; B, C: [batch, seqlen, ngroups, dstate];                   */
/* h0, h_last: [batch, nheads, headdim, dstate];                             */
/* chunk_states: [batch, nchunks, nheads, headdim, dstate], the state after  */
/* the last step of each chunk.                                              */
/* ------------------------------------------------------------------------ */
typedef struct {
  const double *x, *delta, *A, *B, *C, *D, *z, *h0;
  double *y, *chunk_states, *h_last;
  long batch, seqlen, nheads, headdim, ngroups, dstate, chunk;
  long unit_begin, unit_end;
} ssd_job;

static void ssd_unit(const ssd_job* j, long b, long hd) {
  const long L = j->seqlen, H = j->nheads, P = j->headdim, G = j->ngroups, N = j->dstate;
  const long g = hd / (H / G);
  const long nchunks = (L + j->chunk - 1) / j->chunk;
  double* S = (double*)malloc(sizeof(double) * (size_t)(P * N));
  for (long i = 0; i < P * N; ++i) S[i] = j->h0 ? j->h0[(b * H + hd) * P * N + i] : 0.0;
  for (long t = 0; t < L; ++t) {
    const double dlt = j->delta[(b * L + t) * H + hd];
    const double abar = exp(dlt * j->A[hd]);
    const double* Bt = j->B + ((b * L + t) * G + g) * N;
    const double* Ct = j->C + ((b * L + t) * G + g) * N;
    const double* xt = j->x + ((b * L + t) * H + hd) * P;
    double* yt = j->y + ((b * L + t) * H + hd) * P;
    for (long p = 0; p < P; ++p) {
      double acc = 0.0;
      for (long n = 0; n < N; ++n) {
        S[p * N + n] = abar * S[p * N + n] + dlt * Bt[n] * xt[p];
        acc += Ct[n] * S[p * N + n];
      }
      double out = acc + (j->D ? j->D[hd] : 0.0) * xt[p];
      yt[p] = j->z ? out * silu(j->z[((b * L + t) * H + hd) * P + p]) : out;
    }
    if (j->chunk_states && ((t + 1) % j->chunk == 0 || t == L - 1)) {
      long c = t / j->chunk;
      memcpy(j->chunk_states + (((b * nchunks + c) * H + hd) * P * N), S, sizeof(double) * (size_t)(P * N));
    }
  }
  if (j->h_last) memcpy(j->h_last + (b * H + hd) * P * N, S, sizeof(double) * (size_t)(P * N));
  free(S);
}

static void* ssd_worker(void* arg) {
  const ssd_job* j = (const ssd_job*)arg;
  for (long k = j->unit_begin; k < j->unit_end; ++k) ssd_unit(j, k / j->nheads, k % j->nheads);
  return NULL;
}

void oracle_ssd(const double* x, const double* delta, const double* A, const double* B,
                const double* C, const double* D, const double* z, const double* h0, double* y,
                double* chunk_states, double* h_last, long batch, long seqlen, long nheads,
                long headdim, long ngroups, long dstate, long chunk, int nthreads) {
  long units = batch * nheads;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > units) nthreads = (int)(units > 0 ? units : 1);
  ssd_job* jobs = (ssd_job*)calloc((size_t)nthreads, sizeof(ssd_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int i = 0; i < nthreads; ++i) {
    ssd_job j = {x, delta, A, B, C, D, z, h0, y, chunk_states, h_last, batch, seqlen, nheads,
                 headdim, ngroups, dstate, chunk, units * i / nthreads, units * (i + 1) / nthreads};
    jobs[i] = j;
    pthread_create(&th[i], NULL, ssd_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
}

/* ------------------------------------------------------------------------ */
/* Scan prologue: the short causal convolution that feeds u, and delta from */
/* its raw value.                                                            */
/* x, delta_raw, u, delta: [batch, dim, seqlen]; conv_w: [dim, 4] (tap 3     */
/* multiplies the current step); conv_b, delta_bias: [dim] or NULL.          */
/*                                                                           */
/* Sources: "Mamba (deep learning)", paragraph on the block (an input        */
/* projection, a short convolution, the selective state space layer and a    */
/* gate); "Mamba State-Space Models", usage example (d_conv = 4, the         */
/* convolution's kernel size).  Readings where the pages are silent: the     */
/* convolution is depthwise (one 4-tap filter per channel) and causal, with  */
/* zeros before the first step, plus a per-channel bias; its output is used  */
/* as is, or through silu when conv_silu is set; delta is                    */
/* softplus(delta_raw + bias) when softplus is set (the form of the          */
/* workload's delta), else delta_raw + bias.  softplus(v) = log(1 + exp(v)). */
/* ------------------------------------------------------------------------ */
static double softplus(double v) { return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v)); }

void oracle_scan_prologue(const double* x, const double* conv_w, const double* conv_b, const double* delta_raw,
                          const double* delta_bias, double* u, double* delta, long batch, long dim, long seqlen,
                          int conv_silu, int use_softplus) {
  for (long b = 0; b < batch; ++b) {
    for (long d = 0; d < dim; ++d) {
      const double* xr = x + (b * dim + d) * seqlen;
      const double* dr = delta_raw + (b * dim + d) * seqlen;
      double* ur = u + (b * dim + d) * seqlen;
      double* dlr = delta + (b * dim + d) * seqlen;
      for (long t = 0; t < seqlen; ++t) {
        double acc = conv_b ? conv_b[d] : 0.0;
        for (long k = 0; k < 4; ++k) {
          const long s = t - 3 + k; /* tap k reads step t - 3 + k */
          if (s >= 0) acc += conv_w[d * 4 + k] * xr[s];
        }
        ur[t] = conv_silu ? silu(acc) : acc;
        const double v = dr[t] + (delta_bias ? delta_bias[d] : 0.0);
        dlr[t] = use_softplus ? softplus(v) : v;
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Mamba-3 state update (one generation step), with its three changes to    */
/* the recurrence as options.                                                */
/*                                                                           */
/* Source: "Mamba-1/2/3 visual guide" (blog.yecov.com), section 4: Mamba-3  */
/* updates the state with an exponential-trapezoidal discretisation (an     */
/* exponential transition and an input approximation that uses both ends of */
/* the step), a complex-valued state that decays while it rotates, and MIMO */
/* (several inputs and outputs per state update, as a small matrix product */
/* that raises decode's arithmetic intensity); the section 4 table keeps    */
/* the Mamba-2 head structure (scalar decay per head, heads of a group      */
/* sharing B and C).  The page gives no formulas; the readings taken:       */
/*  - trapezoid: the input integral over the step,                           */
/*    int_0^delta exp(A (delta - s)) b(s) ds with b = B x, by the trapezoid  */
/*    rule: (delta/2) (alpha b_prev + b_cur), alpha the step's transition;   */
/*    without it the Euler-style term delta * b_cur of the other calls.      */
/*  - complex state: per head and state n the transition is                  */
/*    alpha_n = exp(delta A_h) (cos(delta theta_n) + i sin(delta theta_n)),  */
/*    the rotation angle growing with delta (data dependent); B, C, x are   */
/*    real; the readout takes the real part of C . h.                       */
/*  - MIMO rank R: per head, R input vectors x_r (headdim P) and R pairs of  */
/*    B_r, C_r (dstate N): H <- alpha H + w sum_r x_r B_r^T and R outputs    */
/*    y_r = Re(H) C_r (+ D x_r, times silu(z_r)); R = 1 is the SISO update. */
/* Per (b, head h), g = h / (H/G), state row p and state n:                 */
/*   alpha = exp(delta A_h) [* (cos, sin)(delta theta[h, n])]                */
/*   u_cur = sum_r x[b,h,r,p] B[b,g,r,n];  u_prev likewise from x_prev, B_prev */
/*   h[p,n] <- alpha h[p,n] + (delta/2)(alpha u_prev + u_cur)   (trapezoid)  */
/*   h[p,n] <- alpha h[p,n] + delta u_cur                       (otherwise)  */
/*   y[b,h,r,p] = (sum_n C[b,g,r,n] Re h[p,n] + D_h x[b,h,r,p]) * silu(z)    */
/* Layouts: h [batch, nheads, headdim, dstate] (x2 re/im last when complex); */
/* x, x_prev, z, y [batch, nheads, rank, headdim]; B, C, B_prev [batch,      */
/* ngroups, rank, dstate]; delta [batch, nheads]; A, D [nheads]; theta       */
/* [nheads, dstate].  x_prev and B_prev NULL = no trapezoid.                  */
/* ------------------------------------------------------------------------ */
typedef struct {
  double* h;
  const double *x, *x_prev, *delta, *A, *theta, *B, *B_prev, *C, *D, *z;
  double* y;
  long batch, nheads, headdim, ngroups, dstate, rank;
  int complex_state;
  long unit_begin, unit_end;
} m3_job;

static void m3_unit(const m3_job* j, long b, long hd) {
  const long H = j->nheads, P = j->headdim, G = j->ngroups, N = j->dstate, R = j->rank;
  const long g = hd / (H / G);
  const double dlt = j->delta[b * H + hd];
  const double a = exp(dlt * j->A[hd]);
  const int trap = j->x_prev != NULL;
  const double* xs = j->x + (b * H + hd) * R * P;
  const double* xp = trap ? j->x_prev + (b * H + hd) * R * P : NULL;
  const double* Bs = j->B + (b * G + g) * R * N;
  const double* Bp = trap ? j->B_prev + (b * G + g) * R * N : NULL;
  const double* Cs = j->C + (b * G + g) * R * N;
  const long stride = j->complex_state ? 2 : 1;
  double* hs = j->h + (b * H + hd) * P * N * stride;
  for (long p = 0; p < P; ++p) {
    for (long n = 0; n < N; ++n) {
      double ucur = 0.0, uprev = 0.0;
      for (long r = 0; r < R; ++r) {
        ucur += xs[r * P + p] * Bs[r * N + n];
        if (trap) uprev += xp[r * P + p] * Bp[r * N + n];
      }
      double ar = a, ai = 0.0; /* the transition alpha = ar + i ai */
      if (j->complex_state) {
        const double ang = dlt * j->theta[hd * N + n];
        ar = a * cos(ang);
        ai = a * sin(ang);
      }
      double* e = hs + (p * N + n) * stride;
      const double re = e[0], im = j->complex_state ? e[1] : 0.0;
      double nre = ar * re - ai * im, nim = ar * im + ai * re; /* alpha * h */
      if (trap) {
        nre += 0.5 * dlt * (ar * uprev + ucur);
        nim += 0.5 * dlt * (ai * uprev);
      } else {
        nre += dlt * ucur;
      }
      e[0] = nre;
      if (j->complex_state) e[1] = nim;
    }
  }
  for (long r = 0; r < R; ++r) {
    for (long p = 0; p < P; ++p) {
      double acc = 0.0;
      for (long n = 0; n < N; ++n) acc += Cs[r * N + n] * hs[(p * N + n) * stride];
      double out = acc + (j->D ? j->D[hd] : 0.0) * xs[r * P + p];
      const long o = ((b * H + hd) * R + r) * P + p;
      j->y[o] = j->z ? out * silu(j->z[o]) : out;
    }
  }
}

static void* m3_worker(void* arg) {
  const m3_job* j = (const m3_job*)arg;
  for (long k = j->unit_begin; k < j->unit_end; ++k) m3_unit(j, k / j->nheads, k % j->nheads);
  return NULL;
}

void oracle_mamba3_step(double* h, const double* x, const double* x_prev, const double* delta, const double* A,
                        const double* theta, const double* B, const double* B_prev, const double* C, const double* D,
                        const double* z, double* y, long batch, long nheads, long headdim, long ngroups,
                        long dstate, long rank, int complex_state, int nthreads) {
  long units = batch * nheads;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > units) nthreads = (int)(units > 0 ? units : 1);
  m3_job* jobs = (m3_job*)calloc((size_t)nthreads, sizeof(m3_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int i = 0; i < nthreads; ++i) {
    m3_job j = {h, x, x_prev, delta, A, theta, B, B_prev, C, D, z, y, batch, nheads, headdim, ngroups, dstate,
                rank, complex_state, units * i / nthreads, units * (i + 1) / nthreads};
    jobs[i] = j;
    pthread_create(&th[i], NULL, m3_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
}

/* ------------------------------------------------------------------------ */
/* Mamba-2 (SSD) layer, backward: the gradient of a scalar loss through      */
/* oracle_ssd, given dy = dloss/dy and optionally dh_last = dloss/dh_last.   */
/* Training runs the layer over whole sequences ("Mamba (deep learning)",   */
/* paragraph on training and generation; "Mamba-1/2/3 visual guide",        */
/* section 3 table: Mamba-2 trains with the chunked algorithm); its gradient */
/* is the chain rule through the recurrence, here in reverse time, one step */
/* at a time.  Per (b, head h, group g), with G the gradient of the state   */
/* after step t and a_t = exp(delta_t A_h):                                  */
/*   dout = dy * silu(z);  dz = dy * out * silu'(z)    (out = C.S + D x)     */
/*   G += dout C_t^T;  dC_t += S_t^T dout;  dD += dout . x_t                 */
/*   dx_t = delta_t G B_t + D dout;  dB_t += delta_t G^T x_t                 */
/*   ddelta_t = x_t^T G B_t + A_h a_t <G, S_{t-1}>;  dA_h += delta_t a_t <G, S_{t-1}> */
/*   G *= a_t   (the gradient of S_{t-1});  dh0 = G at the end               */
/* dB and dC are summed over the heads of a group.  Layouts as oracle_ssd;  */
/* dx, dz [batch, seqlen, nheads, headdim]; ddelta [batch, seqlen, nheads]; */
/* dA, dD [nheads]; dB, dC [batch, seqlen, ngroups, dstate]; dh0 [batch,    */
/* nheads, headdim, dstate].  The forward states are kept (seqlen x P x N   */
/* per unit).  Units are (b, head); each thread sums its units' dB and dC   */
/* parts in arrays of its own, added in thread order at the end.            */
/* ------------------------------------------------------------------------ */
typedef struct {
  const double *x, *delta, *A, *B, *C, *D, *z, *h0, *dy, *dh_last;
  double *dx, *ddelta, *dA_part, *dB, *dC, *dD_part, *dz, *dh0;
  long batch, seqlen, nheads, headdim, ngroups, dstate;
  long unit_begin, unit_end;
} ssd_bwd_job;

static double dsilu(double z) { /* d/dz of z sigma(z) */
  const double sg = 1.0 / (1.0 + exp(-z));
  return sg * (1.0 + z * (1.0 - sg));
}

static void ssd_bwd_head(const ssd_bwd_job* j, long b, long hd) {
  const long L = j->seqlen, H = j->nheads, P = j->headdim, G = j->ngroups, N = j->dstate;
  const long g = hd / (H / G);
  const double A = j->A[hd], D = j->D ? j->D[hd] : 0.0;
  /* forward, keeping every state: Ss[t+1] is the state after step t, Ss[0] the initial one */
  double* Ss = (double*)malloc(sizeof(double) * (size_t)((L + 1) * P * N));
  for (long i = 0; i < P * N; ++i) Ss[i] = j->h0 ? j->h0[(b * H + hd) * P * N + i] : 0.0;
  for (long t = 0; t < L; ++t) {
    const double dlt = j->delta[(b * L + t) * H + hd], a = exp(dlt * A);
    const double* Bt = j->B + ((b * L + t) * G + g) * N;
    const double* xt = j->x + ((b * L + t) * H + hd) * P;
    const double* prev = Ss + t * P * N;
    double* cur = Ss + (t + 1) * P * N;
    for (long p = 0; p < P; ++p)
      for (long n = 0; n < N; ++n) cur[p * N + n] = a * prev[p * N + n] + dlt * Bt[n] * xt[p];
  }
  /* reverse */
  double* Gs = (double*)malloc(sizeof(double) * (size_t)(P * N));
  double* dout = (double*)malloc(sizeof(double) * (size_t)P);
  for (long i = 0; i < P * N; ++i) Gs[i] = j->dh_last ? j->dh_last[(b * H + hd) * P * N + i] : 0.0;
  double dA = 0.0, dD = 0.0;
  for (long t = L - 1; t >= 0; --t) {
    const double dlt = j->delta[(b * L + t) * H + hd], a = exp(dlt * A);
    const double* Bt = j->B + ((b * L + t) * G + g) * N;
    const double* Ct = j->C + ((b * L + t) * G + g) * N;
    const long xo = ((b * L + t) * H + hd) * P;
    const double* xt = j->x + xo;
    const double* St = Ss + (t + 1) * P * N;
    const double* Sp = Ss + t * P * N;
    for (long p = 0; p < P; ++p) {
      double out = D * xt[p];
      for (long n = 0; n < N; ++n) out += Ct[n] * St[p * N + n];
      const double dyv = j->dy[xo + p];
      if (j->z) {
        const double zv = j->z[xo + p];
        dout[p] = dyv * (zv / (1.0 + exp(-zv)));
        j->dz[xo + p] = dyv * out * dsilu(zv);
      } else {
        dout[p] = dyv;
      }
      dD += dout[p] * xt[p];
    }
    double* dCt = j->dC + ((b * L + t) * G + g) * N;
    double* dBt = j->dB + ((b * L + t) * G + g) * N;
    for (long n = 0; n < N; ++n) {
      double acc = 0.0;
      for (long p = 0; p < P; ++p) {
        Gs[p * N + n] += dout[p] * Ct[n];
        acc += St[p * N + n] * dout[p];
      }
      dCt[n] += acc;
    }
    double gsp = 0.0, xgb = 0.0;
    for (long p = 0; p < P; ++p) {
      double gb = 0.0;
      for (long n = 0; n < N; ++n) {
        gb += Gs[p * N + n] * Bt[n];
        gsp += Gs[p * N + n] * Sp[p * N + n];
      }
      j->dx[xo + p] = dlt * gb + D * dout[p];
      xgb += xt[p] * gb;
    }
    for (long n = 0; n < N; ++n) {
      double acc = 0.0;
      for (long p = 0; p < P; ++p) acc += Gs[p * N + n] * xt[p];
      dBt[n] += dlt * acc;
    }
    j->ddelta[(b * L + t) * H + hd] = xgb + A * a * gsp;
    dA += dlt * a * gsp;
    for (long i = 0; i < P * N; ++i) Gs[i] *= a;
  }
  if (j->dh0) memcpy(j->dh0 + (b * H + hd) * P * N, Gs, sizeof(double) * (size_t)(P * N));
  j->dA_part[b * H + hd] = dA;
  j->dD_part[b * H + hd] = dD;
  free(dout);
  free(Gs);
  free(Ss);
}

static void* ssd_bwd_worker(void* arg) {
  const ssd_bwd_job* j = (const ssd_bwd_job*)arg;
  for (long k = j->unit_begin; k < j->unit_end; ++k) ssd_bwd_head(j, k / j->nheads, k % j->nheads);
  return NULL;
}

void oracle_ssd_bwd(const double* x, const double* delta, const double* A, const double* B, const double* C,
                    const double* D, const double* z, const double* h0, const double* dy, const double* dh_last,
                    double* dx, double* ddelta, double* dA, double* dB, double* dC, double* dD, double* dz,
                    double* dh0, long batch, long seqlen, long nheads, long headdim, long ngroups, long dstate,
                    int nthreads) {
  const long H = nheads;
  memset(dB, 0, sizeof(double) * (size_t)(batch * seqlen * ngroups * dstate));
  memset(dC, 0, sizeof(double) * (size_t)(batch * seqlen * ngroups * dstate));
  double* dA_part = (double*)calloc((size_t)(batch * H), sizeof(double));
  double* dD_part = (double*)calloc((size_t)(batch * H), sizeof(double));
  long units = batch * H;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > units) nthreads = (int)(units > 0 ? units : 1);
  const size_t nbc = (size_t)(batch * seqlen * ngroups * dstate);
  ssd_bwd_job* jobs = (ssd_bwd_job*)calloc((size_t)nthreads, sizeof(ssd_bwd_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int i = 0; i < nthreads; ++i) {
    /* thread 0 sums into the outputs, the others into arrays of their own */
    double* pB = i == 0 ? dB : (double*)calloc(nbc, sizeof(double));
    double* pC = i == 0 ? dC : (double*)calloc(nbc, sizeof(double));
    ssd_bwd_job jb = {x, delta, A, B, C, D, z, h0, dy, dh_last, dx, ddelta, dA_part, pB, pC, dD_part, dz, dh0,
                      batch, seqlen, nheads, headdim, ngroups, dstate, units * i / nthreads,
                      units * (i + 1) / nthreads};
    jobs[i] = jb;
    pthread_create(&th[i], NULL, ssd_bwd_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  for (int i = 1; i < nthreads; ++i) {
    for (size_t e = 0; e < nbc; ++e) {
      dB[e] += jobs[i].dB[e];
      dC[e] += jobs[i].dC[e];
    }
    free(jobs[i].dB);
    free(jobs[i].dC);
  }
  for (long hd = 0; hd < H; ++hd) {
    double sa = 0.0, sd = 0.0;
    for (long b = 0; b < batch; ++b) {
      sa += dA_part[b * H + hd];
      sd += dD_part[b * H + hd];
    }
    dA[hd] = sa;
    if (dD) dD[hd] = sd;
  }
  free(th);
  free(jobs);
  free(dD_part);
  free(dA_part);
}
