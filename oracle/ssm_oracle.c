/*
 * Plain fp64 CPU oracle for the selective state-space scan forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's cpu_baseline leg may load this library.  The product path (the
 * HIP library) shares no code with it.
 *
 * What it computes follows the pages' statement of the method, written out as
 * the plain serial definition (no blocking, no reordering):
 *
 *  - Recurrence and readout (pwwt.cn article, section 1.1 "the recursion"):
 *        h_t = Abar_t * h_{t-1} + Bbar_t * x_t,   y_t = C_t . h_t + D * x_t
 *    with y_t using the state after step t has been absorbed and the same-step
 *    C_t.
 *  - Diagonal state transition per (channel, state), A = -exp(A_log) < 0 and
 *    Delta = softplus(raw) > 0, so Abar = exp(Delta * A) lies in (0, 1)
 *    (pwwt.cn section 2.4 "numerical stability").  Bbar * x is Delta * B * x.
 *  - Optional clip of Delta after softplus (pwwt.cn section 3.3 "fusion
 *    boundary": softplus, then upper/lower clip).
 *  - Padding folded in as the identity element (a, b) = (1, 0) so that padded
 *    steps leave the state unchanged (pwwt.cn section 2.3 "segments and
 *    resets"); y at padded steps is +0.0 and the final state is the state after
 *    the last valid step.
 *  - Zero initial state unless h0 is given (pwwt.cn section 4.1, the naive
 *    reference loop starts from zeros when no h0 is passed).
 *  - Optional extras of the fused kernel the nxbn.cn article describes
 *    (section 3, its kernel body): a per-channel bias added to the raw delta
 *    before softplus, and an output gate y <- y * silu(z), silu(z) =
 *    z / (1 + e^-z), applied to the full readout (C.h + D x).  Optional
 *    chunk-boundary states: the state after the last step of every chunk of
 *    chunk_len steps (the boundary states of the pwwt.cn article, section 3.4,
 *    kept for recomputation).
 *
 * Every input arrives as fp64 (bf16 and fp32 inputs convert exactly); all
 * arithmetic is fp64 with the C library's exp/log1p.
 *
 * Readings taken where the pages are silent (see the design notes): Delta is
 * passed raw and softplus is a step of the method; clamp after softplus;
 * valid lengths are clamped to [0, L]; B and C are shared by all channels of a
 * batch row.
 *
 * ORACLE_MUTATION (compile-time, tests only) plants one known mistake so the
 * tests can show that their pins notice it.  0 = the correct oracle.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTATION
#define ORACLE_MUTATION 0
#endif

#if defined(__GNUC__)
#define ORACLE_API __attribute__((visibility("default")))
#else
#define ORACLE_API
#endif

/* h_t = a_t * h_{t-1} + b_t for t = 0..L-1 starting from h0 (pwwt.cn section
 * 2.1: the step as the affine map h -> a*h + b; section 4.1: the serial loop).
 */
ORACLE_API void oracle_scan_ab(const double* a, const double* b, double h0, int64_t L, double* h) {
  double s = h0;
  for (int64_t t = 0; t < L; ++t) {
#if ORACLE_MUTATION == 1
    s = a[t] * (s + b[t]); /* planted: input absorbed before the decay */
#else
    s = a[t] * s + b[t];
#endif
    h[t] = s;
  }
}

/* softplus(v) = log(1 + e^v), written in the overflow-free form
 * max(v, 0) + log1p(exp(-|v|)). */
ORACLE_API double oracle_softplus(double v) {
  double m = v > 0.0 ? v : 0.0;
  return m + log1p(exp(-fabs(v)));
}

typedef struct {
  const double *x, *delta, *A_log, *B, *C, *D, *h0;
  const int32_t* valid_len;
  int64_t nb, L, nd, N;
  int softplus, clamp;
  double dmin, dmax;
  const double* delta_bias; /* [nd] or NULL */
  const double* z;          /* [nb, L, nd] or NULL */
  double* chunk_states;     /* [nb, nchunks, nd, N] or NULL (full runs only) */
  int64_t chunk_len;
} problem_t;

/* silu(v) = v * sigmoid(v) = v / (1 + e^-v). */
ORACLE_API double oracle_silu(double v) { return v / (1.0 + exp(-v)); }

/* One (b, d) row over all L steps.  y_out[t] for t in [0, L) with stride
 * y_stride; h_out[n] for n in [0, N). */
static void scan_row(const problem_t* p, int64_t b, int64_t d, double* y_out, int64_t y_stride, double* h_out,
                     double* h /* scratch, N */, double* A /* scratch, N */, double* cs_out /* chunk states or NULL */) {
  const int64_t L = p->L, N = p->N, nd = p->nd;
  int64_t len = L;
  if (p->valid_len) {
    int64_t v = p->valid_len[b];
    len = v < 0 ? 0 : (v > L ? L : v);
  }
  for (int64_t n = 0; n < N; ++n) {
#if ORACLE_MUTATION == 3
    A[n] = exp(p->A_log[d * N + n]); /* planted: sign of A dropped */
#else
    A[n] = -exp(p->A_log[d * N + n]);
#endif
    h[n] = p->h0 ? p->h0[(b * nd + d) * N + n] : 0.0;
  }
  const double dskip = p->D ? p->D[d] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    if (t >= len) {
#if ORACLE_MUTATION == 7
      for (int64_t n = 0; n < N; ++n) h[n] = 0.0; /* planted: padding resets the state */
#endif
      y_out[t * y_stride] = 0.0;
      if (cs_out && ((t + 1) % p->chunk_len == 0 || t == L - 1))
        for (int64_t n = 0; n < N; ++n) cs_out[(t / p->chunk_len) * p->nd * N + n] = h[n];
      continue;
    }
    const int64_t i = (b * L + t) * nd + d;
    const double xt = p->x[i];
    double dt = p->delta[i];
#if ORACLE_MUTATION == 10
#if ORACLE_MUTATION != 5
    if (p->softplus) dt = oracle_softplus(dt);
#endif
    if (p->delta_bias) dt += p->delta_bias[d]; /* planted: bias added after softplus */
#else
    if (p->delta_bias) dt += p->delta_bias[d];
#if ORACLE_MUTATION != 5
    if (p->softplus) dt = oracle_softplus(dt);
#endif
#endif
    if (p->clamp) {
      if (dt < p->dmin) dt = p->dmin;
      if (dt > p->dmax) dt = p->dmax;
    }
    const double* Bt = p->B + (b * L + t) * N;
    const double* Ct = p->C + (b * L + t) * N;
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double abar = exp(dt * A[n]);
#if ORACLE_MUTATION == 6
      const double bx = Bt[n] * xt; /* planted: Delta missing from the input term */
#elif ORACLE_MUTATION == 8
      const double bx = dt * Ct[n] * xt; /* planted: B and C swapped */
#else
      const double bx = dt * Bt[n] * xt;
#endif
#if ORACLE_MUTATION == 2
      acc += Ct[n] * h[n]; /* planted: readout before the update */
      h[n] = abar * h[n] + bx;
#elif ORACLE_MUTATION == 1
      h[n] = abar * (h[n] + bx);
      acc += Ct[n] * h[n];
#else
      h[n] = abar * h[n] + bx;
      acc += Ct[n] * h[n];
#endif
    }
#if ORACLE_MUTATION == 4
    double yt = acc; /* planted: skip term dropped */
#else
    double yt = acc + dskip * xt;
#endif
#if ORACLE_MUTATION == 9
    if (p->z) yt = acc * oracle_silu(p->z[i]) + dskip * xt; /* planted: gate before the skip term */
#else
    if (p->z) yt *= oracle_silu(p->z[i]);
#endif
    y_out[t * y_stride] = yt;
    if (cs_out && ((t + 1) % p->chunk_len == 0 || t == L - 1))
      for (int64_t n = 0; n < N; ++n) cs_out[(t / p->chunk_len) * p->nd * N + n] = h[n];
  }
  if (h_out)
    for (int64_t n = 0; n < N; ++n) h_out[n] = h[n];
}

typedef struct {
  const problem_t* p;
  const int64_t* rb;  /* NULL: all rows in (b, d) order */
  const int64_t* rd;
  int64_t nrows;
  double* y;          /* full [B,L,D] when rb == NULL, else [nrows, L] */
  double* h_last;     /* full [B,D,N] when rb == NULL, else [nrows, N]; may be NULL */
  int64_t next;       /* static partition: worker k takes rows k, k+nthreads, ... */
  int nthreads;
  int status;
} job_t;

typedef struct {
  job_t* job;
  int k;
} worker_arg_t;

static void* worker(void* argp) {
  worker_arg_t* wa = (worker_arg_t*)argp;
  job_t* j = wa->job;
  const problem_t* p = j->p;
  double* scratch = (double*)malloc(sizeof(double) * 2 * (size_t)(p->N > 0 ? p->N : 1));
  if (!scratch) {
    j->status = -1;
    return NULL;
  }
  for (int64_t r = wa->k; r < j->nrows; r += j->nthreads) {
    int64_t b, d;
    double *yo, *ho;
    int64_t ystride;
    if (j->rb) {
      b = j->rb[r];
#if ORACLE_MUTATION == 14
      d = j->rd[r > 0 ? r - 1 : 0];
#else
      d = j->rd[r];
#endif
      yo = j->y + r * p->L;
      ystride = 1;
      ho = j->h_last ? j->h_last + r * p->N : NULL;
    } else {
      b = r / p->nd;
      d = r % p->nd;
      yo = j->y + b * p->L * p->nd + d;
      ystride = p->nd;
      ho = j->h_last ? j->h_last + (b * p->nd + d) * p->N : NULL;
    }
    double* cs = NULL;
    if (!j->rb && p->chunk_states) {
      const int64_t nch = (p->L + p->chunk_len - 1) / p->chunk_len;
      cs = p->chunk_states + (b * nch * p->nd + d) * p->N;
    }
    scan_row(p, b, d, yo, ystride, ho, scratch, scratch + p->N, cs);
  }
  free(scratch);
  return NULL;
}

static int run_job(job_t* job, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > job->nrows) nthreads = job->nrows > 0 ? (int)job->nrows : 1;
  job->nthreads = nthreads;
  job->status = 0;
  pthread_t tid[256];
  worker_arg_t args[256];
  int started = 0;
  for (int k = 0; k < nthreads; ++k) {
    args[k].job = job;
    args[k].k = k;
    if (k == 0) continue; /* worker 0 runs on the calling thread */
    if (pthread_create(&tid[k], NULL, worker, &args[k]) != 0) {
      job->status = -2;
      break;
    }
    started = k;
  }
  worker(&args[0]);
  for (int k = 1; k <= started; ++k) pthread_join(tid[k], NULL);
  /* rows of workers that failed to start are done serially here */
  if (job->status == -2) {
    job->status = 0;
    for (int k = started + 1; k < nthreads; ++k) worker(&args[k]);
  }
  return job->status;
}

/* Full forward with the optional extras: delta_bias [nd] (added to the raw
 * delta before softplus), z [nb, L, nd] (output gate y * silu(z)), and
 * chunk_states [nb, ceil(L / chunk_len), nd, N] (state after the last step of
 * each chunk, the last chunk possibly shorter).  Any of them may be NULL. */
ORACLE_API int oracle_selective_scan_ex(const double* x, const double* delta, const double* A_log, const double* B,
                                        const double* C, const double* D, const int32_t* valid_len,
                                        const double* h0, int64_t nb, int64_t L, int64_t nd, int64_t N, int softplus,
                                        int clamp, double dmin, double dmax, const double* delta_bias,
                                        const double* z, double* chunk_states, int64_t chunk_len, double* y,
                                        double* h_last, int nthreads) {
  if (nb < 0 || L < 0 || nd < 0 || N < 1 || !y) return -3;
  if (L > 0 && (!x || !delta || !B || !C)) return -3;
  if (!A_log) return -3;
  if (chunk_states && chunk_len < 1) return -3;
  problem_t p = {x, delta, A_log, B, C, D, h0, valid_len, nb, L, nd, N, softplus, clamp, dmin, dmax,
                 delta_bias, z, chunk_states, chunk_len};
  job_t job;
  memset(&job, 0, sizeof(job));
  job.p = &p;
  job.nrows = nb * nd;
  job.y = y;
  job.h_last = h_last;
  return run_job(&job, nthreads);
}

/* Full forward over every (b, d) row.  Layouts (row-major, contiguous):
 * x, delta, y: [nb, L, nd]; A_log: [nd, N]; B, C: [nb, L, N]; D: [nd] or NULL;
 * valid_len: [nb] or NULL (all L); h0: [nb, nd, N] or NULL (zeros);
 * h_last: [nb, nd, N] or NULL.  Returns 0, or a negative value on bad
 * arguments or failed allocation. */
ORACLE_API int oracle_selective_scan(const double* x, const double* delta, const double* A_log, const double* B,
                                     const double* C, const double* D, const int32_t* valid_len, const double* h0,
                                     int64_t nb, int64_t L, int64_t nd, int64_t N, int softplus, int clamp,
                                     double dmin, double dmax, double* y, double* h_last, int nthreads) {
  if (nb < 0 || L < 0 || nd < 0 || N < 1 || !y) return -3;
  if (L > 0 && (!x || !delta || !B || !C)) return -3;
  if (!A_log) return -3;
  problem_t p = {x, delta, A_log, B, C, D, h0, valid_len, nb, L, nd, N, softplus, clamp, dmin, dmax,
                 NULL, NULL, NULL, 1};
  job_t job;
  memset(&job, 0, sizeof(job));
  job.p = &p;
  job.nrows = nb * nd;
  job.y = y;
  job.h_last = h_last;
  return run_job(&job, nthreads);
}

/* The same forward restricted to the listed (row_b[r], row_d[r]) rows:
 * y_rows [nrows, L] and h_rows [nrows, N] (h_rows may be NULL). */
ORACLE_API int oracle_selective_scan_rows(const double* x, const double* delta, const double* A_log, const double* B,
                                          const double* C, const double* D, const int32_t* valid_len,
                                          const double* h0, int64_t nb, int64_t L, int64_t nd, int64_t N,
                                          int softplus, int clamp, double dmin, double dmax,
                                          const double* delta_bias, const double* z, const int64_t* row_b,
                                          const int64_t* row_d, int64_t nrows, double* y_rows, double* h_rows,
                                          int nthreads) {
  if (nb < 0 || L < 0 || nd < 0 || N < 1 || !y_rows || nrows < 0 || !row_b || !row_d) return -3;
  if (L > 0 && (!x || !delta || !B || !C)) return -3;
  if (!A_log) return -3;
  for (int64_t r = 0; r < nrows; ++r)
    if (row_b[r] < 0 || row_b[r] >= nb || row_d[r] < 0 || row_d[r] >= nd) return -3;
  problem_t p = {x, delta, A_log, B, C, D, h0, valid_len, nb, L, nd, N, softplus, clamp, dmin, dmax,
                 delta_bias, z, NULL, 1};
  job_t job;
  memset(&job, 0, sizeof(job));
  job.p = &p;
  job.rb = row_b;
  job.rd = row_d;
  job.nrows = nrows;
  job.y = y_rows;
  job.h_last = h_rows;
  return run_job(&job, nthreads);
}

/* ---- backward --------------------------------------------------------
 *
 * Gradients of the forward above by reverse-mode differentiation of the plain
 * serial loop (the recomputation from saved states the pwwt.cn article,
 * section 3.4, describes, here with the full per-step history of one row kept
 * in memory, which the oracle can afford).  With the loss
 *     L = sum dy * y + sum dh_last * h_last
 * the adjoint of the state after step t is
 *     g_t = dh_last (t = last valid step) + dypre_t * C_t + Abar_{t+1} g_{t+1},
 * where dypre_t = dy_t * silu(z_t) with the gate (else dy_t), and per step:
 *     dC[b,t,n] += dypre_t h_t[n]                 dB[b,t,n] += g_t[n] Delta_t x_t
 *     dx_t = dypre_t D + sum_n g_t[n] Delta_t B_t[n]
 *     dDelta_t = sum_n g_t[n] (B_t[n] x_t + h_{t-1}[n] Abar_t[n] A[n])
 *     dA[n] += g_t[n] h_{t-1}[n] Abar_t[n] Delta_t,  dA_log = dA * A
 *     dD += dypre_t x_t,   dz_t = dy_t ypre_t silu'(z_t)
 * and dDelta_raw = dDelta * [clip inactive] * sigmoid(raw + bias) (softplus'),
 * ddelta_bias = sum over (b, t) of dDelta_raw, dh0 = Abar_0 g_0 (the adjoint of
 * the state before step 0).  Padded steps contribute nothing and get zero
 * gradients.  The clip passes the gradient where dmin <= softplus <= dmax.
 */

typedef struct {
  const problem_t* p;
  const double* dy;      /* [nb, L, nd] */
  const double* dh_last; /* [nb, nd, N] or NULL */
  double *dx, *ddelta, *dB, *dC, *dz, *dh0; /* full tensors (dz, dh0 may be NULL) */
  double *dA_part, *dD_part, *dbias_part;   /* per batch row: [nb, nd, N], [nb, nd], [nb, nd] */
  int nthreads;
  int status;
} bwd_job_t;

typedef struct {
  bwd_job_t* job;
  int k;
} bwd_arg_t;

static double sigmoid(double v) { return v >= 0.0 ? 1.0 / (1.0 + exp(-v)) : exp(v) / (1.0 + exp(v)); }

/* One (b, d) row: forward with the full history, then the reverse sweep. */
static void bwd_row(bwd_job_t* j, int64_t b, int64_t d, double* hist /* (L+1) * N */, double* abar /* L * N */,
                    double* dlt /* L */, double* dfac /* L */, double* A /* N */, double* g /* N */) {
  const problem_t* p = j->p;
  const int64_t L = p->L, N = p->N, nd = p->nd;
  int64_t len = L;
  if (p->valid_len) {
    int64_t v = p->valid_len[b];
    len = v < 0 ? 0 : (v > L ? L : v);
  }
  for (int64_t n = 0; n < N; ++n) {
    A[n] = -exp(p->A_log[d * N + n]);
    hist[n] = p->h0 ? p->h0[(b * nd + d) * N + n] : 0.0;
  }
  /* forward: hist[(t + 1) * N + n] = h_t[n] */
  for (int64_t t = 0; t < len; ++t) {
    const int64_t i = (b * L + t) * nd + d;
    double raw = p->delta[i];
    if (p->delta_bias) raw += p->delta_bias[d];
    double dt = p->softplus ? oracle_softplus(raw) : raw;
    double fac = p->softplus ? sigmoid(raw) : 1.0;
#if ORACLE_MUTATION == 13
    fac = 1.0; /* planted: softplus derivative missing */
#endif
    if (p->clamp) {
      if (dt < p->dmin || dt > p->dmax) fac = 0.0;
      if (dt < p->dmin) dt = p->dmin;
      if (dt > p->dmax) dt = p->dmax;
    }
    dlt[t] = dt;
    dfac[t] = fac;
    const double xt = p->x[i];
    const double* Bt = p->B + (b * L + t) * N;
    for (int64_t n = 0; n < N; ++n) {
      const double a = exp(dt * A[n]);
      abar[t * N + n] = a;
      hist[(t + 1) * N + n] = a * hist[t * N + n] + dt * Bt[n] * xt;
    }
  }
  /* reverse */
  for (int64_t n = 0; n < N; ++n) g[n] = j->dh_last ? j->dh_last[(b * nd + d) * N + n] : 0.0;
  const double dskip = p->D ? p->D[d] : 0.0;
  double dD = 0.0, dbias = 0.0;
  for (int64_t t = L - 1; t >= 0; --t) {
    const int64_t i = (b * L + t) * nd + d;
    if (t >= len) {
      j->dx[i] = 0.0;
      j->ddelta[i] = 0.0;
      if (j->dz) j->dz[i] = 0.0;
      continue;
    }
    const double xt = p->x[i], dt = dlt[t];
    const double* Bt = p->B + (b * L + t) * N;
    const double* Ct = p->C + (b * L + t) * N;
    const double* ht = hist + (t + 1) * N;
    const double* hp = hist + t * N;
    double dyp = j->dy[i];
    if (p->z) {
      const double zt = p->z[i], sg = sigmoid(zt);
      double ypre = dskip * xt;
      for (int64_t n = 0; n < N; ++n) ypre += Ct[n] * ht[n];
      j->dz[i] = j->dy[i] * ypre * sg * (1.0 + zt * (1.0 - sg));
      dyp = j->dy[i] * zt * sg;
    }
    double dx = dyp * dskip, ddt = 0.0;
    dD += dyp * xt;
    for (int64_t n = 0; n < N; ++n) {
      g[n] += dyp * Ct[n];
      j->dC[(b * L + t) * N + n] += dyp * ht[n];
      const double a = abar[t * N + n];
      const double da = g[n] * hp[n];
      ddt += g[n] * Bt[n] * xt + da * a * A[n];
      dx += g[n] * dt * Bt[n];
      j->dB[(b * L + t) * N + n] += g[n] * dt * xt;
#if ORACLE_MUTATION == 12
      j->dA_part[(b * nd + d) * N + n] += da * a; /* planted: dA without the Delta factor */
#else
      j->dA_part[(b * nd + d) * N + n] += da * a * dt;
#endif
#if ORACLE_MUTATION != 11
      g[n] *= a;
#endif
      /* (mutation 11 plants an adjoint that is not decayed through the step) */
    }
    j->dx[i] = dx;
    const double draw = ddt * dfac[t];
    j->ddelta[i] = draw;
    dbias += draw;
  }
  if (j->dh0)
    for (int64_t n = 0; n < N; ++n) j->dh0[(b * nd + d) * N + n] = g[n];
  for (int64_t n = 0; n < N; ++n) j->dA_part[(b * nd + d) * N + n] *= A[n];
  j->dD_part[b * nd + d] = dD;
  j->dbias_part[b * nd + d] = dbias;
}

static void* bwd_worker(void* argp) {
  bwd_arg_t* wa = (bwd_arg_t*)argp;
  bwd_job_t* j = wa->job;
  const problem_t* p = j->p;
  const int64_t L = p->L, N = p->N;
  double* buf = (double*)malloc(sizeof(double) * (size_t)((L + 1) * N + L * N + 2 * L + 2 * N + 4));
  if (!buf) {
    j->status = -1;
    return NULL;
  }
  double* hist = buf;
  double* abar = hist + (L + 1) * N;
  double* dlt = abar + L * N;
  double* dfac = dlt + L;
  double* A = dfac + L;
  double* g = A + N;
  /* batch rows are dealt to workers; one worker owns every channel of its
   * rows, so the sums over channels (dB, dC) need no cross-thread reduction */
  for (int64_t b = wa->k; b < p->nb; b += j->nthreads)
    for (int64_t d = 0; d < p->nd; ++d) bwd_row(j, b, d, hist, abar, dlt, dfac, A, g);
  free(buf);
  return NULL;
}

/* Backward of oracle_selective_scan_ex (same inputs and flags) for the loss
 * sum dy*y + sum dh_last*h_last.  Outputs (all fp64, overwritten):
 * dx, ddelta (w.r.t. the raw delta) [nb, L, nd]; dA_log [nd, N]; dB, dC
 * [nb, L, N]; dD [nd] (may be NULL); ddelta_bias [nd] (may be NULL); dz
 * [nb, L, nd] (needed when z is given, else ignored); dh0 [nb, nd, N] (may be
 * NULL).  Reductions over batch rows run in row order, so the result does not
 * depend on nthreads. */
ORACLE_API int oracle_selective_scan_bwd(const double* x, const double* delta, const double* A_log, const double* B,
                                         const double* C, const double* D, const int32_t* valid_len,
                                         const double* h0, int64_t nb, int64_t L, int64_t nd, int64_t N,
                                         int softplus, int clamp, double dmin, double dmax,
                                         const double* delta_bias, const double* z, const double* dy,
                                         const double* dh_last, double* dx, double* ddelta, double* dA_log,
                                         double* dB, double* dC, double* dD, double* ddelta_bias, double* dz,
                                         double* dh0, int nthreads) {
  if (nb < 0 || L < 0 || nd < 0 || N < 1 || !A_log || !dA_log) return -3;
  if (L > 0 && (!x || !delta || !B || !C || !dy || !dx || !ddelta || !dB || !dC)) return -3;
  if (z && !dz) return -3;
  problem_t p = {x, delta, A_log, B, C, D, h0, valid_len, nb, L, nd, N, softplus, clamp, dmin, dmax,
                 delta_bias, z, NULL, 1};
  double* part = (double*)calloc((size_t)(nb * nd * N + 2 * nb * nd + 1), sizeof(double));
  if (!part) return -1;
  if (L > 0) {
    memset(dB, 0, sizeof(double) * (size_t)(nb * L * N));
    memset(dC, 0, sizeof(double) * (size_t)(nb * L * N));
  }
  bwd_job_t job = {&p, dy, dh_last, dx, ddelta, dB, dC, z ? dz : NULL, dh0,
                   part, part + nb * nd * N, part + nb * nd * N + nb * nd, 1, 0};
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > nb) nthreads = nb > 0 ? (int)nb : 1;
  job.nthreads = nthreads;
  pthread_t tid[256];
  bwd_arg_t args[256];
  int started = 0;
  for (int k = 0; k < nthreads; ++k) {
    args[k].job = &job;
    args[k].k = k;
    if (k == 0) continue;
    if (pthread_create(&tid[k], NULL, bwd_worker, &args[k]) != 0) {
      job.status = -2;
      break;
    }
    started = k;
  }
  bwd_worker(&args[0]);
  for (int k = 1; k <= started; ++k) pthread_join(tid[k], NULL);
  if (job.status == -2) {
    job.status = 0;
    for (int k = started + 1; k < nthreads; ++k) bwd_worker(&args[k]);
  }
  if (job.status == 0) {
    for (int64_t i = 0; i < nd * N; ++i) {
      double s = 0.0;
      for (int64_t b = 0; b < nb; ++b) s += job.dA_part[b * nd * N + i];
      dA_log[i] = s;
    }
    for (int64_t d = 0; d < nd; ++d) {
      double s = 0.0, sb = 0.0;
      for (int64_t b = 0; b < nb; ++b) {
        s += job.dD_part[b * nd + d];
        sb += job.dbias_part[b * nd + d];
      }
      if (dD) dD[d] = s;
      if (ddelta_bias) ddelta_bias[d] = sb;
    }
  }
  free(part);
  return job.status;
}

ORACLE_API int oracle_mutation_id(void) { return ORACLE_MUTATION; }
