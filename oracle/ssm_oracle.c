/*
 * ssm_oracle.c -- plain fp64 CPU oracle of the selective-SSM scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the CPU-baseline
 * leg of bench.py may load this library.  It shares no code, header, table or
 * helper with the HIP path, and the HIP path never calls it.
 *
 * What it computes (Mamba, Gu & Dao, arXiv 2312.00752, as the reading guide on
 * xyznot.com summarises it):
 *   - the discrete linear recurrence h_t = Abar_t h_{t-1} + Bbar_t x_t,
 *     y_t = C_t h_t ("Yöntem" section, discretisation equations), with
 *     Abar_t = exp(delta_t * A) (zero-order hold) and, as in the sequential
 *     loop quoted on the mamba-minimal news page (ja.news.hada.io, Hacker News
 *     comments), the input term deltaB_u = delta_t * B_t * u_t;
 *   - the selection mechanism: B_t, C_t and delta_t vary per token, with
 *     delta_t = softplus(parameter + s(x_t)) ("Seçim Mekanizması (S6)"
 *     section, delta equation), here softplus(delta_raw + delta_bias);
 *   - the output skip D*u and the multiplicative SiLU gate of the Mamba block
 *     ("Temel Fikirler": gated block combining H3 and a SwiGLU-style MLP);
 *   - the single-token recurrent update used in generation (reading guide,
 *     "Sorular", the question on KV caches: a fixed D x N state per layer);
 *   - the gradient of the forward map (the reading guide's "Donanım Duyarlı
 *     Durum Genişletme" section recomputes states in the backward pass; here
 *     the plain reverse-mode derivative of the recurrence, with every state
 *     of a channel kept in memory).
 *
 * Options (the flags argument of the *_ex entry points; 0 = the above):
 *   ORACLE_ZOH (1): the exact zero-order-hold input term of the reading
 *     guide's "Yöntem" discretisation, Bbar = (dt A)^-1 (exp(dt A) - 1) dt B,
 *     so the input coefficient is expm1(dt A) / A (= dt when A = 0) instead
 *     of dt;
 *   ORACLE_REVERSE (2): the recurrence runs from the last step to the first
 *     (the backward direction of a bidirectional mixer such as Hydra, listed
 *     on the zenn.dev reading list); h0 is the state before the last step
 *     and chunk slot k is the state before scan step k*chunk_len, i.e. before
 *     time L-1-k*chunk_len;
 *   ORACLE_DELTA_PER_TOKEN (4): delta is (B,L), one raw step size per token
 *     shared by every channel (the reading guide's "Seçim Mekanizması (S6)"
 *     delta equation broadcasts one value per token over D); ddelta is then
 *     (B,L), the sum over channels.
 *
 * The causal depthwise convolution of the Mamba block (the Italian overview
 * article, "Iniziare con Mamba": the block applies a causal Conv1d before the
 * selective SSM; reading guide, "Temel terimler", Mamba block) is a separate
 * pair of functions, oracle_conv1d_silu and oracle_conv1d_silu_bwd: per
 * channel a width-K filter over time with a bias, then SiLU.
 *
 * Everything is fp64.  Channels (b, d) are independent recurrences; threads
 * split the channels and never reorder the arithmetic inside one channel.
 * Reductions over channels (dB, dC, and over (b, t) for dA, dD, dbias) are
 * accumulated per thread and summed in thread order.
 *
 * Layouts (row-major, contiguous): u, delta, z, y, dy, du, ddelta, dz (B,L,D);
 * Bm, Cm, dB, dC (B,L,N); A, dA (D,N); Dskip, delta_bias, dD, dbias (D);
 * h0, h_final, dh_final, dh0, state (B,D,N); chunk_states (B,K,D,N) with
 * K = ceil(L / chunk_len), slot k = state before step k*chunk_len.
 * Optional inputs are NULL; NULL Dskip/delta_bias/h0 mean zeros, NULL z means
 * no gate.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* softplus(x) = log(1 + e^x), written so that neither branch overflows. */
double oracle_softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

/* logistic sigmoid; for very negative x, exp(-x) = inf and the result is 0. */
double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

double oracle_silu(double x) { return x * oracle_sigmoid(x); }

#define ORACLE_ZOH 1
#define ORACLE_REVERSE 2
#define ORACLE_DELTA_PER_TOKEN 4

typedef struct {
  int64_t B, L, D, N;
  int flags;
  const double *u, *delta, *A, *Bm, *Cm, *Dskip, *z, *bias, *h0;
  int softplus;
  /* forward outputs */
  double *y, *h_final, *chunk_states;
  int64_t chunk_len;
  /* backward */
  const double *dy, *dh_final;
  double *du, *ddelta, *dz, *dh0;
  /* per-thread partial sums, [thread][...] */
  double *dA_part, *dB_part, *dC_part, *dD_part, *dbias_part, *ddelta_part;
  int nthreads;
} job_t;

typedef struct {
  job_t *job;
  int tid;
} targ_t;

/* Memory row of scan step s. */
static int64_t row_of(const job_t *j, int64_t s) { return (j->flags & ORACLE_REVERSE) ? j->L - 1 - s : s; }

/* Index of the raw step size of (b, t, d). */
static int64_t delta_index(const job_t *j, int64_t b, int64_t t, int64_t d) {
  return (j->flags & ORACLE_DELTA_PER_TOKEN) ? b * j->L + t : (b * j->L + t) * j->D + d;
}

static double step_size(const job_t *j, int64_t b, int64_t t, int64_t d, double *s_out) {
  double s = j->delta[delta_index(j, b, t, d)] + (j->bias ? j->bias[d] : 0.0);
  if (s_out) *s_out = s;
  return j->softplus ? oracle_softplus(s) : s;
}

/* Input coefficient: dt (first-order form) or, with ORACLE_ZOH, the exact
 * zero-order hold expm1(dt A) / A (limit dt as A -> 0). */
static double in_coef(const job_t *j, double dt, double A) {
  if (!(j->flags & ORACLE_ZOH)) return dt;
  return A == 0.0 ? dt : expm1(dt * A) / A;
}

/* d/dA of expm1(dt A) / A = dt^2 psi(dt A), psi(x) = (x e^x - e^x + 1) / x^2
 * = sum_k x^k (k+1)/(k+2)!; the series is used where the closed form cancels. */
static double zoh_dcoef_dA(double dt, double A) {
  const double x = dt * A;
  if (fabs(x) < 1e-2) {
    const double psi = 1.0 / 2 + x * (1.0 / 3 + x * (1.0 / 8 + x * (1.0 / 30 + x * (1.0 / 144 + x * (1.0 / 840 + x / 5760.0)))));
    return dt * dt * psi;
  }
  return (dt * exp(x) - expm1(x) / A) / A;
}

/* ---- forward ------------------------------------------------------------ */

static void fwd_channel(const job_t *j, int64_t b, int64_t d, double *h) {
  const int64_t L = j->L, D = j->D, N = j->N;
  for (int64_t n = 0; n < N; ++n) h[n] = j->h0 ? j->h0[(b * D + d) * N + n] : 0.0;
  const int64_t K = j->chunk_states ? (L + j->chunk_len - 1) / j->chunk_len : 0;
  for (int64_t st = 0; st < L; ++st) { /* scan step st at memory row t */
    const int64_t t = row_of(j, st);
    if (j->chunk_states && st % j->chunk_len == 0) {
      int64_t k = st / j->chunk_len;
      for (int64_t n = 0; n < N; ++n) j->chunk_states[((b * K + k) * D + d) * N + n] = h[n];
    }
    const int64_t idx = (b * L + t) * D + d;
    const double dt = step_size(j, b, t, d, NULL);
    const double x = j->u[idx];
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double An = j->A[d * N + n];
      const double a = exp(dt * An);
      h[n] = a * h[n] + in_coef(j, dt, An) * j->Bm[(b * L + t) * N + n] * x;
      acc += j->Cm[(b * L + t) * N + n] * h[n];
    }
    if (j->Dskip) acc += j->Dskip[d] * x;
    j->y[idx] = j->z ? acc * oracle_silu(j->z[idx]) : acc;
  }
  if (j->h_final)
    for (int64_t n = 0; n < N; ++n) j->h_final[(b * D + d) * N + n] = h[n];
}

static void *fwd_worker(void *p) {
  targ_t *a = (targ_t *)p;
  const job_t *j = a->job;
  double *h = (double *)malloc(sizeof(double) * (size_t)j->N);
  for (int64_t c = a->tid; c < j->B * j->D; c += j->nthreads) fwd_channel(j, c / j->D, c % j->D, h);
  free(h);
  return NULL;
}

/* ---- backward ----------------------------------------------------------- */

static void bwd_channel(const job_t *j, int tid, int64_t b, int64_t d, double *hist, double *lam) {
  const int64_t L = j->L, D = j->D, N = j->N;
  /* hist[(st+1)*N + n] = state after scan step st, hist[n] = the initial state. */
  for (int64_t n = 0; n < N; ++n) hist[n] = j->h0 ? j->h0[(b * D + d) * N + n] : 0.0;
  for (int64_t st = 0; st < L; ++st) {
    const int64_t t = row_of(j, st);
    const int64_t idx = (b * L + t) * D + d;
    const double dt = step_size(j, b, t, d, NULL);
    for (int64_t n = 0; n < N; ++n) {
      const double An = j->A[d * N + n];
      const double a = exp(dt * An);
      hist[(st + 1) * N + n] =
          a * hist[st * N + n] + in_coef(j, dt, An) * j->Bm[(b * L + t) * N + n] * j->u[idx];
    }
  }
  double *dA = j->dA_part + (size_t)tid * D * N;
  double *dB = j->dB_part + (size_t)tid * j->B * L * N;
  double *dC = j->dC_part + (size_t)tid * j->B * L * N;
  /* lam[n] holds dLoss/dh_t coming from later steps (a_{t+1} * lambda_{t+1}),
   * or dLoss/dh_final at the last step. */
  for (int64_t n = 0; n < N; ++n) lam[n] = j->dh_final ? j->dh_final[(b * D + d) * N + n] : 0.0;
  double dDsum = 0.0, dbias_sum = 0.0;
  const int zoh = (j->flags & ORACLE_ZOH) != 0;
  for (int64_t st = L - 1; st >= 0; --st) {
    const int64_t t = row_of(j, st);
    const int64_t idx = (b * L + t) * D + d;
    double s;
    const double dt = step_size(j, b, t, d, &s);
    const double x = j->u[idx];
    const double g = j->dy[idx];
    double e = g; /* dLoss/d(pre-gate output) */
    if (j->z) {
      const double zz = j->z[idx];
      const double sz = oracle_sigmoid(zz);
      double pre = 0.0; /* sum_n C h + D u at this step */
      for (int64_t n = 0; n < N; ++n) pre += j->Cm[(b * L + t) * N + n] * hist[(st + 1) * N + n];
      if (j->Dskip) pre += j->Dskip[d] * x;
      e = g * zz * sz;
      j->dz[idx] = g * pre * sz * (1.0 + zz * (1.0 - sz));
    }
    double du = j->Dskip ? j->Dskip[d] * e : 0.0;
    double ddt = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double Bv = j->Bm[(b * L + t) * N + n];
      const double Cv = j->Cm[(b * L + t) * N + n];
      const double An = j->A[d * N + n];
      const double a = exp(dt * An);
      const double cf = in_coef(j, dt, An);
      const double hprev = hist[st * N + n];
      const double lt = e * Cv + lam[n]; /* lambda at this step */
      dC[(b * L + t) * N + n] += e * hist[(st + 1) * N + n];
      dB[(b * L + t) * N + n] += lt * cf * x;
      du += lt * cf * Bv;
      /* d coef / d dt is 1 (first-order form) or exp(dt A) (zero-order hold) */
      ddt += lt * (hprev * a * An + Bv * x * (zoh ? a : 1.0));
      dA[d * N + n] += lt * hprev * a * dt + (zoh ? lt * Bv * x * zoh_dcoef_dA(dt, An) : 0.0);
      lam[n] = a * lt;
    }
    j->du[idx] = du;
    const double draw = j->softplus ? ddt * oracle_sigmoid(s) : ddt;
    if (j->flags & ORACLE_DELTA_PER_TOKEN)
      j->ddelta_part[(size_t)tid * j->B * L + b * L + t] += draw;
    else
      j->ddelta[idx] = draw;
    dbias_sum += draw;
    dDsum += e * x;
  }
  j->dD_part[(size_t)tid * D + d] += dDsum;
  j->dbias_part[(size_t)tid * D + d] += dbias_sum;
  if (j->dh0)
    for (int64_t n = 0; n < N; ++n) j->dh0[(b * D + d) * N + n] = lam[n];
}

static void *bwd_worker(void *p) {
  targ_t *a = (targ_t *)p;
  const job_t *j = a->job;
  double *hist = (double *)malloc(sizeof(double) * (size_t)(j->L + 1) * j->N);
  double *lam = (double *)malloc(sizeof(double) * (size_t)j->N);
  for (int64_t c = a->tid; c < j->B * j->D; c += j->nthreads)
    bwd_channel(j, a->tid, c / j->D, c % j->D, hist, lam);
  free(hist);
  free(lam);
  return NULL;
}

static void run_threads(job_t *j, void *(*fn)(void *)) {
  if (j->nthreads < 1) j->nthreads = 1;
  if (j->nthreads > j->B * j->D) j->nthreads = (int)(j->B * j->D);
  if (j->nthreads < 1) j->nthreads = 1;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)j->nthreads);
  targ_t *args = (targ_t *)malloc(sizeof(targ_t) * (size_t)j->nthreads);
  for (int i = 0; i < j->nthreads; ++i) {
    args[i].job = j;
    args[i].tid = i;
    pthread_create(&th[i], NULL, fn, &args[i]);
  }
  for (int i = 0; i < j->nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(args);
}

/* Returns 0 on success, -1 on bad sizes or flags. */
int oracle_scan_fwd_ex(int64_t B, int64_t L, int64_t D, int64_t N, const double *u,
                       const double *delta, const double *A, const double *Bm, const double *Cm,
                       const double *Dskip, const double *z, const double *delta_bias, int softplus,
                       const double *h0, double *y, double *h_final, int64_t chunk_len,
                       double *chunk_states, int nthreads, int flags) {
  if (B < 1 || L < 1 || D < 1 || N < 1) return -1;
  if (chunk_states && chunk_len < 1) return -1;
  if (flags & ~(ORACLE_ZOH | ORACLE_REVERSE | ORACLE_DELTA_PER_TOKEN)) return -1;
  job_t j;
  memset(&j, 0, sizeof(j));
  j.B = B, j.L = L, j.D = D, j.N = N, j.flags = flags;
  j.u = u, j.delta = delta, j.A = A, j.Bm = Bm, j.Cm = Cm, j.Dskip = Dskip, j.z = z;
  j.bias = delta_bias, j.h0 = h0, j.softplus = softplus;
  j.y = y, j.h_final = h_final, j.chunk_states = chunk_states, j.chunk_len = chunk_len;
  j.nthreads = nthreads;
  run_threads(&j, fwd_worker);
  return 0;
}

int oracle_scan_fwd(int64_t B, int64_t L, int64_t D, int64_t N, const double *u, const double *delta,
                    const double *A, const double *Bm, const double *Cm, const double *Dskip,
                    const double *z, const double *delta_bias, int softplus, const double *h0,
                    double *y, double *h_final, int64_t chunk_len, double *chunk_states,
                    int nthreads) {
  return oracle_scan_fwd_ex(B, L, D, N, u, delta, A, Bm, Cm, Dskip, z, delta_bias, softplus, h0, y,
                            h_final, chunk_len, chunk_states, nthreads, 0);
}

/* Gradients are overwritten.  dz must be non-NULL iff z is; dD/ddelta_bias/dh0
 * may be NULL (not wanted).  Returns 0 on success, -1 on bad sizes, -2 on
 * allocation failure. */
int oracle_scan_bwd_ex(int64_t B, int64_t L, int64_t D, int64_t N, const double *u,
                       const double *delta, const double *A, const double *Bm, const double *Cm,
                       const double *Dskip, const double *z, const double *delta_bias, int softplus,
                       const double *h0, const double *dy, const double *dh_final, double *du,
                       double *ddelta, double *dA, double *dB, double *dC, double *dD, double *dz,
                       double *ddelta_bias, double *dh0, int nthreads, int flags) {
  if (B < 1 || L < 1 || D < 1 || N < 1) return -1;
  if ((z == NULL) != (dz == NULL)) return -1;
  if (flags & ~(ORACLE_ZOH | ORACLE_REVERSE | ORACLE_DELTA_PER_TOKEN)) return -1;
  job_t j;
  memset(&j, 0, sizeof(j));
  j.B = B, j.L = L, j.D = D, j.N = N, j.flags = flags;
  j.u = u, j.delta = delta, j.A = A, j.Bm = Bm, j.Cm = Cm, j.Dskip = Dskip, j.z = z;
  j.bias = delta_bias, j.h0 = h0, j.softplus = softplus;
  j.dy = dy, j.dh_final = dh_final, j.du = du, j.ddelta = ddelta, j.dz = dz, j.dh0 = dh0;
  j.nthreads = nthreads < 1 ? 1 : nthreads;
  if (j.nthreads > B * D) j.nthreads = (int)(B * D);
  const size_t T = (size_t)j.nthreads;
  j.dA_part = (double *)calloc(T * D * N, sizeof(double));
  j.dB_part = (double *)calloc(T * B * L * N, sizeof(double));
  j.dC_part = (double *)calloc(T * B * L * N, sizeof(double));
  j.dD_part = (double *)calloc(T * D, sizeof(double));
  j.dbias_part = (double *)calloc(T * D, sizeof(double));
  const int per_token = (flags & ORACLE_DELTA_PER_TOKEN) != 0;
  if (per_token) j.ddelta_part = (double *)calloc(T * B * L, sizeof(double));
  int rc = 0;
  if (!j.dA_part || !j.dB_part || !j.dC_part || !j.dD_part || !j.dbias_part ||
      (per_token && !j.ddelta_part)) {
    rc = -2;
  } else {
    run_threads(&j, bwd_worker);
    const size_t nDN = (size_t)D * N, nBLN = (size_t)B * L * N;
    for (size_t i = 0; i < nDN; ++i) {
      double s = 0.0;
      for (size_t k = 0; k < T; ++k) s += j.dA_part[k * nDN + i];
      dA[i] = s;
    }
    for (size_t i = 0; i < nBLN; ++i) {
      double sb = 0.0, sc = 0.0;
      for (size_t k = 0; k < T; ++k) {
        sb += j.dB_part[k * nBLN + i];
        sc += j.dC_part[k * nBLN + i];
      }
      dB[i] = sb;
      dC[i] = sc;
    }
    for (int64_t i = 0; i < D; ++i) {
      double sd = 0.0, sbias = 0.0;
      for (size_t k = 0; k < T; ++k) {
        sd += j.dD_part[k * D + i];
        sbias += j.dbias_part[k * D + i];
      }
      if (dD) dD[i] = sd;
      if (ddelta_bias) ddelta_bias[i] = sbias;
    }
    if (per_token) {
      const size_t nBL = (size_t)B * L;
      for (size_t i = 0; i < nBL; ++i) {
        double sd = 0.0;
        for (size_t k = 0; k < T; ++k) sd += j.ddelta_part[k * nBL + i];
        ddelta[i] = sd;
      }
    }
  }
  free(j.dA_part);
  free(j.dB_part);
  free(j.dC_part);
  free(j.dD_part);
  free(j.dbias_part);
  free(j.ddelta_part);
  return rc;
}

int oracle_scan_bwd(int64_t B, int64_t L, int64_t D, int64_t N, const double *u, const double *delta,
                    const double *A, const double *Bm, const double *Cm, const double *Dskip,
                    const double *z, const double *delta_bias, int softplus, const double *h0,
                    const double *dy, const double *dh_final, double *du, double *ddelta,
                    double *dA, double *dB, double *dC, double *dD, double *dz,
                    double *ddelta_bias, double *dh0, int nthreads) {
  return oracle_scan_bwd_ex(B, L, D, N, u, delta, A, Bm, Cm, Dskip, z, delta_bias, softplus, h0, dy,
                            dh_final, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, nthreads, 0);
}

/* One token of the recurrence, in place on state (B,D,N).  u, delta, z, y are
 * (B,D); Bm, Cm are (B,N).  Same arithmetic as one step of the forward scan. */
int oracle_state_update_ex(int64_t B, int64_t D, int64_t N, double *state, const double *u,
                           const double *delta, const double *A, const double *Bm, const double *Cm,
                           const double *Dskip, const double *z, const double *delta_bias,
                           int softplus, double *y, int flags) {
  if (B < 1 || D < 1 || N < 1) return -1;
  if (flags & ~ORACLE_ZOH) return -1; /* one token: no direction, delta is (B,D) */
  job_t j; /* only for in_coef */
  memset(&j, 0, sizeof(j));
  j.flags = flags;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t d = 0; d < D; ++d) {
      const int64_t idx = b * D + d;
      double s = delta[idx] + (delta_bias ? delta_bias[d] : 0.0);
      const double dt = softplus ? oracle_softplus(s) : s;
      const double x = u[idx];
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        double *h = &state[idx * N + n];
        const double An = A[d * N + n];
        *h = exp(dt * An) * *h + in_coef(&j, dt, An) * Bm[b * N + n] * x;
        acc += Cm[b * N + n] * *h;
      }
      if (Dskip) acc += Dskip[d] * x;
      y[idx] = z ? acc * oracle_silu(z[idx]) : acc;
    }
  }
  return 0;
}

int oracle_state_update(int64_t B, int64_t D, int64_t N, double *state, const double *u,
                        const double *delta, const double *A, const double *Bm, const double *Cm,
                        const double *Dskip, const double *z, const double *delta_bias, int softplus,
                        double *y) {
  return oracle_state_update_ex(B, D, N, state, u, delta, A, Bm, Cm, Dskip, z, delta_bias, softplus, y,
                                0);
}

/* ---- causal depthwise convolution + SiLU --------------------------------- */

/* pre[b,t,d] = bias[d] + sum_{k<K} w[d,k] x[b, t-(K-1)+k, d] (x = 0 before the
 * first step), u = silu(pre).  bias may be NULL (zero); pre or u may be NULL
 * (not wanted).  Layouts: x, pre, u (B,L,D); w (D,K). */
int oracle_conv1d_silu(int64_t B, int64_t L, int64_t D, int64_t K, const double *x, const double *w,
                       const double *bias, double *pre, double *u) {
  if (B < 1 || L < 1 || D < 1 || K < 1) return -1;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t t = 0; t < L; ++t)
      for (int64_t d = 0; d < D; ++d) {
        double acc = bias ? bias[d] : 0.0;
        for (int64_t k = 0; k < K; ++k) {
          const int64_t ts = t - (K - 1) + k;
          if (ts >= 0) acc += w[d * K + k] * x[(b * L + ts) * D + d];
        }
        const int64_t i = (b * L + t) * D + d;
        if (pre) pre[i] = acc;
        if (u) u[i] = oracle_silu(acc);
      }
  return 0;
}

/* Backward of oracle_conv1d_silu given du = dLoss/du:
 *   g = du * silu'(pre), silu'(p) = sigmoid(p) (1 + p (1 - sigmoid(p)))
 *   dx[b,t,d] = sum_k w[d,k] g[b, t+(K-1)-k, d]   (g = 0 past the last step)
 *   dw[d,k]   = sum_{b,t} x[b, t-(K-1)+k, d] g[b,t,d]
 *   dbias[d]  = sum_{b,t} g[b,t,d]
 * dbias may be NULL.  Outputs are overwritten. */
int oracle_conv1d_silu_bwd(int64_t B, int64_t L, int64_t D, int64_t K, const double *x,
                           const double *w, const double *bias, const double *du, double *dx,
                           double *dw, double *dbias) {
  if (B < 1 || L < 1 || D < 1 || K < 1) return -1;
  double *g = (double *)malloc(sizeof(double) * (size_t)(B * L * D));
  if (!g) return -2;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t t = 0; t < L; ++t)
      for (int64_t d = 0; d < D; ++d) {
        double p = bias ? bias[d] : 0.0;
        for (int64_t k = 0; k < K; ++k) {
          const int64_t ts = t - (K - 1) + k;
          if (ts >= 0) p += w[d * K + k] * x[(b * L + ts) * D + d];
        }
        const double sg = oracle_sigmoid(p);
        const int64_t i = (b * L + t) * D + d;
        g[i] = du[i] * sg * (1.0 + p * (1.0 - sg));
      }
  for (int64_t i = 0; i < D * K; ++i) dw[i] = 0.0;
  if (dbias)
    for (int64_t d = 0; d < D; ++d) dbias[d] = 0.0;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t t = 0; t < L; ++t)
      for (int64_t d = 0; d < D; ++d) {
        const int64_t i = (b * L + t) * D + d;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
          const int64_t tf = t + (K - 1) - k;
          if (tf < L) acc += w[d * K + k] * g[(b * L + tf) * D + d];
          const int64_t ts = t - (K - 1) + k;
          if (ts >= 0) dw[d * K + k] += x[(b * L + ts) * D + d] * g[i];
        }
        dx[i] = acc;
        if (dbias) dbias[d] += g[i];
      }
  free(g);
  return 0;
}

/* ---- scan of affine maps ------------------------------------------------ */

/* The sequential fold of the maps h -> a h + b along each row of row-major
 * (rows, len) arrays: s = h0[r] (0 if h0 is NULL), then for i in scan order
 * (0 .. len-1, or len-1 .. 0 if reverse) s = a[r,i] * s + b[r,i] and
 * h[r,i] = s.  One step of the recurrence above is such a map (reading guide,
 * "Yöntem": the new state is Abar times the old one plus the input term). */
int oracle_affine_scan(int64_t rows, int64_t len, const double *a, const double *b,
                       const double *h0, double *h, int reverse) {
  if (rows < 1 || len < 1) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    double s = h0 ? h0[r] : 0.0;
    for (int64_t k = 0; k < len; ++k) {
      const int64_t i = r * len + (reverse ? len - 1 - k : k);
      s = a[i] * s + b[i];
      h[i] = s;
    }
  }
  return 0;
}
