/*
 * ttt_oracle.c -- fp64 CPU reference of the TTT-layer forward scan.
 *
 * TEST INFRASTRUCTURE ONLY (see ttt_oracle.h for the sources, the readings
 * taken and the layouts).  Deliberately plain: one token at a time, explicit
 * gradients, sequential sums, no blocking and no reordering.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared ttt_oracle.c -o libttt_oracle.so
 *        -lm -lpthread     (no -ffast-math: the loop order is the reference)
 */
#include "ttt_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Layer norm over the d features of one token, and its backward.      */
/* [KT5]: LayerNorm inside f.  Biased variance, caller's epsilon.      */
/* ------------------------------------------------------------------ */

typedef struct {
  double mean;
  double sigma;  /* sqrt(var + eps) */
} ln_stats;

static ln_stats ln_forward(int d, const double* h, const double* gamma,
                           const double* beta, double eps, double* xhat,
                           double* y) {
  ln_stats st;
  double s = 0.0;
  for (int j = 0; j < d; ++j) s += h[j];
  st.mean = s / d;
  double var = 0.0;
  for (int j = 0; j < d; ++j) {
    double e = h[j] - st.mean;
    var += e * e;
  }
  var /= d;
  st.sigma = sqrt(var + eps);
  for (int j = 0; j < d; ++j) {
    xhat[j] = (h[j] - st.mean) / st.sigma;
    y[j] = gamma[j] * xhat[j] + beta[j];
  }
  return st;
}

/* Given dL/dy, returns dL/dh for y = gamma * (h - mean) / sigma + beta. */
static void ln_backward(int d, const double* gy, const double* xhat,
                        const double* gamma, ln_stats st, double* gh) {
  double ma = 0.0, max = 0.0;
  for (int j = 0; j < d; ++j) {
    double a = gamma[j] * gy[j];
    ma += a;
    max += a * xhat[j];
  }
  ma /= d;
  max /= d;
  for (int j = 0; j < d; ++j) {
    double a = gamma[j] * gy[j];
    gh[j] = (a - ma - xhat[j] * max) / st.sigma;
  }
}

/* GELU, exact erf form, and its derivative Phi(x) + x*phi(x). */
static double gelu(double x) { return 0.5 * x * (1.0 + erf(x / sqrt(2.0))); }
static double gelu_grad(double x) {
  const double inv_sqrt_2pi = 0.39894228040143267794;
  return 0.5 * (1.0 + erf(x / sqrt(2.0))) + x * inv_sqrt_2pi * exp(-0.5 * x * x);
}

/* ------------------------------------------------------------------ */
/* TTT-Linear: f(x) = [x +] [LN](x W)                                  */
/* ------------------------------------------------------------------ */

void ttt_oracle_linear_apply(int d, int use_ln, int use_residual,
                             double ln_eps, const double* W, const double* x,
                             const double* gamma, const double* beta,
                             double* out) {
  double* h = (double*)malloc(sizeof(double) * 3 * d);
  double* xh = h + d;
  double* y = h + 2 * d;
  for (int j = 0; j < d; ++j) {
    double s = 0.0;
    for (int i = 0; i < d; ++i) s += x[i] * W[(size_t)i * d + j];
    h[j] = s;
  }
  if (use_ln) ln_forward(d, h, gamma, beta, ln_eps, xh, y);
  else memcpy(y, h, sizeof(double) * d);
  for (int j = 0; j < d; ++j) out[j] = (use_residual ? x[j] : 0.0) + y[j];
  free(h);
}

/* l(W; k, v) = || f(k; W) - v ||^2 and dl/dW = k^T g_h ([KT2]). */
double ttt_oracle_linear_loss_grad(int d, int use_ln, int use_residual,
                                   double ln_eps, const double* W,
                                   const double* k, const double* v,
                                   const double* gamma, const double* beta,
                                   double* gW) {
  double* h = (double*)malloc(sizeof(double) * 5 * d);
  double* xh = h + d;
  double* y = h + 2 * d;
  double* gy = h + 3 * d;
  double* gh = h + 4 * d;
  for (int j = 0; j < d; ++j) {
    double s = 0.0;
    for (int i = 0; i < d; ++i) s += k[i] * W[(size_t)i * d + j];
    h[j] = s;
  }
  ln_stats st = {0.0, 1.0};
  if (use_ln) st = ln_forward(d, h, gamma, beta, ln_eps, xh, y);
  else memcpy(y, h, sizeof(double) * d);
  double loss = 0.0;
  for (int j = 0; j < d; ++j) {
    double r = (use_residual ? k[j] : 0.0) + y[j] - v[j];
    loss += r * r;
    gy[j] = 2.0 * r;
  }
  if (gW) {
    if (use_ln) ln_backward(d, gy, xh, gamma, st, gh);
    else memcpy(gh, gy, sizeof(double) * d);
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) gW[(size_t)i * d + j] = k[i] * gh[j];
  }
  free(h);
  return loss;
}

/* ------------------------------------------------------------------ */
/* TTT-MLP: f(x) = [x +] [LN](GELU(x W1 + b1) W2 + b2)                  */
/* ------------------------------------------------------------------ */

void ttt_oracle_mlp_apply(int d, int m, int use_ln, int use_residual,
                          double ln_eps, const double* W1, const double* b1,
                          const double* W2, const double* b2, const double* x,
                          const double* gamma, const double* beta,
                          double* out) {
  double* a = (double*)malloc(sizeof(double) * (m + 3 * d));
  double* o = a + m;
  double* xh = o + d;
  double* y = xh + d;
  for (int n = 0; n < m; ++n) {
    double s = b1[n];
    for (int i = 0; i < d; ++i) s += x[i] * W1[(size_t)i * m + n];
    a[n] = gelu(s);
  }
  for (int j = 0; j < d; ++j) {
    double s = b2[j];
    for (int n = 0; n < m; ++n) s += a[n] * W2[(size_t)n * d + j];
    o[j] = s;
  }
  if (use_ln) ln_forward(d, o, gamma, beta, ln_eps, xh, y);
  else memcpy(y, o, sizeof(double) * d);
  for (int j = 0; j < d; ++j) out[j] = (use_residual ? x[j] : 0.0) + y[j];
  free(a);
}

double ttt_oracle_mlp_loss_grad(int d, int m, int use_ln, int use_residual,
                                double ln_eps,
                                const double* W1, const double* b1,
                                const double* W2, const double* b2,
                                const double* k, const double* v,
                                const double* gamma, const double* beta,
                                double* gW1, double* gb1,
                                double* gW2, double* gb2) {
  double* p = (double*)malloc(sizeof(double) * (3 * m + 5 * d));
  double* a = p + m;
  double* gp = a + m;
  double* o = gp + m;
  double* xh = o + d;
  double* y = xh + d;
  double* gy = y + d;
  double* go = gy + d;
  for (int n = 0; n < m; ++n) {
    double s = b1[n];
    for (int i = 0; i < d; ++i) s += k[i] * W1[(size_t)i * m + n];
    p[n] = s;
    a[n] = gelu(s);
  }
  for (int j = 0; j < d; ++j) {
    double s = b2[j];
    for (int n = 0; n < m; ++n) s += a[n] * W2[(size_t)n * d + j];
    o[j] = s;
  }
  ln_stats st = {0.0, 1.0};
  if (use_ln) st = ln_forward(d, o, gamma, beta, ln_eps, xh, y);
  else memcpy(y, o, sizeof(double) * d);
  double loss = 0.0;
  for (int j = 0; j < d; ++j) {
    double r = (use_residual ? k[j] : 0.0) + y[j] - v[j];
    loss += r * r;
    gy[j] = 2.0 * r;
  }
  if (gW1) {
    if (use_ln) ln_backward(d, gy, xh, gamma, st, go);
    else memcpy(go, gy, sizeof(double) * d);
    /* output layer: dW2 = a^T g_o, db2 = g_o */
    for (int n = 0; n < m; ++n)
      for (int j = 0; j < d; ++j) gW2[(size_t)n * d + j] = a[n] * go[j];
    for (int j = 0; j < d; ++j) gb2[j] = go[j];
    /* hidden layer: g_p = (g_o W2^T) * GELU'(p); dW1 = k^T g_p, db1 = g_p */
    for (int n = 0; n < m; ++n) {
      double s = 0.0;
      for (int j = 0; j < d; ++j) s += go[j] * W2[(size_t)n * d + j];
      gp[n] = s * gelu_grad(p[n]);
    }
    for (int i = 0; i < d; ++i)
      for (int n = 0; n < m; ++n) gW1[(size_t)i * m + n] = k[i] * gp[n];
    for (int n = 0; n < m; ++n) gb1[n] = gp[n];
  }
  free(p);
  return loss;
}

/* ------------------------------------------------------------------ */
/* The scan: one unit (batch b, head h) at a time.                     */
/* ------------------------------------------------------------------ */

static void widen(int n, const float* src, double* dst) {
  for (int i = 0; i < n; ++i) dst[i] = (double)src[i];
}

typedef struct {
  const ttt_oracle_cfg* cfg;
  int is_mlp, m;
  const float *q, *k, *v, *eta;
  const float *s0[4];   /* Linear: s0[0] = W0.  MLP: W1, b1, W2, b2 */
  const float *gamma, *beta;
  double* z;
  double* s_out[4];
  int next_unit;        /* shared work counter, guarded by lock */
  pthread_mutex_t lock;
} scan_job;

/* Sizes of the state pieces (in elements). */
static void state_sizes(const scan_job* job, int sz[4], int* nparts) {
  int d = job->cfg->d;
  if (!job->is_mlp) {
    sz[0] = d * d; sz[1] = sz[2] = sz[3] = 0;
    *nparts = 1;
  } else {
    sz[0] = d * job->m; sz[1] = job->m; sz[2] = job->m * d; sz[3] = d;
    *nparts = 4;
  }
}

static void run_unit(scan_job* job, int unit) {
  const ttt_oracle_cfg* c = job->cfg;
  const int d = c->d, T = c->T, H = c->H;
  const int bsz = c->mini_batch;
  const int head = unit % H;
  const size_t tok0 = (size_t)unit * T;

  int sz[4], np;
  state_sizes(job, sz, &np);
  int total = 0;
  for (int p = 0; p < np; ++p) total += sz[p];

  /* S: running state; Sb: state at the start of the mini-batch;
   * G: one token's gradient; all laid out piece after piece. */
  double* S = (double*)malloc(sizeof(double) * 3 * (size_t)total);
  double* Sb = S + total;
  double* G = Sb + total;
  double* vec = (double*)malloc(sizeof(double) * 6 * (size_t)d);
  double *kk = vec, *vv = vec + d, *qq = vec + 2 * d, *zz = vec + 3 * d;
  double *gam = vec + 4 * d, *bet = vec + 5 * d;

  size_t sunit = c->state0_per_batch ? (size_t)unit : (size_t)head;
  int off = 0;
  for (int p = 0; p < np; ++p) {
    widen(sz[p], job->s0[p] + sunit * sz[p], S + off);
    off += sz[p];
  }
  if (c->use_ln) {
    widen(d, job->gamma + (size_t)head * d, gam);
    widen(d, job->beta + (size_t)head * d, bet);
  } else {
    for (int j = 0; j < d; ++j) { gam[j] = 1.0; bet[j] = 0.0; }
  }

  for (int t0 = 0; t0 < T; t0 += bsz) {
    int t1 = t0 + bsz < T ? t0 + bsz : T;
    memcpy(Sb, S, sizeof(double) * total);              /* gradient point */
    for (int t = t0; t < t1; ++t) {
      const size_t row = (tok0 + t) * d;
      widen(d, job->k + row, kk);
      widen(d, job->v + row, vv);
      widen(d, job->q + row, qq);
      const double eta = (double)job->eta[tok0 + t];
      if (!job->is_mlp) {
        ttt_oracle_linear_loss_grad(d, c->use_ln, c->use_residual, c->ln_eps,
                                    Sb, kk, vv, gam, bet, G);
      } else {
        const int m = job->m;
        ttt_oracle_mlp_loss_grad(d, m, c->use_ln, c->use_residual, c->ln_eps,
                                 Sb, Sb + sz[0], Sb + sz[0] + sz[1],
                                 Sb + sz[0] + sz[1] + sz[2], kk, vv, gam, bet,
                                 G, G + sz[0], G + sz[0] + sz[1],
                                 G + sz[0] + sz[1] + sz[2]);
      }
      for (int i = 0; i < total; ++i) S[i] -= eta * G[i];   /* update rule */
      if (!job->is_mlp) {                                  /* output rule */
        ttt_oracle_linear_apply(d, c->use_ln, c->use_residual, c->ln_eps, S,
                                qq, gam, bet, zz);
      } else {
        const int m = job->m;
        ttt_oracle_mlp_apply(d, m, c->use_ln, c->use_residual, c->ln_eps, S,
                             S + sz[0], S + sz[0] + sz[1],
                             S + sz[0] + sz[1] + sz[2], qq, gam, bet, zz);
      }
      memcpy(job->z + row, zz, sizeof(double) * d);
    }
  }

  off = 0;
  for (int p = 0; p < np; ++p) {
    if (job->s_out[p])
      memcpy(job->s_out[p] + (size_t)unit * sz[p], S + off,
             sizeof(double) * sz[p]);
    off += sz[p];
  }
  free(vec);
  free(S);
}

static void* worker(void* arg) {
  scan_job* job = (scan_job*)arg;
  const int units = job->cfg->B * job->cfg->H;
  for (;;) {
    pthread_mutex_lock(&job->lock);
    int u = job->next_unit++;
    pthread_mutex_unlock(&job->lock);
    if (u >= units) break;
    run_unit(job, u);
  }
  return NULL;
}

static int run_scan(scan_job* job, int n_threads) {
  const int units = job->cfg->B * job->cfg->H;
  if (n_threads < 1) n_threads = 1;
  if (n_threads > units) n_threads = units;
  job->next_unit = 0;
  pthread_mutex_init(&job->lock, NULL);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)n_threads);
  int started = 0, rc = 0;
  for (int i = 1; i < n_threads; ++i) {
    if (pthread_create(&th[i], NULL, worker, job) != 0) { rc = -2; break; }
    ++started;
  }
  worker(job);  /* the calling thread works too */
  for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&job->lock);
  return rc;
}

static int cfg_ok(const ttt_oracle_cfg* c) {
  return c && c->B >= 1 && c->H >= 1 && c->T >= 1 && c->d >= 1 &&
         c->mini_batch >= 1 && c->ln_eps >= 0.0;
}

int ttt_oracle_linear(const ttt_oracle_cfg* cfg,
                      const float* q, const float* k, const float* v,
                      const float* eta, const float* w0,
                      const float* gamma, const float* beta,
                      double* z, double* w_out, int n_threads) {
  if (!cfg_ok(cfg) || !q || !k || !v || !eta || !w0 || !z) return -1;
  if (cfg->use_ln && (!gamma || !beta)) return -1;
  scan_job job;
  memset(&job, 0, sizeof job);
  job.cfg = cfg;
  job.is_mlp = 0;
  job.q = q; job.k = k; job.v = v; job.eta = eta;
  job.s0[0] = w0;
  job.gamma = gamma; job.beta = beta;
  job.z = z;
  job.s_out[0] = w_out;
  return run_scan(&job, n_threads);
}

int ttt_oracle_mlp(const ttt_oracle_cfg* cfg, int hidden,
                   const float* q, const float* k, const float* v,
                   const float* eta,
                   const float* w1_0, const float* b1_0,
                   const float* w2_0, const float* b2_0,
                   const float* gamma, const float* beta,
                   double* z, double* w1_out, double* b1_out,
                   double* w2_out, double* b2_out, int n_threads) {
  if (!cfg_ok(cfg) || hidden < 1 || !q || !k || !v || !eta || !w1_0 ||
      !b1_0 || !w2_0 || !b2_0 || !z)
    return -1;
  if (cfg->use_ln && (!gamma || !beta)) return -1;
  scan_job job;
  memset(&job, 0, sizeof job);
  job.cfg = cfg;
  job.is_mlp = 1;
  job.m = hidden;
  job.q = q; job.k = k; job.v = v; job.eta = eta;
  job.s0[0] = w1_0; job.s0[1] = b1_0; job.s0[2] = w2_0; job.s0[3] = b2_0;
  job.gamma = gamma; job.beta = beta;
  job.z = z;
  job.s_out[0] = w1_out; job.s_out[1] = b1_out;
  job.s_out[2] = w2_out; job.s_out[3] = b2_out;
  return run_scan(&job, n_threads);
}
