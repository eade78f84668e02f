/*
 * TTT forward-scan oracle: plain, slow, sequential fp64 PRIMAL form.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with
 * the HIP kernels.
 *
 * What it computes (sources: "论文速览 | TTT", the equinox-blog close reading
 * of "Learning to (Learn at Test Time): RNNs with Expressive Hidden States"):
 *
 *  - §3.1 Naive TTT: the state is the parameter set W of an inner model f;
 *    each token first takes a gradient step on its own loss and the output is
 *    then read from the UPDATED state:  W_t = W_{t-1} - eta * grad l(W_?; x_t),
 *    z_t = f(x_t; W_t).
 *  - §3.3 Multi-view reconstruction: l(W; x_t) = || f(k_t; W) - v_t ||^2 and
 *    z_t = f(q_t; W_t), with k, v, q the training, label and test views.  The
 *    views arrive already projected, so k_t, v_t, q_t are inputs here.
 *  - §3.5 Mini-batch GD: the sequence is cut into mini-batches of b tokens;
 *    every token of a mini-batch takes its gradient at W_{t'}, the state at
 *    the last position before that mini-batch, while the updates still
 *    accumulate token by token: W_t = W_{t-1} - eta_t * G_t.
 *  - §4.6 Learnable inner learning rate: eta depends on the token, so eta_t
 *    is a per-token input that scales token t's own gradient (no 1/b).
 *  - §4.4 Inner models: TTT-Linear f(x) = W x; TTT-MLP f(x) = W2 GELU(W1 x)
 *    with a hidden width that the caller chooses (4x the input on the page).
 *  - §4.4 LayerNorm + residual wrapper around either inner model:
 *    f(x) = x + LN(W x) or x + LN(W2 GELU(W1 x)), LN(y) = gamma * (y -
 *    mean(y)) / sqrt(var(y) + eps) + beta over the d output components of one
 *    token (population variance; gamma, beta per head and eps are inputs: the
 *    page names the wrapper but not its parameters).  The gradient goes
 *    through the LayerNorm.
 *
 * Decode steps (§6.11: token-by-token generation uses the primal form): one
 * token per (batch, head) unit per call.  A unit carries its current state W
 * and its gradient point Wg, the state at the start of the current
 * mini-batch; for a token at position p = pos mod b, p = 0 first sets
 * Wg = W.  Then the token's gradient is taken at Wg, W takes the step, and the
 * output is read from the updated W: exactly one iteration of the scans above.
 *
 * Backward (§6.12: training differentiates through the inner loop): the
 * reverse pass of the TTT-Linear and TTT-MLP primal recurrences above, token
 * by token in reverse, given the adjoints of Z and of the final state.  It keeps every
 * intermediate state, which is fine at test sizes (the pages' kernels keep
 * one per mini-batch and recompute; that is a memory trade, not another
 * result).
 *
 * Inner learning-rate gate (§4.6): eta(x) = eta_base * sigmoid(theta_lr . x)
 * with x the layer's input token and sigmoid(a) = 1 / (1 + exp(-a)).  The
 * page gives theta_lr as one vector; each head runs its own inner loop, so
 * here every head h has its own theta_lr[h] (H = 1 is the page's case), and
 * the gated scan is the scan above fed with eta[b][h][t] from the gate.
 *
 * Gate backward: given dL/deta, the chain rule through the sigmoid,
 * d eta / d a = eta_base sigmoid(a) (1 - sigmoid(a)), a = theta_lr[h] . x,
 * gives dL/dtheta_lr[h] = sum_{b,t} da x[b][t] and dL/dx[b][t] = sum_h da
 * theta_lr[h].
 *
 * The loss is the squared L2 norm summed over output components, so its
 * gradient carries the factor 2 (§3.6 linear derivation: G_t = 2(W0 x - x)x^T).
 * GELU is the exact erf form x * Phi(x).  Mini-batches start at token 0, b,
 * 2b, ...; a final partial mini-batch is simply shorter.
 *
 * Layouts (row-major, contiguous):
 *   q, k, v : [B][H][T][d]        eta : [B][H][T]
 *   Linear  : w0 [H][d][d] (w0_per_batch = 0) or [B][H][d][d] (= 1),
 *             W[i][j] with i the output index, f(x)_i = sum_j W[i][j] x_j
 *   MLP     : w1 [.][hidden][d], w2 [.][d][hidden] (same per-batch rule)
 *   z       : [B][H][T][d]        state outputs : [B][H][...]
 *   gate    : x [B][T][dx], theta_lr [H][dx]  ->  eta [B][H][T]
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread (no fused
 * multiply-add contraction, so every product is rounded as written).
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* TTT-Linear: one (batch, head) unit, primal mini-batch GD.           */
/* ------------------------------------------------------------------ */
static void linear_unit(const double *q, const double *k, const double *v,
                        const double *eta, const double *w0, long T, long d,
                        long b, double *z, double *w_out, double *Ws,
                        double *g) {
  double *W = w_out; /* the running state lives directly in the output */
  memcpy(W, w0, sizeof(double) * (size_t)(d * d));
  for (long m0 = 0; m0 < T; m0 += b) {
    long m1 = m0 + b < T ? m0 + b : T;
    /* gradient point W_{t'}: the state before this mini-batch (§3.5) */
    memcpy(Ws, W, sizeof(double) * (size_t)(d * d));
    for (long t = m0; t < m1; ++t) {
      const double *kt = k + t * d, *vt = v + t * d, *qt = q + t * d;
      const double et = eta[t];
      /* G_t = 2 (Ws k_t - v_t) k_t^T ; keep the vector factor g */
      for (long i = 0; i < d; ++i) {
        double s = 0.0;
        for (long j = 0; j < d; ++j) s += Ws[i * d + j] * kt[j];
        g[i] = 2.0 * (s - vt[i]);
      }
      /* W_t = W_{t-1} - eta_t G_t */
      for (long i = 0; i < d; ++i)
        for (long j = 0; j < d; ++j) W[i * d + j] -= et * g[i] * kt[j];
      /* z_t = f(q_t; W_t): output after the update (§3.1) */
      for (long i = 0; i < d; ++i) {
        double s = 0.0;
        for (long j = 0; j < d; ++j) s += W[i * d + j] * qt[j];
        z[t * d + i] = s;
      }
    }
  }
}

/* ------------------------------------------------------------------ */
/* TTT-Linear with LayerNorm + residual: f(x) = x + LN(W x).           */
/* ------------------------------------------------------------------ */
/* yhat = (y - mean(y)) / sqrt(var(y) + eps) over the d components; returns
 * 1 / sqrt(var + eps).  Two passes: the mean, then the squared deviations. */
static double ln_normalise(const double *y, long d, double eps, double *yhat) {
  double mu = 0.0;
  for (long i = 0; i < d; ++i) mu += y[i];
  mu /= (double)d;
  double var = 0.0;
  for (long i = 0; i < d; ++i) var += (y[i] - mu) * (y[i] - mu);
  var /= (double)d;
  const double rs = 1.0 / sqrt(var + eps);
  for (long i = 0; i < d; ++i) yhat[i] = (y[i] - mu) * rs;
  return rs;
}

static void linear_ln_unit(const double *q, const double *k, const double *v,
                           const double *eta, const double *w0, const double *gamma,
                           const double *beta, double eps, long T, long d, long b,
                           double *z, double *w_out, double *Ws, double *y,
                           double *yhat, double *gy) {
  double *W = w_out;
  memcpy(W, w0, sizeof(double) * (size_t)(d * d));
  for (long m0 = 0; m0 < T; m0 += b) {
    long m1 = m0 + b < T ? m0 + b : T;
    memcpy(Ws, W, sizeof(double) * (size_t)(d * d)); /* gradient point W_{t'} */
    for (long t = m0; t < m1; ++t) {
      const double *kt = k + t * d, *vt = v + t * d, *qt = q + t * d;
      const double et = eta[t];
      /* forward on the training view at the gradient point */
      for (long i = 0; i < d; ++i) {
        double acc = 0.0;
        for (long j = 0; j < d; ++j) acc += Ws[i * d + j] * kt[j];
        y[i] = acc;
      }
      const double rs = ln_normalise(y, d, eps, yhat);
      /* l = sum_i (k_i + gamma_i yhat_i + beta_i - v_i)^2;
         dl/dyhat_i = 2 gamma_i (f_i - v_i) */
      double m1s = 0.0, m2s = 0.0;
      for (long i = 0; i < d; ++i) {
        const double f = kt[i] + gamma[i] * yhat[i] + beta[i];
        gy[i] = 2.0 * gamma[i] * (f - vt[i]);
        m1s += gy[i];
        m2s += gy[i] * yhat[i];
      }
      m1s /= (double)d;
      m2s /= (double)d;
      /* LayerNorm VJP: dl/dy = rs (g - mean(g) - yhat mean(g yhat)) */
      for (long i = 0; i < d; ++i) gy[i] = rs * (gy[i] - m1s - yhat[i] * m2s);
      for (long i = 0; i < d; ++i)
        for (long j = 0; j < d; ++j) W[i * d + j] -= et * gy[i] * kt[j];
      /* z_t = q_t + LN(W_t q_t) with the updated state */
      for (long i = 0; i < d; ++i) {
        double acc = 0.0;
        for (long j = 0; j < d; ++j) acc += W[i * d + j] * qt[j];
        y[i] = acc;
      }
      ln_normalise(y, d, eps, yhat);
      for (long i = 0; i < d; ++i) z[t * d + i] = qt[i] + gamma[i] * yhat[i] + beta[i];
    }
  }
}

/* ------------------------------------------------------------------ */
/* TTT-MLP: f(x) = W2 GELU(W1 x), one unit, primal mini-batch GD.      */
/* ------------------------------------------------------------------ */
static double gelu(double x) { return 0.5 * x * (1.0 + erf(x / sqrt(2.0))); }

/* d/dx [x Phi(x)] = Phi(x) + x phi(x) */
static double gelu_grad(double x) {
  const double pi = 3.14159265358979323846;
  return 0.5 * (1.0 + erf(x / sqrt(2.0))) + x * exp(-0.5 * x * x) / sqrt(2.0 * pi);
}

typedef struct {
  double *W1s, *W2s, *a, *x, *e, *delta, *hq;
} mlp_scratch;

static void mlp_unit(const double *q, const double *k, const double *v,
                     const double *eta, const double *w1_0, const double *w2_0,
                     long T, long d, long hd, long b, double *z, double *W1,
                     double *W2, mlp_scratch *s) {
  memcpy(W1, w1_0, sizeof(double) * (size_t)(hd * d));
  memcpy(W2, w2_0, sizeof(double) * (size_t)(d * hd));
  for (long m0 = 0; m0 < T; m0 += b) {
    long m1 = m0 + b < T ? m0 + b : T;
    memcpy(s->W1s, W1, sizeof(double) * (size_t)(hd * d));
    memcpy(s->W2s, W2, sizeof(double) * (size_t)(d * hd));
    for (long t = m0; t < m1; ++t) {
      const double *kt = k + t * d, *vt = v + t * d, *qt = q + t * d;
      const double et = eta[t];
      /* forward at the gradient point: a = W1s k, x = GELU(a), y = W2s x */
      for (long u = 0; u < hd; ++u) {
        double acc = 0.0;
        for (long j = 0; j < d; ++j) acc += s->W1s[u * d + j] * kt[j];
        s->a[u] = acc;
        s->x[u] = gelu(acc);
      }
      /* dl/dy = 2 (y - v) */
      for (long i = 0; i < d; ++i) {
        double acc = 0.0;
        for (long u = 0; u < hd; ++u) acc += s->W2s[i * hd + u] * s->x[u];
        s->e[i] = 2.0 * (acc - vt[i]);
      }
      /* dl/dW2 = e x^T ; dl/da = (W2s^T e) * GELU'(a) ; dl/dW1 = delta k^T */
      for (long u = 0; u < hd; ++u) {
        double acc = 0.0;
        for (long i = 0; i < d; ++i) acc += s->W2s[i * hd + u] * s->e[i];
        s->delta[u] = acc * gelu_grad(s->a[u]);
      }
      for (long i = 0; i < d; ++i)
        for (long u = 0; u < hd; ++u) W2[i * hd + u] -= et * s->e[i] * s->x[u];
      for (long u = 0; u < hd; ++u)
        for (long j = 0; j < d; ++j) W1[u * d + j] -= et * s->delta[u] * kt[j];
      /* z_t = W2_t GELU(W1_t q_t) with the updated state */
      for (long u = 0; u < hd; ++u) {
        double acc = 0.0;
        for (long j = 0; j < d; ++j) acc += W1[u * d + j] * qt[j];
        s->hq[u] = gelu(acc);
      }
      for (long i = 0; i < d; ++i) {
        double acc = 0.0;
        for (long u = 0; u < hd; ++u) acc += W2[i * hd + u] * s->hq[u];
        z[t * d + i] = acc;
      }
    }
  }
}

/* ------------------------------------------------------------------ */
/* TTT-MLP with LayerNorm + residual: f(x) = x + LN(W2 GELU(W1 x)).    */
/* ------------------------------------------------------------------ */
/* The MLP's output y = W2 GELU(W1 x) takes the place of W x in the linear
 * wrapper above: the loss sum_i (k_i + LN(y)_i - v_i)^2 sends
 * g_i = 2 gamma_i (f_i - v_i) into the LayerNorm's VJP, which gives dl/dy;
 * from there the MLP's own backpropagation (as in mlp_unit) gives the two
 * layers' gradients, all at the mini-batch's gradient point. */
static void mlp_ln_unit(const double *q, const double *k, const double *v,
                        const double *eta, const double *w1_0, const double *w2_0,
                        const double *gamma, const double *beta, double eps, long T,
                        long d, long hd, long b, double *z, double *W1, double *W2,
                        mlp_scratch *s, double *y, double *yhat) {
  memcpy(W1, w1_0, sizeof(double) * (size_t)(hd * d));
  memcpy(W2, w2_0, sizeof(double) * (size_t)(d * hd));
  for (long m0 = 0; m0 < T; m0 += b) {
    long m1 = m0 + b < T ? m0 + b : T;
    memcpy(s->W1s, W1, sizeof(double) * (size_t)(hd * d));
    memcpy(s->W2s, W2, sizeof(double) * (size_t)(d * hd));
    for (long t = m0; t < m1; ++t) {
      const double *kt = k + t * d, *vt = v + t * d, *qt = q + t * d;
      const double et = eta[t];
      /* forward at the gradient point */
      for (long u = 0; u < hd; ++u) {
        double acc = 0.0;
        for (long j = 0; j < d; ++j) acc += s->W1s[u * d + j] * kt[j];
        s->a[u] = acc;
        s->x[u] = gelu(acc);
      }
      for (long i = 0; i < d; ++i) {
        double acc = 0.0;
        for (long u = 0; u < hd; ++u) acc += s->W2s[i * hd + u] * s->x[u];
        y[i] = acc;
      }
      const double rs = ln_normalise(y, d, eps, yhat);
      /* dl/dyhat_i = 2 gamma_i (k_i + gamma_i yhat_i + beta_i - v_i), then the
         LayerNorm VJP: e = dl/dy = rs (g - mean(g) - yhat mean(g yhat)) */
      double m1s = 0.0, m2s = 0.0;
      for (long i = 0; i < d; ++i) {
        const double resid = kt[i] + beta[i] - vt[i] + gamma[i] * yhat[i]; /* f_i - v_i */
        s->e[i] = 2.0 * gamma[i] * resid;
        m1s += s->e[i];
        m2s += s->e[i] * yhat[i];
      }
      m1s /= (double)d;
      m2s /= (double)d;
      for (long i = 0; i < d; ++i) s->e[i] = rs * (s->e[i] - m1s - yhat[i] * m2s);
      /* the MLP below the LayerNorm: dl/dW2 = e x^T, delta = (W2s^T e) * GELU'(a) */
      for (long u = 0; u < hd; ++u) {
        double back = 0.0;
        for (long i = 0; i < d; ++i) back += s->e[i] * s->W2s[i * hd + u];
        s->delta[u] = gelu_grad(s->a[u]) * back;
      }
      for (long i = 0; i < d; ++i) {
        const double step = et * s->e[i];
        for (long u = 0; u < hd; ++u) W2[i * hd + u] -= step * s->x[u];
      }
      for (long u = 0; u < hd; ++u)
        for (long j = 0; j < d; ++j) W1[u * d + j] -= et * s->delta[u] * kt[j];
      /* z_t = q_t + LN(W2_t GELU(W1_t q_t)) with the updated state */
      for (long u = 0; u < hd; ++u) {
        double pre = 0.0;
        for (long j = 0; j < d; ++j) pre += qt[j] * W1[u * d + j];
        s->hq[u] = gelu(pre);
      }
      for (long i = 0; i < d; ++i) {
        double acc = 0.0;
        for (long u = 0; u < hd; ++u) acc += W2[i * hd + u] * s->hq[u];
        y[i] = acc;
      }
      ln_normalise(y, d, eps, yhat);
      for (long i = 0; i < d; ++i) z[t * d + i] = gamma[i] * yhat[i] + beta[i] + qt[i];
    }
  }
}

/* ------------------------------------------------------------------ */
/* Threading: units (batch, head) are independent; static round robin. */
/* ------------------------------------------------------------------ */
typedef struct {
  int kind; /* 0 linear, 1 mlp, 2 linear with LayerNorm + residual, 3 mlp with it */
  const double *q, *k, *v, *eta, *w0a, *w0b, *gamma, *beta;
  double eps;
  int w0_per_batch;
  long B, H, T, d, hd, b;
  double *z, *outa, *outb;
  int tid, nthreads, status;
} job;

static void *worker(void *arg) {
  job *jb = (job *)arg;
  const long d = jb->d, hd = jb->hd, T = jb->T;
  const long units = jb->B * jb->H;
  double *buf = NULL;
  size_t need = jb->kind == 0   ? (size_t)(d * d + d)
                : jb->kind == 2 ? (size_t)(d * d + 3 * d)
                                : (size_t)(2 * hd * d + 4 * hd + 3 * d);
  buf = (double *)malloc(sizeof(double) * need);
  if (!buf) { jb->status = 1; return NULL; }
  for (long u = jb->tid; u < units; u += jb->nthreads) {
    long hh = u % jb->H;
    long wsel = jb->w0_per_batch ? u : hh;
    const double *qu = jb->q + u * T * d, *ku = jb->k + u * T * d,
                 *vu = jb->v + u * T * d, *eu = jb->eta + u * T;
    double *zu = jb->z + u * T * d;
    if (jb->kind == 0) {
      linear_unit(qu, ku, vu, eu, jb->w0a + wsel * d * d, T, d, jb->b, zu,
                  jb->outa + u * d * d, buf, buf + d * d);
    } else if (jb->kind == 2) {
      linear_ln_unit(qu, ku, vu, eu, jb->w0a + wsel * d * d, jb->gamma + hh * d,
                     jb->beta + hh * d, jb->eps, T, d, jb->b, zu, jb->outa + u * d * d,
                     buf, buf + d * d, buf + d * d + d, buf + d * d + 2 * d);
    } else {
      mlp_scratch s;
      s.W1s = buf;
      s.W2s = buf + hd * d;
      s.a = buf + 2 * hd * d;
      s.x = s.a + hd;
      s.delta = s.x + hd;
      s.hq = s.delta + hd;
      s.e = s.hq + hd;
      if (jb->kind == 1)
        mlp_unit(qu, ku, vu, eu, jb->w0a + wsel * hd * d, jb->w0b + wsel * d * hd,
                 T, d, hd, jb->b, zu, jb->outa + u * hd * d, jb->outb + u * d * hd,
                 &s);
      else
        mlp_ln_unit(qu, ku, vu, eu, jb->w0a + wsel * hd * d, jb->w0b + wsel * d * hd,
                    jb->gamma + hh * d, jb->beta + hh * d, jb->eps, T, d, hd, jb->b, zu,
                    jb->outa + u * hd * d, jb->outb + u * d * hd, &s, s.e + d, s.e + 2 * d);
    }
  }
  free(buf);
  return NULL;
}

static int run(job proto, int nthreads) {
  if (proto.B < 0 || proto.H < 0 || proto.T < 0 || proto.d <= 0 || proto.b <= 0)
    return 2;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  job *jobs = (job *)calloc((size_t)nthreads, sizeof(job));
  pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) { free(jobs); free(th); return 1; }
  int rc = 0;
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = proto;
    jobs[i].tid = i;
    jobs[i].nthreads = nthreads;
    jobs[i].status = 0;
  }
  for (int i = 1; i < nthreads; ++i)
    if (pthread_create(&th[i], NULL, worker, &jobs[i]) != 0) { jobs[i].status = 3; th[i] = 0; }
  worker(&jobs[0]);
  for (int i = 1; i < nthreads; ++i) {
    if (jobs[i].status == 3) {
      worker(&jobs[i]); /* thread creation failed: run its share inline */
      jobs[i].status = 0;
    } else {
      pthread_join(th[i], NULL);
    }
  }
  for (int i = 0; i < nthreads; ++i) rc |= jobs[i].status;
  free(jobs);
  free(th);
  return rc;
}

int ttt_oracle_linear(const double *q, const double *k, const double *v,
                      const double *eta, const double *w0, int w0_per_batch,
                      long B, long H, long T, long d, long b, double *z,
                      double *w_out, int nthreads) {
  job p;
  memset(&p, 0, sizeof p);
  p.kind = 0; p.q = q; p.k = k; p.v = v; p.eta = eta; p.w0a = w0;
  p.w0_per_batch = w0_per_batch; p.B = B; p.H = H; p.T = T; p.d = d; p.hd = 0;
  p.b = b; p.z = z; p.outa = w_out;
  return run(p, nthreads);
}

int ttt_oracle_mlp(const double *q, const double *k, const double *v,
                   const double *eta, const double *w1_0, const double *w2_0,
                   int w0_per_batch, long B, long H, long T, long d, long hidden,
                   long b, double *z, double *w1_out, double *w2_out,
                   int nthreads) {
  if (hidden <= 0) return 2;
  job p;
  memset(&p, 0, sizeof p);
  p.kind = 1; p.q = q; p.k = k; p.v = v; p.eta = eta; p.w0a = w1_0; p.w0b = w2_0;
  p.w0_per_batch = w0_per_batch; p.B = B; p.H = H; p.T = T; p.d = d; p.hd = hidden;
  p.b = b; p.z = z; p.outa = w1_out; p.outb = w2_out;
  return run(p, nthreads);
}

int ttt_oracle_linear_ln(const double *q, const double *k, const double *v,
                         const double *eta, const double *w0, int w0_per_batch,
                         const double *gamma, const double *beta, double eps,
                         long B, long H, long T, long d, long b, double *z,
                         double *w_out, int nthreads) {
  if (!(eps >= 0.0)) return 2;
  job p;
  memset(&p, 0, sizeof p);
  p.kind = 2; p.q = q; p.k = k; p.v = v; p.eta = eta; p.w0a = w0;
  p.gamma = gamma; p.beta = beta; p.eps = eps;
  p.w0_per_batch = w0_per_batch; p.B = B; p.H = H; p.T = T; p.d = d; p.hd = 0;
  p.b = b; p.z = z; p.outa = w_out;
  return run(p, nthreads);
}

int ttt_oracle_mlp_ln(const double *q, const double *k, const double *v,
                      const double *eta, const double *w1_0, const double *w2_0,
                      int w0_per_batch, const double *gamma, const double *beta, double eps,
                      long B, long H, long T, long d, long hidden, long b, double *z,
                      double *w1_out, double *w2_out, int nthreads) {
  if (hidden <= 0 || !(eps >= 0.0)) return 2;
  job p;
  memset(&p, 0, sizeof p);
  p.kind = 3; p.q = q; p.k = k; p.v = v; p.eta = eta; p.w0a = w1_0; p.w0b = w2_0;
  p.gamma = gamma; p.beta = beta; p.eps = eps;
  p.w0_per_batch = w0_per_batch; p.B = B; p.H = H; p.T = T; p.d = d; p.hd = hidden;
  p.b = b; p.z = z; p.outa = w1_out; p.outb = w2_out;
  return run(p, nthreads);
}

/* ------------------------------------------------------------------ */
/* Decode steps: one token per unit, primal form (§6.11).              */
/* Layouts: q, k, v [B][H][d]; eta [B][H]; pos [B]; states [B][H][...]; */
/* z [B][H][d].  States are updated in place.                          */
/* ------------------------------------------------------------------ */
static int step_args_ok(long B, long H, long d, long b) {
  return B >= 0 && H >= 0 && d > 0 && b > 0;
}

int ttt_oracle_linear_step(const double *q, const double *k, const double *v,
                           const double *eta, double *w, double *wg,
                           const int *pos, long B, long H, long d, long b,
                           double *z) {
  if (!step_args_ok(B, H, d, b)) return 2;
  double *gr = (double *)malloc(sizeof(double) * (size_t)d);
  if (!gr) return 1;
  for (long u = 0; u < B * H; ++u) {
    const long bi = u / H;
    const double *ku = k + u * d, *vu = v + u * d, *qu = q + u * d;
    double *W = w + u * d * d, *Wg = wg + u * d * d;
    if (pos[bi] % b == 0) memcpy(Wg, W, sizeof(double) * (size_t)(d * d));
    /* gradient of ||W k - v||^2 at the gradient point: 2 (Wg k - v) k^T */
    for (long i = 0; i < d; ++i) {
      double pk = 0.0;
      for (long j = 0; j < d; ++j) pk += Wg[i * d + j] * ku[j];
      gr[i] = 2.0 * (pk - vu[i]);
    }
    for (long i = 0; i < d; ++i)
      for (long j = 0; j < d; ++j) W[i * d + j] -= eta[u] * gr[i] * ku[j];
    for (long i = 0; i < d; ++i) {
      double zq = 0.0;
      for (long j = 0; j < d; ++j) zq += W[i * d + j] * qu[j];
      z[u * d + i] = zq;
    }
  }
  free(gr);
  return 0;
}

int ttt_oracle_linear_ln_step(const double *q, const double *k, const double *v,
                              const double *eta, double *w, double *wg,
                              const int *pos, const double *gamma,
                              const double *beta, double eps, long B, long H,
                              long d, long b, double *z) {
  if (!step_args_ok(B, H, d, b) || !(eps >= 0.0)) return 2;
  double *y = (double *)malloc(sizeof(double) * (size_t)(3 * d));
  if (!y) return 1;
  double *yh = y + d, *gy = y + 2 * d;
  for (long u = 0; u < B * H; ++u) {
    const long bi = u / H, hh = u % H;
    const double *ku = k + u * d, *vu = v + u * d, *qu = q + u * d;
    const double *ga = gamma + hh * d, *be = beta + hh * d;
    double *W = w + u * d * d, *Wg = wg + u * d * d;
    if (pos[bi] % b == 0) memcpy(Wg, W, sizeof(double) * (size_t)(d * d));
    for (long i = 0; i < d; ++i) {
      double pk = 0.0;
      for (long j = 0; j < d; ++j) pk += Wg[i * d + j] * ku[j];
      y[i] = pk;
    }
    const double rs = ln_normalise(y, d, eps, yh);
    /* f(k) = k + gamma yhat + beta; dl/dyhat_i = 2 gamma_i (f_i - v_i) */
    double mg = 0.0, mgy = 0.0;
    for (long i = 0; i < d; ++i) {
      gy[i] = 2.0 * ga[i] * (ku[i] + ga[i] * yh[i] + be[i] - vu[i]);
      mg += gy[i];
      mgy += gy[i] * yh[i];
    }
    mg /= (double)d;
    mgy /= (double)d;
    for (long i = 0; i < d; ++i) {
      const double dy = rs * (gy[i] - mg - yh[i] * mgy); /* LayerNorm VJP */
      for (long j = 0; j < d; ++j) W[i * d + j] -= eta[u] * dy * ku[j];
    }
    for (long i = 0; i < d; ++i) {
      double zq = 0.0;
      for (long j = 0; j < d; ++j) zq += W[i * d + j] * qu[j];
      y[i] = zq;
    }
    ln_normalise(y, d, eps, yh);
    for (long i = 0; i < d; ++i) z[u * d + i] = qu[i] + ga[i] * yh[i] + be[i];
  }
  free(y);
  return 0;
}

int ttt_oracle_mlp_step(const double *q, const double *k, const double *v,
                        const double *eta, double *w1, double *w2, double *w1g,
                        double *w2g, const int *pos, long B, long H, long d,
                        long hidden, long b, double *z) {
  if (!step_args_ok(B, H, d, b) || hidden <= 0) return 2;
  const long hd = hidden;
  double *sc = (double *)malloc(sizeof(double) * (size_t)(4 * hd + d));
  if (!sc) return 1;
  double *a = sc, *x = sc + hd, *dl = sc + 2 * hd, *hq = sc + 3 * hd, *e = sc + 4 * hd;
  for (long u = 0; u < B * H; ++u) {
    const long bi = u / H;
    const double *ku = k + u * d, *vu = v + u * d, *qu = q + u * d;
    double *W1 = w1 + u * hd * d, *W2 = w2 + u * d * hd;
    double *W1g = w1g + u * hd * d, *W2g = w2g + u * d * hd;
    if (pos[bi] % b == 0) {
      memcpy(W1g, W1, sizeof(double) * (size_t)(hd * d));
      memcpy(W2g, W2, sizeof(double) * (size_t)(d * hd));
    }
    /* forward and backward at the gradient point */
    for (long h = 0; h < hd; ++h) {
      double ak = 0.0;
      for (long j = 0; j < d; ++j) ak += W1g[h * d + j] * ku[j];
      a[h] = ak;
      x[h] = gelu(ak);
    }
    for (long i = 0; i < d; ++i) {
      double yo = 0.0;
      for (long h = 0; h < hd; ++h) yo += W2g[i * hd + h] * x[h];
      e[i] = 2.0 * (yo - vu[i]);
    }
    for (long h = 0; h < hd; ++h) {
      double bp = 0.0;
      for (long i = 0; i < d; ++i) bp += W2g[i * hd + h] * e[i];
      dl[h] = bp * gelu_grad(a[h]);
    }
    for (long i = 0; i < d; ++i)
      for (long h = 0; h < hd; ++h) W2[i * hd + h] -= eta[u] * e[i] * x[h];
    for (long h = 0; h < hd; ++h)
      for (long j = 0; j < d; ++j) W1[h * d + j] -= eta[u] * dl[h] * ku[j];
    for (long h = 0; h < hd; ++h) {
      double aq = 0.0;
      for (long j = 0; j < d; ++j) aq += W1[h * d + j] * qu[j];
      hq[h] = gelu(aq);
    }
    for (long i = 0; i < d; ++i) {
      double zo = 0.0;
      for (long h = 0; h < hd; ++h) zo += W2[i * hd + h] * hq[h];
      z[u * d + i] = zo;
    }
  }
  free(sc);
  return 0;
}

/* ------------------------------------------------------------------ */
/* TTT-Linear backward: reverse pass of the primal recurrence.         */
/* ------------------------------------------------------------------ */
/* Forward, one unit (as linear_unit), keeping every state:
 *   Wst[0] = W0, Wst[t+1] = Wst[t] - eta_t g_t k_t^T,
 *   g_t = 2 (Wst[m0] k_t - v_t) with m0 the first token of t's mini-batch,
 *   z_t = Wst[t+1] q_t.
 * Reverse, with A the adjoint of the state after token t (starting from the
 * adjoint of W_T) and Ag the adjoint collected for the current mini-batch's
 * gradient point:
 *   dq_t = Wst[t+1]^T dz_t,            A += dz_t q_t^T
 *   gb = -eta_t A k_t                  (adjoint of g_t)
 *   dk_t = -eta_t A^T g_t + 2 Wst[m0]^T gb,  deta_t = -g_t^T A k_t,
 *   dv_t = -2 gb,  Ag += 2 gb k_t^T
 *   at t = m0 the gradient point is Wst[t]: A += Ag, Ag = 0.
 * A then carries over unchanged to the state before token t. */
static int linear_bwd_unit(const double *q, const double *k, const double *v,
                           const double *eta, const double *w0, long T, long d,
                           long b, const double *dz, const double *dwT, double *dq,
                           double *dk, double *dv, double *deta, double *dw0) {
  const size_t dd = (size_t)(d * d);
  double *Wst = (double *)malloc(sizeof(double) * dd * (size_t)(T + 1));
  double *Ag = (double *)calloc(dd, sizeof(double));
  double *g = (double *)malloc(sizeof(double) * (size_t)(3 * d));
  if (!Wst || !Ag || !g) { free(Wst); free(Ag); free(g); return 1; }
  double *gb = g + d, *Ak = g + 2 * d;
  memcpy(Wst, w0, sizeof(double) * dd);
  for (long t = 0; t < T; ++t) {
    const long m0 = (t / b) * b;
    const double *Wg = Wst + (size_t)m0 * dd, *Wp = Wst + (size_t)t * dd;
    double *Wn = Wst + (size_t)(t + 1) * dd;
    const double *kt = k + t * d, *vt = v + t * d;
    for (long i = 0; i < d; ++i) {
      double pk = 0.0;
      for (long j = 0; j < d; ++j) pk += Wg[i * d + j] * kt[j];
      g[i] = 2.0 * (pk - vt[i]);
    }
    for (long i = 0; i < d; ++i)
      for (long j = 0; j < d; ++j) Wn[i * d + j] = Wp[i * d + j] - eta[t] * g[i] * kt[j];
  }
  double *A = dw0; /* the running adjoint lives in the output */
  if (dwT) memcpy(A, dwT, sizeof(double) * dd);
  else memset(A, 0, sizeof(double) * dd);
  for (long t = T - 1; t >= 0; --t) {
    const long m0 = (t / b) * b;
    const double *Wg = Wst + (size_t)m0 * dd, *Wn = Wst + (size_t)(t + 1) * dd;
    const double *kt = k + t * d, *vt = v + t * d, *qt = q + t * d, *zt = dz + t * d;
    /* z_t = W_t q_t */
    for (long j = 0; j < d; ++j) {
      double s = 0.0;
      for (long i = 0; i < d; ++i) s += Wn[i * d + j] * zt[i];
      dq[t * d + j] = s;
    }
    for (long i = 0; i < d; ++i)
      for (long j = 0; j < d; ++j) A[i * d + j] += zt[i] * qt[j];
    /* W_t = W_{t-1} - eta_t g_t k_t^T */
    for (long i = 0; i < d; ++i) {
      double pk = 0.0;
      for (long j = 0; j < d; ++j) pk += Wg[i * d + j] * kt[j];
      g[i] = 2.0 * (pk - vt[i]);
    }
    double de = 0.0;
    for (long i = 0; i < d; ++i) {
      double s = 0.0;
      for (long j = 0; j < d; ++j) s += A[i * d + j] * kt[j];
      Ak[i] = s;
      gb[i] = -eta[t] * s;
      de -= g[i] * s;
    }
    deta[t] = de;
    for (long j = 0; j < d; ++j) {
      double s1 = 0.0, s2 = 0.0;
      for (long i = 0; i < d; ++i) {
        s1 += A[i * d + j] * g[i];
        s2 += Wg[i * d + j] * gb[i];
      }
      dk[t * d + j] = -eta[t] * s1 + 2.0 * s2;
    }
    /* g_t = 2 (W_{t'} k_t - v_t) */
    for (long i = 0; i < d; ++i) {
      dv[t * d + i] = -2.0 * gb[i];
      for (long j = 0; j < d; ++j) Ag[i * d + j] += 2.0 * gb[i] * kt[j];
    }
    if (t == m0) { /* the gradient point of this mini-batch is the state before t */
      for (size_t e = 0; e < dd; ++e) {
        A[e] += Ag[e];
        Ag[e] = 0.0;
      }
    }
  }
  free(Wst);
  free(Ag);
  free(g);
  return 0;
}

int ttt_oracle_linear_bwd(const double *q, const double *k, const double *v,
                          const double *eta, const double *w0, int w0_per_batch,
                          long B, long H, long T, long d, long b, const double *dz,
                          const double *dwT, double *dq, double *dk, double *dv,
                          double *deta, double *dw0) {
  if (B < 0 || H < 0 || T < 0 || d <= 0 || b <= 0) return 2;
  for (long u = 0; u < B * H; ++u) {
    const long wsel = w0_per_batch ? u : u % H;
    const size_t so = (size_t)u * (size_t)(T * d);
    int rc = linear_bwd_unit(q + so, k + so, v + so, eta + (size_t)u * (size_t)T,
                             w0 + (size_t)wsel * (size_t)(d * d), T, d, b, dz + so,
                             dwT ? dwT + (size_t)u * (size_t)(d * d) : NULL, dq + so, dk + so,
                             dv + so, deta + (size_t)u * (size_t)T, dw0 + (size_t)u * (size_t)(d * d));
    if (rc) return rc;
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* TTT-Linear with LayerNorm + residual: backward (§6.12 with §4.4).   */
/* ------------------------------------------------------------------ */
/* Forward, one unit (as linear_ln_unit), keeping every state: S[t+1] =
 * S[t] - eta_t dy_t k_t^T with, at the gradient point P = S[m0]:
 *   y = P k, mu = mean(y), c = y - mu, var = mean(c^2), rs = (var+eps)^-1/2,
 *   yh = c rs, f = k + gamma yh + beta, r = f - v, g = 2 gamma r,
 *   dy = rs (g - mean(g) - yh mean(g yh));
 * and the output z = q + gamma LNhat(S[t+1] q) + beta.
 * Reverse: each forward operation's adjoint, in the opposite order, with A
 * the adjoint of the state after token t (starting from dW_T), Ag that of
 * the current mini-batch's gradient point (added to A at its first token),
 * and dgamma, dbeta summed over the tokens. */
static void ln_stats(const double *y, long d, double eps, double *c, double *rs) {
  double mu = 0.0, var = 0.0;
  for (long i = 0; i < d; ++i) mu += y[i];
  mu /= (double)d;
  for (long i = 0; i < d; ++i) {
    c[i] = y[i] - mu;
    var += c[i] * c[i];
  }
  var = var / (double)d;
  *rs = 1.0 / sqrt(eps + var);
}

/* adjoint of yh = LNhat(y) (yh = c rs, c = y - mean(y), rs = (mean(c^2) +
 * eps)^-1/2) given dyh and the extra adjoint drs0 of rs: returns dy */
static void ln_hat_adjoint(const double *c, double rs, const double *dyh, double drs0, long d,
                           double *dc, double *dy) {
  double drs = drs0;
  for (long i = 0; i < d; ++i) {
    dc[i] = rs * dyh[i];
    drs += c[i] * dyh[i];
  }
  const double dvar = -0.5 * rs * rs * rs * drs;
  double mdc = 0.0;
  for (long i = 0; i < d; ++i) {
    dc[i] += 2.0 / (double)d * c[i] * dvar;
    mdc += dc[i];
  }
  mdc /= (double)d;
  for (long i = 0; i < d; ++i) dy[i] = dc[i] - mdc;
}

static int linear_ln_bwd_unit(const double *q, const double *k, const double *v,
                              const double *eta, const double *w0, const double *gamma,
                              const double *beta, double eps, long T, long d, long b,
                              const double *dz, const double *dwT, double *dq, double *dk,
                              double *dv, double *deta, double *dw0, double *dgam, double *dbet) {
  const size_t dd = (size_t)(d * d);
  double *S = (double *)malloc(sizeof(double) * dd * (size_t)(T + 1));
  double *Ag = (double *)calloc(dd, sizeof(double));
  double *vec = (double *)malloc(sizeof(double) * (size_t)(16 * d));
  if (!S || !Ag || !vec) { free(S); free(Ag); free(vec); return 1; }
  double *y = vec, *c = y + d, *yh = c + d, *r = yh + d, *g = r + d, *dy = g + d;
  double *cq = dy + d, *yhq = cq + d, *dyh = yhq + d, *dc = dyh + d, *dyq = dc + d;
  double *Ak = dyq + d, *ddy = Ak + d, *dg = ddy + d, *dyv = dg + d, *tmp = dyv + d;
  (void)tmp;
  memcpy(S, w0, sizeof(double) * dd);
  /* forward, keeping every state */
  for (long t = 0; t < T; ++t) {
    const long m0 = (t / b) * b;
    const double *P = S + (size_t)m0 * dd, *C = S + (size_t)t * dd;
    double *N = S + (size_t)(t + 1) * dd;
    const double *kt = k + t * d, *vt = v + t * d;
    double rs;
    for (long i = 0; i < d; ++i) {
      double acc = 0.0;
      for (long j = 0; j < d; ++j) acc += P[i * d + j] * kt[j];
      y[i] = acc;
    }
    ln_stats(y, d, eps, c, &rs);
    double gbar = 0.0, m = 0.0;
    for (long i = 0; i < d; ++i) {
      yh[i] = c[i] * rs;
      g[i] = 2.0 * gamma[i] * (kt[i] + gamma[i] * yh[i] + beta[i] - vt[i]);
      gbar += g[i];
      m += g[i] * yh[i];
    }
    gbar /= (double)d;
    m /= (double)d;
    for (long i = 0; i < d; ++i) dy[i] = rs * (g[i] - gbar - yh[i] * m);
    for (long i = 0; i < d; ++i)
      for (long j = 0; j < d; ++j) N[i * d + j] = C[i * d + j] - eta[t] * dy[i] * kt[j];
  }
  /* reverse */
  double *A = dw0;
  if (dwT) memcpy(A, dwT, sizeof(double) * dd);
  else memset(A, 0, sizeof(double) * dd);
  memset(dgam, 0, sizeof(double) * (size_t)d);
  memset(dbet, 0, sizeof(double) * (size_t)d);
  for (long t = T - 1; t >= 0; --t) {
    const long m0 = (t / b) * b;
    const double *P = S + (size_t)m0 * dd, *N = S + (size_t)(t + 1) * dd;
    const double *kt = k + t * d, *vt = v + t * d, *qt = q + t * d, *zt = dz + t * d;
    const double et = eta[t];
    double rs, rsq;
    /* the token's forward quantities at the gradient point */
    for (long i = 0; i < d; ++i) {
      double acc = 0.0;
      for (long j = 0; j < d; ++j) acc += P[i * d + j] * kt[j];
      y[i] = acc;
    }
    ln_stats(y, d, eps, c, &rs);
    double gbar = 0.0, m = 0.0;
    for (long i = 0; i < d; ++i) {
      yh[i] = c[i] * rs;
      r[i] = kt[i] + gamma[i] * yh[i] + beta[i] - vt[i];
      g[i] = 2.0 * gamma[i] * r[i];
      gbar += g[i];
      m += g[i] * yh[i];
    }
    gbar /= (double)d;
    m /= (double)d;
    for (long i = 0; i < d; ++i) dy[i] = rs * (g[i] - gbar - yh[i] * m);
    /* output z = q + gamma LNhat(N q) + beta */
    for (long i = 0; i < d; ++i) {
      double acc = 0.0;
      for (long j = 0; j < d; ++j) acc += N[i * d + j] * qt[j];
      y[i] = acc;
    }
    ln_stats(y, d, eps, cq, &rsq);
    for (long i = 0; i < d; ++i) {
      yhq[i] = cq[i] * rsq;
      dyh[i] = gamma[i] * zt[i];
      dgam[i] += yhq[i] * zt[i];
      dbet[i] += zt[i];
    }
    ln_hat_adjoint(cq, rsq, dyh, 0.0, d, dc, dyq);
    for (long i = 0; i < d; ++i)
      for (long j = 0; j < d; ++j) A[i * d + j] += dyq[i] * qt[j];
    for (long j = 0; j < d; ++j) {
      double acc = zt[j]; /* the residual q */
      for (long i = 0; i < d; ++i) acc += N[i * d + j] * dyq[i];
      dq[t * d + j] = acc;
    }
    /* the update N = S[t] - eta dy k^T */
    double de = 0.0;
    for (long i = 0; i < d; ++i) {
      double acc = 0.0;
      for (long j = 0; j < d; ++j) acc += A[i * d + j] * kt[j];
      Ak[i] = acc;
      ddy[i] = -et * acc;
      de -= dy[i] * acc;
    }
    deta[t] = de;
    for (long j = 0; j < d; ++j) {
      double acc = 0.0;
      for (long i = 0; i < d; ++i) acc += A[i * d + j] * dy[i];
      dk[t * d + j] = -et * acc;
    }
    /* dy = rs (g - gbar - yh m) */
    double drs = 0.0, sdd = 0.0, dm = 0.0;
    for (long i = 0; i < d; ++i) {
      drs += ddy[i] * (g[i] - gbar - yh[i] * m);
      sdd += ddy[i];
      dm -= rs * ddy[i] * yh[i];
    }
    const double dgbar = -rs * sdd;
    for (long i = 0; i < d; ++i) {
      dg[i] = rs * ddy[i] + dm / (double)d * yh[i] + dgbar / (double)d; /* m, gbar */
      dyh[i] = -rs * m * ddy[i] + dm / (double)d * g[i];
    }
    /* g = 2 gamma r, r = f - v, f = k + gamma yh + beta */
    for (long i = 0; i < d; ++i) {
      const double dr = 2.0 * gamma[i] * dg[i];
      dgam[i] += 2.0 * r[i] * dg[i] + yh[i] * dr;
      dbet[i] += dr;
      dv[t * d + i] = -dr;
      dk[t * d + i] += dr;
      dyh[i] += gamma[i] * dr;
    }
    /* yh = LNhat(y), y = P k */
    ln_hat_adjoint(c, rs, dyh, drs, d, dc, dyv);
    for (long i = 0; i < d; ++i)
      for (long j = 0; j < d; ++j) Ag[i * d + j] += dyv[i] * kt[j];
    for (long j = 0; j < d; ++j) {
      double acc = 0.0;
      for (long i = 0; i < d; ++i) acc += P[i * d + j] * dyv[i];
      dk[t * d + j] += acc;
    }
    if (t == m0) { /* the gradient point of this mini-batch is the state before t */
      for (size_t e = 0; e < dd; ++e) {
        A[e] = A[e] + Ag[e];
        Ag[e] = 0.0;
      }
    }
  }
  free(S);
  free(Ag);
  free(vec);
  return 0;
}

int ttt_oracle_linear_ln_bwd(const double *q, const double *k, const double *v,
                             const double *eta, const double *w0, int w0_per_batch,
                             const double *gamma, const double *beta, double eps, long B, long H,
                             long T, long d, long b, const double *dz, const double *dwT,
                             double *dq, double *dk, double *dv, double *deta, double *dw0,
                             double *dgamma, double *dbeta) {
  if (B < 0 || H < 0 || T < 0 || d <= 0 || b <= 0 || !(eps >= 0.0)) return 2;
  for (long u = 0; u < B * H; ++u) {
    const long h = u % H, wsel = w0_per_batch ? u : h;
    const size_t so = (size_t)u * (size_t)(T * d);
    int rc = linear_ln_bwd_unit(q + so, k + so, v + so, eta + (size_t)u * (size_t)T,
                                w0 + (size_t)wsel * (size_t)(d * d), gamma + (size_t)h * (size_t)d,
                                beta + (size_t)h * (size_t)d, eps, T, d, b, dz + so,
                                dwT ? dwT + (size_t)u * (size_t)(d * d) : NULL, dq + so, dk + so,
                                dv + so, deta + (size_t)u * (size_t)T,
                                dw0 + (size_t)u * (size_t)(d * d), dgamma + (size_t)u * (size_t)d,
                                dbeta + (size_t)u * (size_t)d);
    if (rc) return rc;
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* TTT-MLP backward: reverse pass of the primal recurrence.            */
/* ------------------------------------------------------------------ */
/* d^2/dx^2 [x Phi(x)] = 2 phi(x) + x phi'(x) = phi(x) (2 - x^2) */
static double gelu_grad2(double x) {
  const double pi = 3.14159265358979323846;
  return exp(-0.5 * x * x) / sqrt(2.0 * pi) * (2.0 - x * x);
}

/* Forward, one unit (as mlp_unit), keeping every state: S1[t], S2[t] are W1,
 * W2 after t tokens; token t of the mini-batch starting at m0 takes
 *   a = S1[m0] k_t, x = GELU(a), e = 2 (S2[m0] x - v_t),
 *   s = S2[m0]^T e, delta = s * GELU'(a),
 *   S1[t+1] = S1[t] - eta_t delta k_t^T,  S2[t+1] = S2[t] - eta_t e x^T,
 *   z_t = S2[t+1] GELU(S1[t+1] q_t).
 * Reverse, with A1, A2 the adjoints of the state after token t (starting
 * from those of the final state) and G1, G2 the adjoints collected for the
 * current mini-batch's gradient point (S1[m0], S2[m0]); for token t:
 *   output:  aq = S1[t+1] q, xq = GELU(aq); A2 += dz xq^T;
 *            daq = (S2[t+1]^T dz) * GELU'(aq); A1 += daq q^T;
 *            dq = S1[t+1]^T daq;
 *   update:  ddelta = -eta A1 k, dk = -eta A1^T delta, de = -eta A2 x,
 *            dx = -eta A2^T e, deta = -delta^T A1 k - e^T A2 x;
 *   delta:   ds = ddelta * GELU'(a), da = ddelta * s * GELU''(a);
 *   s:       G2 += e ds^T, de += S2[m0] ds;
 *   e:       dv = -2 de;  y = S2[m0] x:  G2 += 2 de x^T, dx += 2 S2[m0]^T de;
 *   x:       da += dx * GELU'(a);
 *   a:       G1 += da k^T, dk += S1[m0]^T da;
 *   at t = m0: A1 += G1, A2 += G2, G1 = G2 = 0.
 * The adjoints then carry over unchanged to the state before token t. */
static int mlp_bwd_unit(const double *q, const double *k, const double *v, const double *eta,
                        const double *w1_0, const double *w2_0, long T, long d, long hd, long b,
                        const double *dz, const double *dw1T, const double *dw2T, double *dq,
                        double *dk, double *dv, double *deta, double *dw1_0, double *dw2_0) {
  const size_t n = (size_t)(hd * d);
  double *S1 = (double *)malloc(sizeof(double) * n * (size_t)(T + 1));
  double *S2 = (double *)malloc(sizeof(double) * n * (size_t)(T + 1));
  double *G1 = (double *)calloc(n, sizeof(double));
  double *G2 = (double *)calloc(n, sizeof(double));
  double *vec = (double *)malloc(sizeof(double) * (size_t)(11 * hd + 2 * d));
  if (!S1 || !S2 || !G1 || !G2 || !vec) {
    free(S1); free(S2); free(G1); free(G2); free(vec);
    return 1;
  }
  double *a = vec, *x = a + hd, *s = x + hd, *dl = s + hd, *aq = dl + hd, *xq = aq + hd;
  double *daq = xq + hd, *ddl = daq + hd, *ds = ddl + hd, *da = ds + hd, *dx = da + hd;
  double *e = dx + hd, *de = e + d;
  memcpy(S1, w1_0, sizeof(double) * n);
  memcpy(S2, w2_0, sizeof(double) * n);
  /* forward, keeping every state */
  for (long t = 0; t < T; ++t) {
    const long m0 = (t / b) * b;
    const double *P1 = S1 + (size_t)m0 * n, *P2 = S2 + (size_t)m0 * n;
    const double *C1 = S1 + (size_t)t * n, *C2 = S2 + (size_t)t * n;
    double *N1 = S1 + (size_t)(t + 1) * n, *N2 = S2 + (size_t)(t + 1) * n;
    const double *kt = k + t * d, *vt = v + t * d;
    for (long u = 0; u < hd; ++u) {
      double acc = 0.0;
      for (long j = 0; j < d; ++j) acc += P1[u * d + j] * kt[j];
      a[u] = acc;
      x[u] = gelu(acc);
    }
    for (long i = 0; i < d; ++i) {
      double acc = 0.0;
      for (long u = 0; u < hd; ++u) acc += P2[i * hd + u] * x[u];
      e[i] = 2.0 * (acc - vt[i]);
    }
    for (long u = 0; u < hd; ++u) {
      double acc = 0.0;
      for (long i = 0; i < d; ++i) acc += P2[i * hd + u] * e[i];
      dl[u] = acc * gelu_grad(a[u]);
    }
    for (long i = 0; i < d; ++i)
      for (long u = 0; u < hd; ++u) N2[i * hd + u] = C2[i * hd + u] - eta[t] * e[i] * x[u];
    for (long u = 0; u < hd; ++u)
      for (long j = 0; j < d; ++j) N1[u * d + j] = C1[u * d + j] - eta[t] * dl[u] * kt[j];
  }
  /* reverse */
  double *A1 = dw1_0, *A2 = dw2_0; /* the running adjoints live in the outputs */
  if (dw1T) memcpy(A1, dw1T, sizeof(double) * n);
  else memset(A1, 0, sizeof(double) * n);
  if (dw2T) memcpy(A2, dw2T, sizeof(double) * n);
  else memset(A2, 0, sizeof(double) * n);
  for (long t = T - 1; t >= 0; --t) {
    const long m0 = (t / b) * b;
    const double *P1 = S1 + (size_t)m0 * n, *P2 = S2 + (size_t)m0 * n;
    const double *N1 = S1 + (size_t)(t + 1) * n, *N2 = S2 + (size_t)(t + 1) * n;
    const double *kt = k + t * d, *vt = v + t * d, *qt = q + t * d, *zt = dz + t * d;
    const double et = eta[t];
    /* forward quantities of token t at the gradient point */
    for (long u = 0; u < hd; ++u) {
      double acc = 0.0;
      for (long j = 0; j < d; ++j) acc += P1[u * d + j] * kt[j];
      a[u] = acc;
      x[u] = gelu(acc);
    }
    for (long i = 0; i < d; ++i) {
      double acc = 0.0;
      for (long u = 0; u < hd; ++u) acc += P2[i * hd + u] * x[u];
      e[i] = 2.0 * (acc - vt[i]);
    }
    for (long u = 0; u < hd; ++u) {
      double acc = 0.0;
      for (long i = 0; i < d; ++i) acc += P2[i * hd + u] * e[i];
      s[u] = acc;
      dl[u] = acc * gelu_grad(a[u]);
    }
    /* output z_t = N2 GELU(N1 q_t) */
    for (long u = 0; u < hd; ++u) {
      double acc = 0.0;
      for (long j = 0; j < d; ++j) acc += N1[u * d + j] * qt[j];
      aq[u] = acc;
      xq[u] = gelu(acc);
    }
    for (long i = 0; i < d; ++i)
      for (long u = 0; u < hd; ++u) A2[i * hd + u] += zt[i] * xq[u];
    for (long u = 0; u < hd; ++u) {
      double acc = 0.0;
      for (long i = 0; i < d; ++i) acc += N2[i * hd + u] * zt[i];
      daq[u] = acc * gelu_grad(aq[u]);
    }
    for (long u = 0; u < hd; ++u)
      for (long j = 0; j < d; ++j) A1[u * d + j] += daq[u] * qt[j];
    for (long j = 0; j < d; ++j) {
      double acc = 0.0;
      for (long u = 0; u < hd; ++u) acc += N1[u * d + j] * daq[u];
      dq[t * d + j] = acc;
    }
    /* the updates N1 = S1[t] - eta delta k^T, N2 = S2[t] - eta e x^T */
    double dsum = 0.0;
    for (long u = 0; u < hd; ++u) {
      double acc = 0.0;
      for (long j = 0; j < d; ++j) acc += A1[u * d + j] * kt[j];
      ddl[u] = -et * acc;
      dsum -= dl[u] * acc;
    }
    for (long j = 0; j < d; ++j) {
      double acc = 0.0;
      for (long u = 0; u < hd; ++u) acc += A1[u * d + j] * dl[u];
      dk[t * d + j] = -et * acc;
    }
    for (long i = 0; i < d; ++i) {
      double acc = 0.0;
      for (long u = 0; u < hd; ++u) acc += A2[i * hd + u] * x[u];
      de[i] = -et * acc;
      dsum -= e[i] * acc;
    }
    for (long u = 0; u < hd; ++u) {
      double acc = 0.0;
      for (long i = 0; i < d; ++i) acc += A2[i * hd + u] * e[i];
      dx[u] = -et * acc;
    }
    deta[t] = dsum;
    /* delta = s * GELU'(a) */
    for (long u = 0; u < hd; ++u) {
      ds[u] = ddl[u] * gelu_grad(a[u]);
      da[u] = ddl[u] * s[u] * gelu_grad2(a[u]);
    }
    /* s = P2^T e */
    for (long i = 0; i < d; ++i) {
      double acc = 0.0;
      for (long u = 0; u < hd; ++u) {
        G2[i * hd + u] += e[i] * ds[u];
        acc += P2[i * hd + u] * ds[u];
      }
      de[i] += acc;
    }
    /* e = 2 (y - v), y = P2 x */
    for (long i = 0; i < d; ++i) {
      dv[t * d + i] = -2.0 * de[i];
      for (long u = 0; u < hd; ++u) G2[i * hd + u] += 2.0 * de[i] * x[u];
    }
    for (long u = 0; u < hd; ++u) {
      double acc = 0.0;
      for (long i = 0; i < d; ++i) acc += P2[i * hd + u] * de[i];
      dx[u] += 2.0 * acc;
    }
    /* x = GELU(a), a = P1 k */
    for (long u = 0; u < hd; ++u) {
      da[u] += dx[u] * gelu_grad(a[u]);
      for (long j = 0; j < d; ++j) G1[u * d + j] += da[u] * kt[j];
    }
    for (long j = 0; j < d; ++j) {
      double acc = 0.0;
      for (long u = 0; u < hd; ++u) acc += P1[u * d + j] * da[u];
      dk[t * d + j] += acc;
    }
    if (t == m0) { /* the gradient point of this mini-batch is the state before t */
      for (size_t i = 0; i < n; ++i) {
        A1[i] += G1[i];
        A2[i] += G2[i];
        G1[i] = 0.0;
        G2[i] = 0.0;
      }
    }
  }
  free(S1); free(S2); free(G1); free(G2); free(vec);
  return 0;
}

int ttt_oracle_mlp_bwd(const double *q, const double *k, const double *v, const double *eta,
                       const double *w1_0, const double *w2_0, int w0_per_batch, long B, long H,
                       long T, long d, long hd, long b, const double *dz, const double *dw1T,
                       const double *dw2T, double *dq, double *dk, double *dv, double *deta,
                       double *dw1_0, double *dw2_0) {
  if (B < 0 || H < 0 || T < 0 || d <= 0 || hd <= 0 || b <= 0) return 2;
  const size_t n = (size_t)(hd * d);
  for (long u = 0; u < B * H; ++u) {
    const long wsel = w0_per_batch ? u : u % H;
    const size_t so = (size_t)u * (size_t)(T * d);
    int rc = mlp_bwd_unit(q + so, k + so, v + so, eta + (size_t)u * (size_t)T,
                          w1_0 + (size_t)wsel * n, w2_0 + (size_t)wsel * n, T, d, hd, b, dz + so,
                          dw1T ? dw1T + (size_t)u * n : NULL, dw2T ? dw2T + (size_t)u * n : NULL,
                          dq + so, dk + so, dv + so, deta + (size_t)u * (size_t)T,
                          dw1_0 + (size_t)u * n, dw2_0 + (size_t)u * n);
    if (rc) return rc;
  }
  return 0;
}

/* §4.6: eta[b][h][t] = eta_base * sigmoid(theta_lr[h] . x[b][t]), the dot
 * product summed in order in fp64. */
int ttt_oracle_lr_gate(const double *x, const double *theta, double eta_base, long B, long T,
                       long H, long dx, double *eta) {
  if (B < 0 || T < 0 || H < 0 || dx <= 0) return 2;
  for (long bi = 0; bi < B; ++bi)
    for (long h = 0; h < H; ++h)
      for (long t = 0; t < T; ++t) {
        const double *xt = x + ((size_t)bi * (size_t)T + (size_t)t) * (size_t)dx;
        const double *th = theta + (size_t)h * (size_t)dx;
        double a = 0.0;
        for (long i = 0; i < dx; ++i) a += th[i] * xt[i];
        eta[((size_t)bi * (size_t)H + (size_t)h) * (size_t)T + (size_t)t] =
            eta_base / (1.0 + exp(-a));
      }
  return 0;
}

/* Backward of the gate above: deta [B][H][T] -> dtheta [H][dx], dx [B][T][dx]
 * (both overwritten), recomputing the logits in fp64. */
int ttt_oracle_lr_gate_bwd(const double *x, const double *theta, double eta_base,
                           const double *deta, long B, long T, long H, long dx, double *dtheta,
                           double *dxo) {
  if (B < 0 || T < 0 || H < 0 || dx <= 0) return 2;
  memset(dtheta, 0, sizeof(double) * (size_t)(H * dx));
  memset(dxo, 0, sizeof(double) * (size_t)(B * T * dx));
  for (long bi = 0; bi < B; ++bi)
    for (long t = 0; t < T; ++t) {
      const size_t tok = (size_t)bi * (size_t)T + (size_t)t;
      const double *xt = x + tok * (size_t)dx;
      double *gx = dxo + tok * (size_t)dx;
      for (long h = 0; h < H; ++h) {
        const double *th = theta + (size_t)(h * dx);
        double a = 0.0;
        for (long i = 0; i < dx; ++i) a += th[i] * xt[i];
        const double sg = 1.0 / (1.0 + exp(-a));
        const size_t gi = ((size_t)bi * (size_t)H + (size_t)h) * (size_t)T + (size_t)t;
        const double da = deta[gi] * eta_base * sg * (1.0 - sg);
        for (long i = 0; i < dx; ++i) {
          dtheta[(size_t)h * (size_t)dx + (size_t)i] += da * xt[i];
          gx[i] += da * th[i];
        }
      }
    }
  return 0;
}
