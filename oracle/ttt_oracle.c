/*
 * TEST INFRASTRUCTURE -- fp64 CPU oracle of the TTT layer forward pass.
 * Only tests/, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no code with the HIP library and is never on the product path.
 *
 * Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，
 * 一夜推翻Transformer" (aharts.cn / itmax.cn).
 *
 * What it computes is the *primal* form, token by token, in fp64:
 *   - the hidden state is the weight W of a model f; the output for token t is
 *     f applied to x_t with the already-updated W_t, and the update is one
 *     gradient step of size eta on a self-supervised loss
 *     ([TTT] 03 §1 "TTT hidden state");
 *   - the loss is the multi-view reconstruction |f(k_t; W) - v_t|^2 and the
 *     output uses the query view q_t ([TTT] 03 §5 "self-supervised task");
 *   - mini-batch GD: every gradient of mini-batch n is taken at the W held
 *     just before the first token of that mini-batch ([TTT] 03 §6);
 *   - TTT-Linear: f(x) = W x with W square; TTT-MLP: two layers, hidden width
 *     dh, GELU in between ([TTT] 03 §9 "two variants");
 *   - with layer norm and residual (03 §9: f always has them for stability):
 *     f(x) = x + LN(W x), LN(y) = gamma * (y - mean(y)) / sqrt(var(y) + eps) + beta
 *     over the d outputs (var the biased mean of squares), gamma/beta per head.
 * The gradient of |W k - v|^2 with respect to W is 2 (W k - v) k^T (summed
 * squared error, no 1/2, no 1/d).  GELU is the exact form x * Phi(x).
 *
 * Layouts (all fp64, caller-expanded per chain, row-major):
 *   q, k, v, z : [n, T, d]        eta : [n, T]
 *   linear: w0, wf : [n, d, d]    (z = W q)
 *   mlp:    w1 : [n, dh, d]  w2 : [n, d, dh]
 * A final mini-batch shorter than b (T % b != 0) is handled by the same rule.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_abi_version(void) { return 1; }

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* y = M x, M is rows x cols row-major */
static void matvec(const double* M, const double* x, double* y, int rows, int cols) {
  for (int i = 0; i < rows; ++i) {
    double s = 0.0;
    const double* m = M + (size_t)i * cols;
    for (int c = 0; c < cols; ++c) s += m[c] * x[c];
    y[i] = s;
  }
}

/* y = M^T x, M is rows x cols row-major, y has cols entries */
static void matvec_t(const double* M, const double* x, double* y, int rows, int cols) {
  for (int c = 0; c < cols; ++c) y[c] = 0.0;
  for (int i = 0; i < rows; ++i) {
    const double* m = M + (size_t)i * cols;
    for (int c = 0; c < cols; ++c) y[c] += m[c] * x[i];
  }
}

/* M -= a * u v^T  (rank one), M rows x cols */
static void rank1_sub(double* M, double a, const double* u, const double* v, int rows, int cols) {
  for (int i = 0; i < rows; ++i) {
    double ai = a * u[i];
    double* m = M + (size_t)i * cols;
    for (int c = 0; c < cols; ++c) m[c] -= ai * v[c];
  }
}

static double gelu(double x) { return 0.5 * x * (1.0 + erf(x / sqrt(2.0))); }
static double gelu_prime(double x) {
  const double inv_sqrt_2pi = 0.39894228040143267794;
  return 0.5 * (1.0 + erf(x / sqrt(2.0))) + x * inv_sqrt_2pi * exp(-0.5 * x * x);
}

/* TTT-Linear primal form for n independent chains. */
void oracle_linear_primal(int n, int T, int d, int b,
                          const double* q, const double* k, const double* v,
                          const double* w0, const double* eta,
                          double* z, double* wf, int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int c = 0; c < n; ++c) {
    const size_t dd = (size_t)d * d;
    double* W = (double*)malloc(dd * sizeof(double));
    double* Wb = (double*)malloc(dd * sizeof(double));
    double* e = (double*)malloc((size_t)d * sizeof(double));
    memcpy(W, w0 + c * dd, dd * sizeof(double));
    for (int t0 = 0; t0 < T; t0 += b) {
      memcpy(Wb, W, dd * sizeof(double)); /* state at the start of the mini-batch */
      int t1 = t0 + b < T ? t0 + b : T;
      for (int t = t0; t < t1; ++t) {
        const size_t o = ((size_t)c * T + t) * d;
        matvec(Wb, k + o, e, d, d);                      /* e = Wb k_t - v_t */
        for (int i = 0; i < d; ++i) e[i] -= v[o + i];
        rank1_sub(W, 2.0 * eta[(size_t)c * T + t], e, k + o, d, d); /* W -= eta * 2 e k^T */
        matvec(W, q + o, z + o, d, d);                   /* z_t = W_t q_t */
      }
    }
    memcpy(wf + c * dd, W, dd * sizeof(double));
    free(W); free(Wb); free(e);
  }
}

/* TTT-MLP primal form: f(x) = W2 GELU(W1 x), W1 dh x d, W2 d x dh. */
void oracle_mlp_primal(int n, int T, int d, int dh, int b,
                       const double* q, const double* k, const double* v,
                       const double* w1_0, const double* w2_0, const double* eta,
                       double* z, double* w1f, double* w2f, int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int c = 0; c < n; ++c) {
    const size_t sz = (size_t)dh * d;
    double* W1 = (double*)malloc(sz * sizeof(double));
    double* W2 = (double*)malloc(sz * sizeof(double));
    double* W1b = (double*)malloc(sz * sizeof(double));
    double* W2b = (double*)malloc(sz * sizeof(double));
    double* h = (double*)malloc((size_t)dh * sizeof(double));
    double* a = (double*)malloc((size_t)dh * sizeof(double));
    double* g1 = (double*)malloc((size_t)dh * sizeof(double));
    double* e = (double*)malloc((size_t)d * sizeof(double));
    memcpy(W1, w1_0 + c * sz, sz * sizeof(double));
    memcpy(W2, w2_0 + c * sz, sz * sizeof(double));
    for (int t0 = 0; t0 < T; t0 += b) {
      memcpy(W1b, W1, sz * sizeof(double));
      memcpy(W2b, W2, sz * sizeof(double));
      int t1 = t0 + b < T ? t0 + b : T;
      for (int t = t0; t < t1; ++t) {
        const size_t o = ((size_t)c * T + t) * d;
        const double et = eta[(size_t)c * T + t];
        /* forward of the reconstruction at the mini-batch-start weights */
        matvec(W1b, k + o, h, dh, d);
        for (int j = 0; j < dh; ++j) a[j] = gelu(h[j]);
        matvec(W2b, a, e, d, dh);
        for (int i = 0; i < d; ++i) e[i] = 2.0 * (e[i] - v[o + i]); /* dl/d(out) */
        /* back-propagate to the hidden pre-activation */
        matvec_t(W2b, e, g1, d, dh);
        for (int j = 0; j < dh; ++j) g1[j] *= gelu_prime(h[j]);
        /* one gradient step on both layers */
        rank1_sub(W2, et, e, a, d, dh);
        rank1_sub(W1, et, g1, k + o, dh, d);
        /* output with the updated weights */
        matvec(W1, q + o, h, dh, d);
        for (int j = 0; j < dh; ++j) a[j] = gelu(h[j]);
        matvec(W2, a, z + o, d, dh);
      }
    }
    memcpy(w1f + c * sz, W1, sz * sizeof(double));
    memcpy(w2f + c * sz, W2, sz * sizeof(double));
    free(W1); free(W2); free(W1b); free(W2b); free(h); free(a); free(g1); free(e);
  }
}

/* LN over d values: yhat = (y - mu) / s, s = sqrt(var + eps); returns s. */
static double ln_normalize(const double* y, double* yhat, int d, double eps) {
  double mu = 0.0;
  for (int i = 0; i < d; ++i) mu += y[i];
  mu /= d;
  double var = 0.0;
  for (int i = 0; i < d; ++i) var += (y[i] - mu) * (y[i] - mu);
  var /= d;
  const double s = sqrt(var + eps);
  for (int i = 0; i < d; ++i) yhat[i] = (y[i] - mu) / s;
  return s;
}

/* TTT-Linear with LN and residual, f(x) = x + LN(W x), primal form.
 * gamma, beta : [n, d] (per chain).  The gradient of |f(k) - v|^2 with respect
 * to W is delta k^T, where delta is the loss gradient back-propagated through
 * LN to y = W k:  g = 2 (f(k) - v) * gamma,
 * delta = (g - mean(g) - yhat * mean(g * yhat)) / s. */
void oracle_linear_ln_primal(int n, int T, int d, int b,
                             const double* q, const double* k, const double* v,
                             const double* w0, const double* gamma, const double* beta, double eps,
                             const double* eta, double* z, double* wf, int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int c = 0; c < n; ++c) {
    const size_t dd = (size_t)d * d;
    const double* gm = gamma + (size_t)c * d;
    const double* bt = beta + (size_t)c * d;
    double* W = (double*)malloc(dd * sizeof(double));
    double* Wb = (double*)malloc(dd * sizeof(double));
    double* y = (double*)malloc((size_t)d * sizeof(double));
    double* yh = (double*)malloc((size_t)d * sizeof(double));
    double* g = (double*)malloc((size_t)d * sizeof(double));
    memcpy(W, w0 + c * dd, dd * sizeof(double));
    for (int t0 = 0; t0 < T; t0 += b) {
      memcpy(Wb, W, dd * sizeof(double));
      int t1 = t0 + b < T ? t0 + b : T;
      for (int t = t0; t < t1; ++t) {
        const size_t o = ((size_t)c * T + t) * d;
        /* reconstruction of v_t from k_t at the mini-batch-start state */
        matvec(Wb, k + o, y, d, d);
        const double s = ln_normalize(y, yh, d, eps);
        double mg = 0.0, mgy = 0.0;
        for (int i = 0; i < d; ++i) {
          const double r = k[o + i] + gm[i] * yh[i] + bt[i] - v[o + i];
          g[i] = 2.0 * r * gm[i];
          mg += g[i];
          mgy += g[i] * yh[i];
        }
        mg /= d;
        mgy /= d;
        for (int i = 0; i < d; ++i) g[i] = (g[i] - mg - yh[i] * mgy) / s; /* delta */
        rank1_sub(W, eta[(size_t)c * T + t], g, k + o, d, d);
        /* output with the updated state */
        matvec(W, q + o, y, d, d);
        ln_normalize(y, yh, d, eps);
        for (int i = 0; i < d; ++i) z[o + i] = q[o + i] + gm[i] * yh[i] + bt[i];
      }
    }
    memcpy(wf + c * dd, W, dd * sizeof(double));
    free(W); free(Wb); free(y); free(yh); free(g);
  }
}

/* TTT-MLP with LN and residual, f(x) = x + LN(W2 GELU(W1 x)), primal form.
 * gamma, beta : [n, d] (per chain).  The loss |f(k) - v|^2 is pulled back
 * through LN to y = W2 GELU(W1 k) as for TTT-Linear with LN:
 *   g = 2 (f(k) - v) * gamma,  delta = (g - mean(g) - yhat * mean(g * yhat)) / s,
 * and through the two layers as for plain TTT-MLP with delta in place of
 * 2 (y - v): the W2 gradient is delta a^T and the W1 gradient
 * ((W2^T delta) * GELU'(h)) k^T, both at the mini-batch-start weights. */
void oracle_mlp_ln_primal(int n, int T, int d, int dh, int b,
                          const double* q, const double* k, const double* v,
                          const double* w1_0, const double* w2_0,
                          const double* gamma, const double* beta, double eps, const double* eta,
                          double* z, double* w1f, double* w2f, int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int c = 0; c < n; ++c) {
    const size_t sz = (size_t)dh * d;
    const double* gm = gamma + (size_t)c * d;
    const double* bt = beta + (size_t)c * d;
    double* W1 = (double*)malloc(sz * sizeof(double));
    double* W2 = (double*)malloc(sz * sizeof(double));
    double* W1b = (double*)malloc(sz * sizeof(double));
    double* W2b = (double*)malloc(sz * sizeof(double));
    double* h = (double*)malloc((size_t)dh * sizeof(double));
    double* a = (double*)malloc((size_t)dh * sizeof(double));
    double* g1 = (double*)malloc((size_t)dh * sizeof(double));
    double* y = (double*)malloc((size_t)d * sizeof(double));
    double* yh = (double*)malloc((size_t)d * sizeof(double));
    double* dl = (double*)malloc((size_t)d * sizeof(double));
    memcpy(W1, w1_0 + c * sz, sz * sizeof(double));
    memcpy(W2, w2_0 + c * sz, sz * sizeof(double));
    for (int t0 = 0; t0 < T; t0 += b) {
      memcpy(W1b, W1, sz * sizeof(double));
      memcpy(W2b, W2, sz * sizeof(double));
      int t1 = t0 + b < T ? t0 + b : T;
      for (int t = t0; t < t1; ++t) {
        const size_t o = ((size_t)c * T + t) * d;
        const double et = eta[(size_t)c * T + t];
        /* reconstruction of v_t from k_t at the mini-batch-start weights */
        matvec(W1b, k + o, h, dh, d);
        for (int j = 0; j < dh; ++j) a[j] = gelu(h[j]);
        matvec(W2b, a, y, d, dh);
        const double s = ln_normalize(y, yh, d, eps);
        double mg = 0.0, mgy = 0.0;
        for (int i = 0; i < d; ++i) {
          dl[i] = 2.0 * (k[o + i] + gm[i] * yh[i] + bt[i] - v[o + i]) * gm[i];
          mg += dl[i];
          mgy += dl[i] * yh[i];
        }
        mg /= d;
        mgy /= d;
        for (int i = 0; i < d; ++i) dl[i] = (dl[i] - mg - yh[i] * mgy) / s; /* dl/dy */
        matvec_t(W2b, dl, g1, d, dh);
        for (int j = 0; j < dh; ++j) g1[j] *= gelu_prime(h[j]);
        rank1_sub(W2, et, dl, a, d, dh);
        rank1_sub(W1, et, g1, k + o, dh, d);
        /* output with the updated weights */
        matvec(W1, q + o, h, dh, d);
        for (int j = 0; j < dh; ++j) a[j] = gelu(h[j]);
        matvec(W2, a, y, d, dh);
        ln_normalize(y, yh, d, eps);
        for (int i = 0; i < d; ++i) z[o + i] = q[o + i] + gm[i] * yh[i] + bt[i];
      }
    }
    memcpy(w1f + c * sz, W1, sz * sizeof(double));
    memcpy(w2f + c * sz, W2, sz * sizeof(double));
    free(W1); free(W2); free(W1b); free(W2b); free(h); free(a); free(g1); free(y); free(yh); free(dl);
  }
}

/* Gradients of TTT-Linear by reverse-mode differentiation of the primal token
 * loop above (fp64), for L = sum(dz * Z) + sum(dwf * W_final):
 *   dq, dk, dv : [n, T, d]   deta : [n, T]   dw0 : [n, d, d]   (dwf may be NULL).
 * The loop's states are recomputed per mini-batch from stored mini-batch-start
 * states.  Token t of the loop does  e_t = Wb k_t - v_t,
 * W_t = W_{t-1} - 2 eta_t e_t k_t^T,  z_t = W_t q_t  (Wb: state at the start of
 * t's mini-batch, which is also W_{t-1} for its first token), so walking back
 * with A = dL/dW_t:
 *   A += dz_t q_t^T;  dq_t = W_t^T dz_t
 *   de_t = -2 eta_t A k_t;  dk_t = -2 eta_t A^T e_t + Wb^T de_t
 *   deta_t = -2 e_t . (A k_t);  dv_t = -de_t;  dWb += de_t k_t^T
 * and A_{t-1} = A_t; at the mini-batch start A += dWb. */
void oracle_linear_primal_grads(int n, int T, int d, int b,
                                const double* q, const double* k, const double* v,
                                const double* w0, const double* eta,
                                const double* dz, const double* dwf,
                                double* dq, double* dk, double* dv, double* deta, double* dw0,
                                int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int c = 0; c < n; ++c) {
    const size_t dd = (size_t)d * d;
    const int nb = (T + b - 1) / b;
    double* Wst = (double*)malloc((size_t)(nb > 0 ? nb : 1) * dd * sizeof(double));
    double* W = (double*)malloc(dd * sizeof(double));
    double* Wt = (double*)malloc((size_t)b * dd * sizeof(double));
    double* E = (double*)malloc((size_t)b * d * sizeof(double));
    double* A = (double*)malloc(dd * sizeof(double));
    double* dWb = (double*)malloc(dd * sizeof(double));
    double* ak = (double*)malloc((size_t)d * sizeof(double));
    double* de = (double*)malloc((size_t)d * sizeof(double));
    double* tmp = (double*)malloc((size_t)d * sizeof(double));
    const double* et = eta + (size_t)c * T;

    /* forward: the state at every mini-batch start */
    memcpy(W, w0 + c * dd, dd * sizeof(double));
    for (int mb = 0; mb < nb; ++mb) {
      double* Wb = Wst + (size_t)mb * dd;
      memcpy(Wb, W, dd * sizeof(double));
      const int t0 = mb * b, t1 = t0 + b < T ? t0 + b : T;
      for (int t = t0; t < t1; ++t) {
        const size_t o = ((size_t)c * T + t) * d;
        matvec(Wb, k + o, tmp, d, d);
        for (int i = 0; i < d; ++i) tmp[i] -= v[o + i];
        rank1_sub(W, 2.0 * et[t], tmp, k + o, d, d);
      }
    }

    /* backward */
    if (dwf) memcpy(A, dwf + c * dd, dd * sizeof(double));
    else memset(A, 0, dd * sizeof(double));
    for (int mb = nb - 1; mb >= 0; --mb) {
      const double* Wb = Wst + (size_t)mb * dd;
      const int t0 = mb * b, t1 = t0 + b < T ? t0 + b : T;
      /* recompute the mini-batch: e_t and W_t */
      memcpy(W, Wb, dd * sizeof(double));
      for (int t = t0; t < t1; ++t) {
        const size_t o = ((size_t)c * T + t) * d;
        double* e = E + (size_t)(t - t0) * d;
        matvec(Wb, k + o, e, d, d);
        for (int i = 0; i < d; ++i) e[i] -= v[o + i];
        rank1_sub(W, 2.0 * et[t], e, k + o, d, d);
        memcpy(Wt + (size_t)(t - t0) * dd, W, dd * sizeof(double));
      }
      memset(dWb, 0, dd * sizeof(double));
      for (int t = t1 - 1; t >= t0; --t) {
        const size_t o = ((size_t)c * T + t) * d;
        const double* e = E + (size_t)(t - t0) * d;
        const double* Wc = Wt + (size_t)(t - t0) * dd;
        matvec_t(Wc, dz + o, dq + o, d, d);               /* dq_t = W_t^T dz_t */
        rank1_sub(A, -1.0, dz + o, q + o, d, d);          /* A += dz_t q_t^T   */
        matvec(A, k + o, ak, d, d);                       /* A k_t             */
        double s = 0.0;
        for (int i = 0; i < d; ++i) {
          de[i] = -2.0 * et[t] * ak[i];
          s += e[i] * ak[i];
        }
        deta[(size_t)c * T + t] = -2.0 * s;
        matvec_t(A, e, dk + o, d, d);                     /* A^T e_t           */
        matvec_t(Wb, de, tmp, d, d);                      /* Wb^T de_t         */
        for (int i = 0; i < d; ++i) {
          dk[o + i] = -2.0 * et[t] * dk[o + i] + tmp[i];
          dv[o + i] = -de[i];
        }
        rank1_sub(dWb, -1.0, de, k + o, d, d);            /* dWb += de_t k_t^T */
      }
      for (size_t x = 0; x < dd; ++x) A[x] += dWb[x];
    }
    memcpy(dw0 + c * dd, A, dd * sizeof(double));
    free(Wst); free(W); free(Wt); free(E); free(A); free(dWb); free(ak); free(de); free(tmp);
  }
}

/* Gradients of TTT-Linear with LN and residual inside f (oracle_linear_ln_primal)
 * by reverse-mode differentiation of its primal token loop (fp64), for
 * L = sum(dz * Z) + sum(dwf * W_final):
 *   dq, dk, dv : [n, T, d]   deta : [n, T]   dw0 : [n, d, d]
 *   dgamma, dbeta : [n, d]   (per chain; dwf may be NULL).
 * Token t of the loop (Wb: the state before t's mini-batch):
 *   y = Wb k,  yhat = (y - mean y) / s,  r = k + gamma yhat + beta - v,
 *   g = 2 r gamma,  c = mean(g yhat),  delta = (g - mean g - yhat c) / s,
 *   W_t = W_{t-1} - eta_t delta k^T,  u = W_t q,  z = q + gamma uhat + beta.
 * Walking back with A = dL/dW_t (the LN backward of a vector x with adjoint
 * h is  (h - mean h - xhat mean(h xhat)) / s_x):
 *   dq = dz;  dgamma += dz uhat;  dbeta += dz;  du = LNback(u, gamma dz)
 *   A += du q^T;  dq += W_t^T du
 *   a = -eta_t A k;  dk = -eta_t A^T delta;  deta_t = delta . (A k) * -1
 *   dg = LNback-projection of a (P a / s, P = I - 11^T/d - yhat yhat^T/d);
 *   dy = -(a . delta) yhat / (s d) - c (P a) / s^2 - (a . yhat) delta / (s d)
 *        (the derivative of delta in y at fixed g)
 *   dr = 2 gamma dg;  dgamma += 2 r dg + dr yhat;  dbeta += dr;  dk += dr;
 *   dv = -dr;  dy += LNback(y, gamma dr)
 *   dWb += dy k^T;  dk += Wb^T dy
 * and at the mini-batch start A += dWb. */
static void ln_back(const double* h, const double* xh, double s, double* out, int d) {
  double m = 0.0, mh = 0.0;
  for (int i = 0; i < d; ++i) {
    m += h[i];
    mh += h[i] * xh[i];
  }
  m /= d;
  mh /= d;
  for (int i = 0; i < d; ++i) out[i] = (h[i] - m - xh[i] * mh) / s;
}

void oracle_linear_ln_primal_grads(int n, int T, int d, int b,
                                   const double* q, const double* k, const double* v,
                                   const double* w0, const double* gamma, const double* beta, double eps,
                                   const double* eta, const double* dz, const double* dwf,
                                   double* dq, double* dk, double* dv, double* deta, double* dw0,
                                   double* dgamma, double* dbeta, int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int c = 0; c < n; ++c) {
    const size_t dd = (size_t)d * d;
    const int nb = (T + b - 1) / b;
    const double* gm = gamma + (size_t)c * d;
    const double* bt = beta + (size_t)c * d;
    double* dgm = dgamma + (size_t)c * d;
    double* dbt = dbeta + (size_t)c * d;
    double* Wst = (double*)malloc((size_t)(nb > 0 ? nb : 1) * dd * sizeof(double));
    double* W = (double*)malloc(dd * sizeof(double));
    double* Wt = (double*)malloc((size_t)b * dd * sizeof(double));
    /* per token of the mini-batch: yhat, s_y, r, delta, c, uhat, s_u */
    double* YH = (double*)malloc((size_t)b * d * sizeof(double));
    double* R = (double*)malloc((size_t)b * d * sizeof(double));
    double* DL = (double*)malloc((size_t)b * d * sizeof(double));
    double* UH = (double*)malloc((size_t)b * d * sizeof(double));
    double* sy = (double*)malloc((size_t)b * sizeof(double));
    double* su = (double*)malloc((size_t)b * sizeof(double));
    double* cc = (double*)malloc((size_t)b * sizeof(double));
    double* A = (double*)malloc(dd * sizeof(double));
    double* dWb = (double*)malloc(dd * sizeof(double));
    double* y = (double*)malloc((size_t)d * sizeof(double));
    double* h = (double*)malloc((size_t)d * sizeof(double));
    double* du = (double*)malloc((size_t)d * sizeof(double));
    double* ak = (double*)malloc((size_t)d * sizeof(double));
    double* a = (double*)malloc((size_t)d * sizeof(double));
    double* pa = (double*)malloc((size_t)d * sizeof(double));
    double* dy = (double*)malloc((size_t)d * sizeof(double));
    double* dr = (double*)malloc((size_t)d * sizeof(double));
    double* tmp = (double*)malloc((size_t)d * sizeof(double));
    const double* et = eta + (size_t)c * T;
    for (int i = 0; i < d; ++i) dgm[i] = dbt[i] = 0.0;

    /* forward: the state at every mini-batch start */
    memcpy(W, w0 + c * dd, dd * sizeof(double));
    for (int mb = 0; mb < nb; ++mb) {
      double* Wb = Wst + (size_t)mb * dd;
      memcpy(Wb, W, dd * sizeof(double));
      const int t0 = mb * b, t1 = t0 + b < T ? t0 + b : T;
      for (int t = t0; t < t1; ++t) {
        const size_t o = ((size_t)c * T + t) * d;
        matvec(Wb, k + o, y, d, d);
        double* yh = YH;  /* scratch */
        const double s = ln_normalize(y, yh, d, eps);
        double mg = 0.0, mgy = 0.0;
        for (int i = 0; i < d; ++i) {
          h[i] = 2.0 * (k[o + i] + gm[i] * yh[i] + bt[i] - v[o + i]) * gm[i];
          mg += h[i];
          mgy += h[i] * yh[i];
        }
        mg /= d;
        mgy /= d;
        for (int i = 0; i < d; ++i) h[i] = (h[i] - mg - yh[i] * mgy) / s;
        rank1_sub(W, et[t], h, k + o, d, d);
      }
    }

    /* backward */
    if (dwf) memcpy(A, dwf + c * dd, dd * sizeof(double));
    else memset(A, 0, dd * sizeof(double));
    for (int mb = nb - 1; mb >= 0; --mb) {
      const double* Wb = Wst + (size_t)mb * dd;
      const int t0 = mb * b, t1 = t0 + b < T ? t0 + b : T;
      /* recompute the mini-batch */
      memcpy(W, Wb, dd * sizeof(double));
      for (int t = t0; t < t1; ++t) {
        const size_t o = ((size_t)c * T + t) * d;
        const int j = t - t0;
        double* yh = YH + (size_t)j * d;
        double* r = R + (size_t)j * d;
        double* dl = DL + (size_t)j * d;
        matvec(Wb, k + o, y, d, d);
        sy[j] = ln_normalize(y, yh, d, eps);
        double mg = 0.0, mgy = 0.0;
        for (int i = 0; i < d; ++i) {
          r[i] = k[o + i] + gm[i] * yh[i] + bt[i] - v[o + i];
          h[i] = 2.0 * r[i] * gm[i];
          mg += h[i];
          mgy += h[i] * yh[i];
        }
        mg /= d;
        mgy /= d;
        cc[j] = mgy;
        for (int i = 0; i < d; ++i) dl[i] = (h[i] - mg - yh[i] * mgy) / sy[j];
        rank1_sub(W, et[t], dl, k + o, d, d);
        memcpy(Wt + (size_t)j * dd, W, dd * sizeof(double));
        matvec(W, q + o, y, d, d);
        su[j] = ln_normalize(y, UH + (size_t)j * d, d, eps);
      }
      memset(dWb, 0, dd * sizeof(double));
      for (int t = t1 - 1; t >= t0; --t) {
        const size_t o = ((size_t)c * T + t) * d;
        const int j = t - t0;
        const double* yh = YH + (size_t)j * d;
        const double* r = R + (size_t)j * d;
        const double* dl = DL + (size_t)j * d;
        const double* uh = UH + (size_t)j * d;
        const double s = sy[j];
        /* output: z = q + gamma uhat + beta */
        for (int i = 0; i < d; ++i) {
          dgm[i] += dz[o + i] * uh[i];
          dbt[i] += dz[o + i];
          h[i] = gm[i] * dz[o + i];
        }
        ln_back(h, uh, su[j], du, d);
        const double* Wc = Wt + (size_t)j * dd;
        matvec_t(Wc, du, tmp, d, d);                      /* W_t^T du          */
        for (int i = 0; i < d; ++i) dq[o + i] = dz[o + i] + tmp[i];
        rank1_sub(A, -1.0, du, q + o, d, d);              /* A += du q^T       */
        /* W_t = W_{t-1} - eta delta k^T */
        matvec(A, k + o, ak, d, d);
        double sd = 0.0;
        for (int i = 0; i < d; ++i) {
          a[i] = -et[t] * ak[i];
          sd += dl[i] * ak[i];
        }
        deta[(size_t)c * T + t] = -sd;
        matvec_t(A, dl, tmp, d, d);                       /* A^T delta         */
        for (int i = 0; i < d; ++i) dk[o + i] = -et[t] * tmp[i];
        /* delta = P g / s: dg = P a / s, and its derivative in y at fixed g */
        double ma = 0.0, ay = 0.0, ad = 0.0;
        for (int i = 0; i < d; ++i) {
          ma += a[i];
          ay += a[i] * yh[i];
          ad += a[i] * dl[i];
        }
        ma /= d;
        for (int i = 0; i < d; ++i) pa[i] = a[i] - ma - yh[i] * ay / d;
        for (int i = 0; i < d; ++i)
          dy[i] = -ad * yh[i] / (s * d) - cc[j] * pa[i] / (s * s) - ay * dl[i] / (s * d);
        /* g = 2 r gamma, r = k + gamma yhat + beta - v */
        for (int i = 0; i < d; ++i) {
          const double dg = pa[i] / s;
          dr[i] = 2.0 * gm[i] * dg;
          dgm[i] += 2.0 * r[i] * dg + dr[i] * yh[i];
          dbt[i] += dr[i];
          dk[o + i] += dr[i];
          dv[o + i] = -dr[i];
          h[i] = gm[i] * dr[i];
        }
        ln_back(h, yh, s, tmp, d);
        for (int i = 0; i < d; ++i) dy[i] += tmp[i];
        /* y = Wb k */
        rank1_sub(dWb, -1.0, dy, k + o, d, d);            /* dWb += dy k^T     */
        matvec_t(Wb, dy, tmp, d, d);
        for (int i = 0; i < d; ++i) dk[o + i] += tmp[i];
      }
      for (size_t x = 0; x < dd; ++x) A[x] += dWb[x];
    }
    memcpy(dw0 + c * dd, A, dd * sizeof(double));
    free(Wst); free(W); free(Wt); free(YH); free(R); free(DL); free(UH); free(sy); free(su); free(cc);
    free(A); free(dWb); free(y); free(h); free(du); free(ak); free(a); free(pa); free(dy); free(dr); free(tmp);
  }
}

static double gelu_second(double x) {
  const double inv_sqrt_2pi = 0.39894228040143267794;
  return inv_sqrt_2pi * exp(-0.5 * x * x) * (2.0 - x * x);  /* d/dx (Phi + x phi) = phi (2 - x^2) */
}

/* Gradients of TTT-MLP by reverse-mode differentiation of its primal token loop
 * (oracle_mlp_primal, fp64), for L = sum(dz * Z) + sum(dw1f * W1_final) +
 * sum(dw2f * W2_final):
 *   dq, dk, dv : [n, T, d]   deta : [n, T]   dw1 : [n, dh, d]   dw2 : [n, d, dh]
 * (dw1f, dw2f may be NULL).  Token t of the loop (W1b, W2b: the state before
 * t's mini-batch; W1_t, W2_t after t's step):
 *   h = W1b k,  a = GELU(h),  e = 2 (W2b a - v),  s = W2b^T e,  g = s * GELU'(h),
 *   W2_t = W2_{t-1} - eta e a^T,  W1_t = W1_{t-1} - eta g k^T,
 *   u = W1_t q,  c = GELU(u),  z = W2_t c.
 * Walking back with A1 = dL/dW1_t, A2 = dL/dW2_t:
 *   A2 += dz c^T;  du = (W2_t^T dz) * GELU'(u);  A1 += du q^T;  dq = W1_t^T du
 *   dg = -eta A1 k;  de = -eta A2 a;  da = -eta A2^T e;  dk = -eta A1^T g
 *   deta = -(e . A2 a) - (g . A1 k)
 *   ds = dg * GELU'(h);  dh = dg * s * GELU''(h);  de += W2b ds;  dW2b += e ds^T
 *   dy = 2 de;  dv = -dy;  da += W2b^T dy;  dW2b += dy a^T
 *   dh += da * GELU'(h);  dW1b += dh k^T;  dk += W1b^T dh
 * and at the mini-batch start A1 += dW1b, A2 += dW2b. */
void oracle_mlp_primal_grads(int n, int T, int d, int dh, int b,
                             const double* q, const double* k, const double* v,
                             const double* w1_0, const double* w2_0, const double* eta,
                             const double* dz, const double* dw1f, const double* dw2f,
                             double* dq, double* dk, double* dv, double* deta, double* dw1, double* dw2,
                             int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int c = 0; c < n; ++c) {
    const size_t sz = (size_t)dh * d;
    const int nb = (T + b - 1) / b;
    const size_t nbs = (size_t)(nb > 0 ? nb : 1);
    double* S1 = (double*)malloc(nbs * sz * sizeof(double)); /* W1 at every mini-batch start */
    double* S2 = (double*)malloc(nbs * sz * sizeof(double));
    double* W1 = (double*)malloc(sz * sizeof(double));
    double* W2 = (double*)malloc(sz * sizeof(double));
    double* W1t = (double*)malloc((size_t)b * sz * sizeof(double)); /* W1_t, W2_t of the mini-batch */
    double* W2t = (double*)malloc((size_t)b * sz * sizeof(double));
    double* A1 = (double*)malloc(sz * sizeof(double));
    double* A2 = (double*)malloc(sz * sizeof(double));
    double* G1 = (double*)malloc(sz * sizeof(double));  /* dL/dW1b, dL/dW2b of the mini-batch */
    double* G2 = (double*)malloc(sz * sizeof(double));
    double* H = (double*)malloc((size_t)b * dh * sizeof(double));   /* h, a, s, g, e per token */
    double* Aa = (double*)malloc((size_t)b * dh * sizeof(double));
    double* Sv = (double*)malloc((size_t)b * dh * sizeof(double));
    double* Gv = (double*)malloc((size_t)b * dh * sizeof(double));
    double* Ev = (double*)malloc((size_t)b * d * sizeof(double));
    double* u = (double*)malloc((size_t)dh * sizeof(double));
    double* cv = (double*)malloc((size_t)dh * sizeof(double));
    double* du = (double*)malloc((size_t)dh * sizeof(double));
    double* vd = (double*)malloc((size_t)dh * sizeof(double));   /* scratch of size dh */
    double* vd2 = (double*)malloc((size_t)dh * sizeof(double));
    double* vd3 = (double*)malloc((size_t)dh * sizeof(double));
    double* x1 = (double*)malloc((size_t)d * sizeof(double));    /* scratch of size d */
    double* x2 = (double*)malloc((size_t)d * sizeof(double));
    double* x3 = (double*)malloc((size_t)d * sizeof(double));
    const double* et = eta + (size_t)c * T;

    /* forward: the state at every mini-batch start */
    memcpy(W1, w1_0 + c * sz, sz * sizeof(double));
    memcpy(W2, w2_0 + c * sz, sz * sizeof(double));
    for (int mb = 0; mb < nb; ++mb) {
      double* W1b = S1 + (size_t)mb * sz;
      double* W2b = S2 + (size_t)mb * sz;
      memcpy(W1b, W1, sz * sizeof(double));
      memcpy(W2b, W2, sz * sizeof(double));
      const int t0 = mb * b, t1 = t0 + b < T ? t0 + b : T;
      for (int t = t0; t < t1; ++t) {
        const size_t o = ((size_t)c * T + t) * d;
        matvec(W1b, k + o, vd, dh, d);
        for (int j = 0; j < dh; ++j) vd2[j] = gelu(vd[j]);
        matvec(W2b, vd2, x1, d, dh);
        for (int i = 0; i < d; ++i) x1[i] = 2.0 * (x1[i] - v[o + i]);
        matvec_t(W2b, x1, vd3, d, dh);
        for (int j = 0; j < dh; ++j) vd3[j] *= gelu_prime(vd[j]);
        rank1_sub(W2, et[t], x1, vd2, d, dh);
        rank1_sub(W1, et[t], vd3, k + o, dh, d);
      }
    }

    /* backward */
    if (dw1f) memcpy(A1, dw1f + c * sz, sz * sizeof(double));
    else memset(A1, 0, sz * sizeof(double));
    if (dw2f) memcpy(A2, dw2f + c * sz, sz * sizeof(double));
    else memset(A2, 0, sz * sizeof(double));
    for (int mb = nb - 1; mb >= 0; --mb) {
      const double* W1b = S1 + (size_t)mb * sz;
      const double* W2b = S2 + (size_t)mb * sz;
      const int t0 = mb * b, t1 = t0 + b < T ? t0 + b : T;
      /* recompute the mini-batch: h, a, e, s, g and the states after each token */
      memcpy(W1, W1b, sz * sizeof(double));
      memcpy(W2, W2b, sz * sizeof(double));
      for (int t = t0; t < t1; ++t) {
        const size_t o = ((size_t)c * T + t) * d;
        const int r = t - t0;
        double *h = H + (size_t)r * dh, *a = Aa + (size_t)r * dh, *s = Sv + (size_t)r * dh;
        double *g = Gv + (size_t)r * dh, *e = Ev + (size_t)r * d;
        matvec(W1b, k + o, h, dh, d);
        for (int j = 0; j < dh; ++j) a[j] = gelu(h[j]);
        matvec(W2b, a, e, d, dh);
        for (int i = 0; i < d; ++i) e[i] = 2.0 * (e[i] - v[o + i]);
        matvec_t(W2b, e, s, d, dh);
        for (int j = 0; j < dh; ++j) g[j] = s[j] * gelu_prime(h[j]);
        rank1_sub(W2, et[t], e, a, d, dh);
        rank1_sub(W1, et[t], g, k + o, dh, d);
        memcpy(W1t + (size_t)r * sz, W1, sz * sizeof(double));
        memcpy(W2t + (size_t)r * sz, W2, sz * sizeof(double));
      }
      memset(G1, 0, sz * sizeof(double));
      memset(G2, 0, sz * sizeof(double));
      for (int t = t1 - 1; t >= t0; --t) {
        const size_t o = ((size_t)c * T + t) * d;
        const int r = t - t0;
        const double *h = H + (size_t)r * dh, *a = Aa + (size_t)r * dh, *s = Sv + (size_t)r * dh;
        const double *g = Gv + (size_t)r * dh, *e = Ev + (size_t)r * d;
        const double* W1c = W1t + (size_t)r * sz;
        const double* W2c = W2t + (size_t)r * sz;
        /* the output z_t = W2_t GELU(W1_t q_t) */
        matvec(W1c, q + o, u, dh, d);
        for (int j = 0; j < dh; ++j) cv[j] = gelu(u[j]);
        rank1_sub(A2, -1.0, dz + o, cv, d, dh);               /* A2 += dz c^T */
        matvec_t(W2c, dz + o, du, d, dh);
        for (int j = 0; j < dh; ++j) du[j] *= gelu_prime(u[j]);
        rank1_sub(A1, -1.0, du, q + o, dh, d);                /* A1 += du q^T */
        matvec_t(W1c, du, dq + o, dh, d);                     /* dq = W1_t^T du */
        /* the two rank-one steps */
        matvec(A1, k + o, vd, dh, d);                         /* A1 k */
        matvec(A2, a, x1, d, dh);                             /* A2 a */
        double se = 0.0, sg = 0.0;
        for (int i = 0; i < d; ++i) se += e[i] * x1[i];
        for (int j = 0; j < dh; ++j) sg += g[j] * vd[j];
        deta[(size_t)c * T + t] = -se - sg;
        for (int i = 0; i < d; ++i) x2[i] = -et[t] * x1[i];  /* de from the W2 step */
        matvec_t(A2, e, vd2, d, dh);                          /* A2^T e */
        for (int j = 0; j < dh; ++j) vd2[j] *= -et[t];        /* da from the W2 step */
        matvec_t(A1, g, dk + o, dh, d);                       /* A1^T g */
        for (int i = 0; i < d; ++i) dk[o + i] *= -et[t];
        /* g = s * GELU'(h), s = W2b^T e; vd = dg */
        for (int j = 0; j < dh; ++j) vd[j] *= -et[t];
        for (int j = 0; j < dh; ++j) {
          const double ds = vd[j] * gelu_prime(h[j]);
          vd3[j] = vd[j] * s[j] * gelu_second(h[j]);        /* dh, first part */
          vd[j] = ds;
        }
        matvec(W2b, vd, x3, d, dh);                           /* W2b ds */
        for (int i = 0; i < d; ++i) x2[i] += x3[i];
        rank1_sub(G2, -1.0, e, vd, d, dh);                    /* dW2b += e ds^T */
        /* e = 2 (W2b a - v) */
        for (int i = 0; i < d; ++i) {
          x2[i] *= 2.0;                                       /* dy */
          dv[o + i] = -x2[i];
        }
        matvec_t(W2b, x2, vd, d, dh);                         /* W2b^T dy (into vd) */
        for (int j = 0; j < dh; ++j) vd2[j] += vd[j];         /* da */
        rank1_sub(G2, -1.0, x2, a, d, dh);                    /* dW2b += dy a^T */
        for (int j = 0; j < dh; ++j) vd3[j] += vd2[j] * gelu_prime(h[j]);  /* dh */
        rank1_sub(G1, -1.0, vd3, k + o, dh, d);               /* dW1b += dh k^T */
        matvec_t(W1b, vd3, x3, dh, d);                        /* W1b^T dh */
        for (int i = 0; i < d; ++i) dk[o + i] += x3[i];
      }
      for (size_t x = 0; x < sz; ++x) {
        A1[x] += G1[x];
        A2[x] += G2[x];
      }
    }
    memcpy(dw1 + c * sz, A1, sz * sizeof(double));
    memcpy(dw2 + c * sz, A2, sz * sizeof(double));
    free(S1); free(S2); free(W1); free(W2); free(W1t); free(W2t); free(A1); free(A2); free(G1); free(G2);
    free(H); free(Aa); free(Sv); free(Gv); free(Ev); free(u); free(cv); free(du); free(vd); free(vd2); free(vd3);
    free(x1); free(x2); free(x3);
  }
}
