/*
 * Memory- and UB-checking driver for the C oracle (test infrastructure, like
 * the oracle itself).  tests/test_oracle_sanitize.py compiles it together with
 * ttt_oracle.c under AddressSanitizer and UndefinedBehaviorSanitizer and runs
 * every oracle entry point on small problems whose buffers are allocated at
 * exactly their documented sizes, at shapes with ragged last mini-batches
 * (T % b != 0), b = 1, b = T and odd d, so any read or write outside a buffer,
 * or any undefined arithmetic, aborts the run.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_linear_primal(int n, int T, int d, int b, const double* q, const double* k, const double* v,
                          const double* w0, const double* eta, double* z, double* wf, int nthreads);
void oracle_mlp_primal(int n, int T, int d, int dh, int b, const double* q, const double* k, const double* v,
                       const double* w1_0, const double* w2_0, const double* eta, double* z, double* w1f,
                       double* w2f, int nthreads);
void oracle_linear_ln_primal(int n, int T, int d, int b, const double* q, const double* k, const double* v,
                             const double* w0, const double* gamma, const double* beta, double eps,
                             const double* eta, double* z, double* wf, int nthreads);
void oracle_mlp_primal_grads(int n, int T, int d, int dh, int b, const double* q, const double* k, const double* v,
                             const double* w1_0, const double* w2_0, const double* eta, const double* dz,
                             const double* dw1f, const double* dw2f, double* dq, double* dk, double* dv,
                             double* deta, double* dw1, double* dw2, int nthreads);
void oracle_linear_primal_grads(int n, int T, int d, int b, const double* q, const double* k, const double* v,
                                const double* w0, const double* eta, const double* dz, const double* dwf,
                                double* dq, double* dk, double* dv, double* deta, double* dw0, int nthreads);
void oracle_linear_ln_primal_grads(int n, int T, int d, int b, const double* q, const double* k, const double* v,
                                   const double* w0, const double* gamma, const double* beta, double eps,
                                   const double* eta, const double* dz, const double* dwf, double* dq, double* dk,
                                   double* dv, double* deta, double* dw0, double* dgamma, double* dbeta,
                                   int nthreads);

static uint64_t state = 0x9E3779B97F4A7C15ull;

/* splitmix64 -> uniform in [-scale, scale) */
static double uni(double scale) {
  uint64_t x = (state += 0x9E3779B97F4A7C15ull);
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  x ^= x >> 31;
  return scale * ((double)(x >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

static double* buf(size_t count, double scale) {
  double* p = (double*)malloc(count * sizeof(double));
  if (!p) exit(3);
  for (size_t i = 0; i < count; ++i) p[i] = uni(scale);
  return p;
}

static int finite_all(const double* p, size_t count) {
  for (size_t i = 0; i < count; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

int main(void) {
  const int shapes[][4] = {/* n, T, d, b */ {2, 10, 3, 4}, {1, 7, 5, 1}, {3, 6, 4, 6}, {2, 9, 2, 16}, {1, 0, 3, 2}};
  int bad = 0;
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
    const int n = shapes[s][0], T = shapes[s][1], d = shapes[s][2], b = shapes[s][3];
    const size_t tok = (size_t)n * T * d, dd = (size_t)n * d * d, nt = (size_t)n * T;
    double *q = buf(tok, 0.5), *k = buf(tok, 0.5), *v = buf(tok, 0.5), *w0 = buf(dd, 0.1), *eta = buf(nt, 0.05);
    double *z = buf(tok, 0), *wf = buf(dd, 0);
    oracle_linear_primal(n, T, d, b, q, k, v, w0, eta, z, wf, 2);
    bad |= !finite_all(z, tok) || !finite_all(wf, dd);

    double *gamma = buf((size_t)n * d, 1.0), *beta = buf((size_t)n * d, 0.1);
    oracle_linear_ln_primal(n, T, d, b, q, k, v, w0, gamma, beta, 1e-5, eta, z, wf, 2);
    bad |= !finite_all(z, tok) || !finite_all(wf, dd);

    const int dh = 2 * d + 1;
    const size_t hd = (size_t)n * dh * d;
    double *w1 = buf(hd, 0.1), *w2 = buf(hd, 0.1), *w1f = buf(hd, 0), *w2f = buf(hd, 0);
    oracle_mlp_primal(n, T, d, dh, b, q, k, v, w1, w2, eta, z, w1f, w2f, 2);
    bad |= !finite_all(z, tok) || !finite_all(w1f, hd) || !finite_all(w2f, hd);
    {
      double *mdz = buf(tok, 1.0), *m1 = buf(hd, 1.0), *m2 = buf(hd, 1.0);
      double *gq = buf(tok, 0), *gk = buf(tok, 0), *gv = buf(tok, 0), *ge = buf(nt, 0), *g1 = buf(hd, 0),
             *g2 = buf(hd, 0);
      oracle_mlp_primal_grads(n, T, d, dh, b, q, k, v, w1, w2, eta, mdz, m1, m2, gq, gk, gv, ge, g1, g2, 2);
      bad |= !finite_all(gq, tok) || !finite_all(gk, tok) || !finite_all(gv, tok) || !finite_all(ge, nt) ||
             !finite_all(g1, hd) || !finite_all(g2, hd);
      oracle_mlp_primal_grads(n, T, d, dh, b, q, k, v, w1, w2, eta, mdz, NULL, NULL, gq, gk, gv, ge, g1, g2, 2);
      bad |= !finite_all(g1, hd) || !finite_all(g2, hd);
      free(mdz); free(m1); free(m2); free(gq); free(gk); free(gv); free(ge); free(g1); free(g2);
    }

    double *dz = buf(tok, 1.0), *dwf = buf(dd, 1.0);
    double *dq = buf(tok, 0), *dk = buf(tok, 0), *dv = buf(tok, 0), *deta = buf(nt, 0), *dw0 = buf(dd, 0);
    oracle_linear_primal_grads(n, T, d, b, q, k, v, w0, eta, dz, dwf, dq, dk, dv, deta, dw0, 2);
    bad |= !finite_all(dq, tok) || !finite_all(dk, tok) || !finite_all(dv, tok) || !finite_all(deta, nt) ||
           !finite_all(dw0, dd);
    oracle_linear_primal_grads(n, T, d, b, q, k, v, w0, eta, dz, NULL, dq, dk, dv, deta, dw0, 2);
    bad |= !finite_all(dw0, dd);

    double *dgamma = buf((size_t)n * d, 0), *dbeta = buf((size_t)n * d, 0);
    oracle_linear_ln_primal_grads(n, T, d, b, q, k, v, w0, gamma, beta, 1e-5, eta, dz, dwf, dq, dk, dv, deta, dw0,
                                  dgamma, dbeta, 2);
    bad |= !finite_all(dq, tok) || !finite_all(dk, tok) || !finite_all(dv, tok) || !finite_all(deta, nt) ||
           !finite_all(dw0, dd) || !finite_all(dgamma, (size_t)n * d) || !finite_all(dbeta, (size_t)n * d);
    oracle_linear_ln_primal_grads(n, T, d, b, q, k, v, w0, gamma, beta, 1e-5, eta, dz, NULL, dq, dk, dv, deta, dw0,
                                  dgamma, dbeta, 2);
    bad |= !finite_all(dw0, dd) || !finite_all(dgamma, (size_t)n * d);
    free(dgamma); free(dbeta);

    free(q); free(k); free(v); free(w0); free(eta); free(z); free(wf); free(gamma); free(beta);
    free(w1); free(w2); free(w1f); free(w2f);
    free(dz); free(dwf); free(dq); free(dk); free(dv); free(deta); free(dw0);
  }
  printf(bad ? "non-finite output\n" : "ok\n");
  return bad ? 1 : 0;
}
