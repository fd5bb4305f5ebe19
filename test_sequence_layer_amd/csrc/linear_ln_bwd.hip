// TTT-Linear backward with layer norm and residual inside f, fp32 arithmetic.
//
// Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
// (aharts.cn / itmax.cn), part 03 §4 (the layer is trained end to end, so the
// gradient flows through the inner steps), §7 (the dual form), §9 (f carries a
// layer norm and a residual connection: f(x) = x + LN(W x)).
//
// The forward of one mini-batch (token-major rows; W the mini-batch-start
// state, W row i = output i; eta_s per token; LN over the d outputs with
// per-head gamma, beta):
//   y_s = W k_s,  yh_s = (y_s - mean) / sigma_s,  g_s = 2 gamma (k_s + gamma yh_s + beta - v_s)
//   delta_s = (g_s - mean(g_s) - yh_s mean(g_s yh_s)) / sigma_s,   G_s = -eta_s delta_s
//   S[s][t] = k_s . q_t,   u_t = W q_t + sum_{s <= t} S[s][t] G_s
//   z_t = q_t + gamma uh_t + beta,   W' = W + sum_s G_s k_s^T
// The forward saves G as it applied it (its bf16 hi + lo split, exact in
// fp32), so the state is rebuilt by undoing the very same steps; delta is
// recomputed from the rebuilt state where its derivatives need it.  The
// backward, given dz_t and A = dL/dW' (dU, dG, dY the adjoints of u, G, y):
//   W      = W' - sum_s G_s k_s^T                            (the state rebuilt)
//   du_t   = (h - mean(h) - uh_t mean(h uh_t)) / sigma_u,   h = gamma dz_t
//   dS[s][t] = G_s . du_t (s <= t)
//   dG_s   = sum_{t >= s} S[s][t] du_t + A k_s,   lam_s = dL/d delta_s = -eta_s dG_s
//   dg_s   = (lam - mean(lam) - yh mean(lam yh)) / sigma      (lam through P = I - 11^T/d - yh yh^T/d)
//   dy_s   = -c dg / sigma - (mean(lam yh) delta + mean(lam delta) yh) / sigma
//            + LNback(2 gamma^2 dg),   c = mean(g yh)             (delta's own dependence on y)
//   dq_t   = dz_t + W^T du_t + sum_{s <= t} dS[s][t] k_s
//   dk_s   = W^T dy_s + A^T G_s + sum_{t >= s} dS[s][t] q_t + 2 gamma dg_s
//   dv_s   = -2 gamma dg_s,   deta_s = -delta_s . dG_s
//   dgamma += sum_t dz_t uh_t + sum_s dg_s 2 (k_s + 2 gamma yh_s + beta - v_s),  dbeta += sum_t dz_t + sum_s 2 gamma dg_s
//   A     <- A + sum_t du_t q_t^T + sum_s dy_s k_s^T           (the adjoint of W, carried back)
//
// One workgroup (256 threads) per (sequence, head) walks the mini-batches from
// last to first with W and A in LDS.  Products are plain fp32 FMA loops over
// LDS tiles; the per-token layer-norm statistics are wave reductions, a
// token's 64 outputs on the 64 lanes of one wave.
#include "args_bwd.h"

namespace ttt {
namespace {

constexpr int D = 64;
constexpr int BMAX = 16;
constexpr int kThreads = 256;
constexpr int P1 = D + 1;  // padded row (floats)

__device__ __forceinline__ float in_val(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }

template <typename T>
__device__ __forceinline__ float g_load(const T* p, size_t i);
template <>
__device__ __forceinline__ float g_load<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float g_load<uint16_t>(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }

template <typename T>
__device__ __forceinline__ void g_store(T* p, size_t i, float x);
template <>
__device__ __forceinline__ void g_store<float>(float* p, size_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void g_store<uint16_t>(uint16_t* p, size_t i, float x) { p[i] = f32_to_bf16_bits(x); }

// Mean over the 64 lanes of a wave (each lane one output of the token).
__device__ __forceinline__ float wave_mean(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x * (1.f / D);
}

template <typename GT>
__global__ __launch_bounds__(kThreads) void ttt_linear_ln_bwd_fp32(BwdArgs a) {
  __shared__ float W[D][P1];
  __shared__ float A[D][P1];
  __shared__ float Ks[BMAX][P1], Qs[BMAX][P1], Vs[BMAX][P1], Gs[BMAX][P1], Zs[BMAX][P1];
  __shared__ float Yh[BMAX][P1];  // W k, then yh
  __shared__ float Uh[BMAX][P1];  // u, then uh
  __shared__ float dU[BMAX][P1];
  __shared__ float Pg[BMAX][P1];  // A k, then dg
  __shared__ float dY[BMAX][P1];
  __shared__ float Ss[BMAX][BMAX + 1];
  __shared__ float dS[BMAX][BMAX + 1];
  __shared__ float et[BMAX], ry[BMAX], mg[BMAX], cg[BMAX];

  const int tid = threadIdx.x;
  const int lane = tid & 63;  // the output / column a thread takes in the per-token passes
  const int wv = tid >> 6;    // tokens wv, wv + 4, ... in those passes
  const int chain = blockIdx.x;
  const int bi = chain / a.H;
  const int h = chain - bi * a.H;
  const int b = a.b;

  const float gam = a.gamma[h * D + lane];
  const float bet = a.beta[h * D + lane];
  const float eps = a.eps;
  float dgam = 0.f, dbet = 0.f;  // this thread's share of column `lane`

  const float* wf = a.Wf + static_cast<int64_t>(chain) * D * D;
  const float* af = a.dWf ? a.dWf + static_cast<int64_t>(chain) * D * D : nullptr;
  for (int x = tid; x < D * D; x += kThreads) {
    W[x / D][x % D] = wf[x];
    A[x / D][x % D] = af ? af[x] : 0.f;
  }

  const size_t base = static_cast<size_t>(chain) * a.T * D;
  const uint16_t* Qg = static_cast<const uint16_t*>(a.Q) + base;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.K) + base;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.V) + base;
  const float* Gg = a.E + base;
  const GT* Zg = static_cast<const GT*>(a.dZ) + base;
  GT* dQg = static_cast<GT*>(a.dQ) + base;
  GT* dKg = static_cast<GT*>(a.dK) + base;
  GT* dVg = static_cast<GT*>(a.dV) + base;
  float* detag = a.deta + static_cast<size_t>(chain) * a.T;
  const float* eg = a.eta + bi * a.esb + h * a.esh;

  const int nb = a.T / b;
  for (int n = nb - 1; n >= 0; --n) {
    const int t0 = n * b;
    __syncthreads();  // the previous mini-batch is done with the tiles, W and A
    for (int x = tid; x < b * D; x += kThreads) {
      const int t = x / D, c = x % D;
      const size_t o = static_cast<size_t>(t0) * D + x;
      Ks[t][c] = in_val(Kg, o);
      Qs[t][c] = in_val(Qg, o);
      Vs[t][c] = in_val(Vg, o);
      Gs[t][c] = Gg[o];
      Zs[t][c] = g_load<GT>(Zg, o);
    }
    for (int t = tid; t < b; t += kThreads) et[t] = eg[static_cast<int64_t>(t0 + t) * a.est];
    __syncthreads();

    // the mini-batch-start state; S; A k at the mini-batch-end adjoint
    for (int x = tid; x < D * D; x += kThreads) {
      const int i = x / D, c = x % D;
      float w = W[i][c];
      for (int s = 0; s < b; ++s) w = fmaf(-Gs[s][i], Ks[s][c], w);
      W[i][c] = w;
    }
    for (int x = tid; x < b * b; x += kThreads) {
      const int s = x / b, t = x % b;
      float sv = 0.f;
      if (s <= t)
        for (int c = 0; c < D; ++c) sv = fmaf(Ks[s][c], Qs[t][c], sv);
      Ss[s][t] = sv;
    }
    for (int x = tid; x < b * D; x += kThreads) {
      const int s = x / D, i = x % D;
      float p = 0.f;
      for (int c = 0; c < D; ++c) p = fmaf(A[i][c], Ks[s][c], p);
      Pg[s][i] = p;
    }
    __syncthreads();

    // y = W k, u = W q + sum_{s <= t} S[s][t] G_s
    for (int x = tid; x < b * D; x += kThreads) {
      const int t = x / D, i = x % D;
      float y = 0.f, u = 0.f;
      for (int c = 0; c < D; ++c) {
        y = fmaf(W[i][c], Ks[t][c], y);
        u = fmaf(W[i][c], Qs[t][c], u);
      }
      for (int s = 0; s <= t; ++s) u = fmaf(Ss[s][t], Gs[s][i], u);
      Yh[t][i] = y;
      Uh[t][i] = u;
    }
    __syncthreads();

    // per token: the two layer norms, mean(g) and c = mean(g yh), du; dgamma, dbeta from z
    for (int t = wv; t < b; t += kThreads / 64) {
      const float y = Yh[t][lane];
      const float my = wave_mean(y);
      const float yc = y - my;
      const float rsy = rsqrtf(wave_mean(yc * yc) + eps);
      const float yh = yc * rsy;
      const float gg = 2.f * gam * (Ks[t][lane] + gam * yh + bet - Vs[t][lane]);
      const float m = wave_mean(gg);
      const float c = wave_mean(gg * yh);
      Yh[t][lane] = yh;
      if (lane == 0) {
        ry[t] = rsy;
        mg[t] = m;
        cg[t] = c;
      }
      const float u = Uh[t][lane];
      const float mu = wave_mean(u);
      const float uc = u - mu;
      const float rsu = rsqrtf(wave_mean(uc * uc) + eps);
      const float uh = uc * rsu;
      const float dz = Zs[t][lane];
      const float hh = gam * dz;
      const float mh = wave_mean(hh);
      const float mhu = wave_mean(hh * uh);
      dU[t][lane] = rsu * (hh - mh - uh * mhu);
      dgam = fmaf(dz, uh, dgam);
      dbet += dz;
    }
    __syncthreads();

    // dS[s][t] = G_s . du_t (s <= t)
    for (int x = tid; x < b * b; x += kThreads) {
      const int s = x / b, t = x % b;
      float m = 0.f;
      if (s <= t)
        for (int i = 0; i < D; ++i) m = fmaf(Gs[s][i], dU[t][i], m);
      dS[s][t] = m;
    }
    __syncthreads();

    // per token: dG, lambda, delta (recomputed), deta, the layer-norm double
    // backward (dg, dy), dv
    for (int s = wv; s < b; s += kThreads / 64) {
      float acc = Pg[s][lane];
      for (int t = s; t < b; ++t) acc = fmaf(Ss[s][t], dU[t][lane], acc);
      const float lam = -et[s] * acc;
      const float yh = Yh[s][lane];
      const float rs = ry[s];
      const float res = Ks[s][lane] + gam * yh + bet - Vs[s][lane];  // f(k) - v
      const float dl = rs * (2.f * gam * res - mg[s] - yh * cg[s]);
      const float de = wave_mean(dl * acc);
      if (lane == 0) detag[t0 + s] = -de * D;
      const float ml = wave_mean(lam);
      const float mly = wave_mean(lam * yh);
      const float mld = wave_mean(lam * dl);
      const float dg = rs * (lam - ml - yh * mly);
      const float h2 = 2.f * gam * gam * dg;
      const float mh2 = wave_mean(h2);
      const float mh2y = wave_mean(h2 * yh);
      const float dy = -cg[s] * rs * dg - rs * (mly * dl + mld * yh) + rs * (h2 - mh2 - yh * mh2y);
      Pg[s][lane] = dg;
      dY[s][lane] = dy;
      dgam = fmaf(2.f * dg, res + gam * yh, dgam);
      dbet = fmaf(2.f * gam, dg, dbet);
      g_store<GT>(dVg, static_cast<size_t>(t0 + s) * D + lane, -2.f * gam * dg);
    }
    __syncthreads();

    // dq, dk (A still the mini-batch-end adjoint)
    for (int x = tid; x < b * D; x += kThreads) {
      const int s = x / D, c = x % D;
      float q = Zs[s][c], k = 2.f * a.gamma[h * D + c] * Pg[s][c];
      for (int i = 0; i < D; ++i) {
        q = fmaf(dU[s][i], W[i][c], q);
        k = fmaf(dY[s][i], W[i][c], k);
        k = fmaf(Gs[s][i], A[i][c], k);
      }
      for (int u = 0; u <= s; ++u) q = fmaf(dS[u][s], Ks[u][c], q);
      for (int u = s; u < b; ++u) k = fmaf(dS[s][u], Qs[u][c], k);
      g_store<GT>(dQg, static_cast<size_t>(t0) * D + x, q);
      g_store<GT>(dKg, static_cast<size_t>(t0) * D + x, k);
    }
    __syncthreads();

    // the adjoint of the mini-batch-start state
    for (int x = tid; x < D * D; x += kThreads) {
      const int i = x / D, c = x % D;
      float av = A[i][c];
      for (int t = 0; t < b; ++t) {
        av = fmaf(dU[t][i], Qs[t][c], av);
        av = fmaf(dY[t][i], Ks[t][c], av);
      }
      A[i][c] = av;
    }
  }
  // dgamma, dbeta: the four partial sums of each column, reduced through the
  // (now free) K and Q tiles
  __syncthreads();
  float* red0 = &Ks[0][0];
  float* red1 = &Qs[0][0];
  red0[tid] = dgam;
  red1[tid] = dbet;
  __syncthreads();
  float* dw = a.dW0 + static_cast<int64_t>(chain) * D * D;
  for (int x = tid; x < D * D; x += kThreads) dw[x] = A[x / D][x % D];
  if (tid < D) {
    float sg = 0.f, sb = 0.f;
    for (int j = 0; j < kThreads / 64; ++j) {
      sg += red0[tid + 64 * j];
      sb += red1[tid + 64 * j];
    }
    a.dgamma[static_cast<int64_t>(chain) * D + tid] = sg;
    a.dbeta[static_cast<int64_t>(chain) * D + tid] = sb;
  }
}

}  // namespace

bool linear_ln_bwd_supported(const BwdArgs& a) { return a.d == D && a.b == 16 && a.in_dtype == 1; }

hipError_t launch_linear_ln_bwd(const BwdArgs& a, hipStream_t s) {
  dim3 grid(a.B * a.H), block(kThreads);
  if (a.out_dtype == 0)
    hipLaunchKernelGGL(ttt_linear_ln_bwd_fp32<float>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(ttt_linear_ln_bwd_fp32<uint16_t>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
