// TTT-MLP backward in the primal form: the token loop differentiated in
// reverse, on the GPU.
//
// Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
// (aharts.cn / itmax.cn), part 03 §4 (the layer is trained end to end), §6
// (mini-batch GD: every gradient of a mini-batch is taken at its start state),
// §9 (TTT-MLP: f(x) = W2 GELU(W1 x), hidden width 4d).
//
// Forward token t (W1b, W2b the mini-batch-start state, W1_t, W2_t after t):
//   h = W1b k, a = GELU(h), e = 2 (W2b a - v), s = W2b^T e, g = s * GELU'(h),
//   W2_t = W2_{t-1} - eta e a^T, W1_t = W1_{t-1} - eta g k^T, z = W2_t GELU(W1_t q).
// Backward, walking the tokens last to first with A1 = dL/dW1_t, A2 = dL/dW2_t:
//   A2 += dz c^T; du = (W2_t^T dz) * GELU'(u); A1 += du q^T; dq = W1_t^T du
//   dg = -eta A1 k; de = -eta A2 a + W2b ds; da = -eta A2^T e + W2b^T dy
//   deta = -(e . A2 a) - (g . A1 k); dk = -eta A1^T g + W1b^T dh
//   ds = dg * GELU'(h); dy = 2 de; dv = -dy; dh = dg * s * GELU''(h) + da * GELU'(h)
// and at the mini-batch start A1 += sum dh k^T, A2 += sum (e ds^T + dy a^T).
// Only the mini-batch-start state is held: the products with the state
// after token t use it and the mini-batch's own vectors,
//   W1_t x = W1b x - sum_{s<=t} eta_s (k_s . x) g_s,
//   W2_t^T y = W2b^T y - sum_{s<=t} eta_s (e_s . y) a_s,
//   W1_t^T y = W1b^T y - sum_{s<=t} eta_s (g_s . y) k_s.
//
// One workgroup of 8 waves per (sequence, head).  A first pass runs the
// forward from W0 and writes the state at every mini-batch start to the
// workspace; the second walks the mini-batches last to first: it reads the
// start state, recomputes h, a, e, s, g of the mini-batch's tokens (kept in
// LDS), then runs the tokens in reverse.  W1b, W2b, A1, A2 live in registers
// in the two layouts of the primal forward kernel (lane l of wave w, g = l/16,
// li = l%16):
//   W1-type  row j = 32 w + 4 r + g, columns 4 li .. 4 li + 3   (r = 0..7)
//   W2-type  row i = 8 w + m, columns 4 l .. 4 l + 3           (m = 0..7)
// fp32 throughout; written for correctness at the TTT-MLP shapes (d = 64,
// dh = 256, b <= 16), not tuned.
#include "args_mlp_bwd.h"
#include "mfma_common.h"

namespace ttt {
namespace {

using mfma::sum16;
using mfma::sum_rows;

constexpr int D = 64;
constexpr int DH = 256;
constexpr int NW = 8;
constexpr int NT = 64 * NW;
constexpr int BT = 16;  // largest mini-batch

template <typename T>
__device__ __forceinline__ float ld_in(const T* p, size_t i);
template <>
__device__ __forceinline__ float ld_in<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_in<uint16_t>(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }

__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return fmaf(a.x, b.x, fmaf(a.y, b.y, fmaf(a.z, b.z, a.w * b.w)));
}
// x + c * y, elementwise
__device__ __forceinline__ float4 axpy(float4 x, float c, float4 y) {
  return make_float4(fmaf(c, y.x, x.x), fmaf(c, y.y, x.y), fmaf(c, y.z, x.z), fmaf(c, y.w, x.w));
}
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 x) { *reinterpret_cast<float4*>(p) = x; }
__device__ __forceinline__ float wave_sum(float x) { return sum_rows(sum16(x)); }
// the sum over the four 16-lane rows at the same position in the row
__device__ __forceinline__ float4 rows4(float4 x) {
  return make_float4(sum_rows(x.x), sum_rows(x.y), sum_rows(x.z), sum_rows(x.w));
}

// GELU(x) = x Phi(x), GELU'(x) = Phi(x) + x phi(x), GELU''(x) = phi(x) (2 - x^2)
__device__ __forceinline__ void gelu3(float x, float& g, float& gp, float& gpp) {
  const float cdf = 0.5f * (1.f + erff(x * 0.70710678118654752f));
  const float pdf = 0.39894228040143268f * __builtin_amdgcn_exp2f(x * x * -0.72134752044448170f);
  g = x * cdf;
  gp = fmaf(x, pdf, cdf);
  gpp = pdf * (2.f - x * x);
}

struct Tiles {
  float K[BT][D], Q[BT][D], V[BT][D], DZ[BT][D];
  float ET[BT];
  float H[BT][DH], A[BT][DH], S[BT][DH], G[BT][DH];
  float E[BT][D];
  float DH_[BT][DH], DS[BT][DH];
  float DY[BT][D];
  float KQ[BT][BT], ED[BT][BT];  // k_s . q_t and e_s . dz_t (s <= t)
  float red1[NW][DH], red1b[NW][DH];
  float red2[NW][D], red2b[NW][D], red2c[NW][D];
  float CV[DH], CPV[DH], DU[DH], DA[DH], DH1[DH];
  float GD[BT];
  float reta[2][NW];
  // layer norm: per token of the mini-batch the normalised pre-norm output, the
  // loss gradient at it (gamma-scaled) and the standard deviation; a 64-vector
  // exchange buffer, the gradient of Delta, the residual part of dk, and
  // e_s . dy_z of the token being reversed
  float YH[BT][D], GF[BT][D];
  float SIG[BT];
  float YB[D], DEB[D], DKR[D];
  float EDT[BT];
};

__device__ __forceinline__ float readlane(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// LN: f(x) = x + LN(W2 GELU(W1 x)), LN(y) = gamma (y - mean y) / sqrt(var y + eps) + beta
// over the d outputs.  The loss gradient at the pre-norm output, Delta =
// (G - mean G - yh mean(G yh)) / sigma with G = 2 (k + LN(y) - v) * gamma, takes
// the place of e = 2 (y - v); z = q + LN(W2_t GELU(W1_t q)).  Each layer norm
// runs in every wave with output i in lane i (its 64 outputs, wave-wide sums),
// after the 8 waves have put their 8 rows of the 64-vector in LDS.  Backward:
//   output side: dy_z = (gamma dz - mean(gamma dz) - yh_z mean(gamma dz yh_z)) / sigma_z,
//     dq += dz, dgamma += dz yh_z, dbeta += dz;
//   K side, from dDelta: dG = P(dDelta) / sigma (P(x) = x - mean x - yh mean(x yh)),
//     dyh = -(mean(G yh) dDelta + mean(dDelta yh) G) / sigma + 2 gamma^2 dG,
//     dsigma = -(dDelta . Delta) / sigma,
//     dy = (dyh - mean dyh - yh mean(dyh yh)) / sigma + dsigma yh / d,
//     dk += 2 gamma dG, dv = -2 gamma dG, dgamma += dG (2 (k + gamma yh + beta - v) + 2 gamma yh),
//     dbeta += 2 gamma dG.
template <typename InT, bool LN>
__global__ __launch_bounds__(NT) void ttt_mlp_bwd_d64h256(MlpBwdArgs a) {
  __shared__ __align__(16) Tiles S_;
  Tiles& L = S_;
  const int tid = threadIdx.x;
  const int l = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), g = l >> 4, li = l & 15;
  const int chain = blockIdx.x;
  const int bi = chain / a.H, h = chain - bi * a.H;
  const int T = a.T, b = a.b;
  const int nb = (T + b - 1) / b;

  // W1b, W2b (mini-batch-start state) and A1, A2 (adjoints; during the
  // first pass the running state W1, W2)
  float4 w1b[8], w2b[8], a1[8], a2[8];
  auto off1 = [&](int r) { return static_cast<int64_t>(32 * w + 4 * r + g) * D + 4 * li; };
  auto off2 = [&](int m) { return static_cast<int64_t>(8 * w + m) * DH + 4 * l; };
  const int64_t st_sz = static_cast<int64_t>(DH) * D;
  const int64_t in_off = bi * a.w_in_bstride + static_cast<int64_t>(h) * st_sz;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    a1[r] = ld4(a.W1_in + in_off + off1(r));
    a2[r] = ld4(a.W2_in + in_off + off2(r));
  }
  float* wsc = a.ws + static_cast<int64_t>(chain) * (nb > 0 ? nb : 1) * 2 * st_sz;

  const size_t base = static_cast<size_t>(chain) * T * D;
  const InT* Qg = static_cast<const InT*>(a.Q) + base;
  const InT* Kg = static_cast<const InT*>(a.K) + base;
  const InT* Vg = static_cast<const InT*>(a.V) + base;
  const float* DZg = a.dZ + base;
  const float* eg = a.eta + bi * a.esb + h * a.esh;
  // layer norm: gamma, beta of output l, and its dgamma, dbeta sums (wave 0)
  float gam = 0.f, bet = 0.f, dgam = 0.f, dbet = 0.f;
  if constexpr (LN) {
    gam = a.gamma[static_cast<int64_t>(h) * D + l];
    bet = a.beta[static_cast<int64_t>(h) * D + l];
  }
  constexpr float RD = 1.f / D;

  auto stage = [&](int t0, int nt) {
    for (int x = tid; x < nt * D; x += NT) {
      const size_t gi = static_cast<size_t>(t0) * D + x;
      L.K[x / D][x % D] = ld_in<InT>(Kg, gi);
      L.Q[x / D][x % D] = ld_in<InT>(Qg, gi);
      L.V[x / D][x % D] = ld_in<InT>(Vg, gi);
      L.DZ[x / D][x % D] = DZg[gi];
    }
    if (tid < nt) L.ET[tid] = eg[static_cast<int64_t>(t0 + tid) * a.est];
  };

  // The forward quantities of token u of the staged mini-batch at the start
  // state (three barriers); with STEP also the step of the running state.
  auto forward_token = [&](int u, bool step) {
    const float4 k4 = ld4(&L.K[u][4 * li]);
    float gp[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float hv = sum16(dot4(w1b[r], k4));
      float av, gpp;
      gelu3(hv, av, gp[r], gpp);
      if (li == 0) {
        const int j = 32 * w + 4 * r + g;
        L.H[u][j] = hv;
        L.A[u][j] = av;
      }
    }
    __syncthreads();
    const float et = L.ET[u];
    const float4 av4 = ld4(&L.A[u][4 * l]);
    float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (LN) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float y = wave_sum(dot4(w2b[m], av4));
        if (l == m) L.YB[8 * w + m] = y;
      }
      __syncthreads();
      const float y = L.YB[l];
      const float dv = y - wave_sum(y) * RD;
      const float sg = sqrtf(wave_sum(dv * dv) * RD + a.eps);
      const float yh = dv / sg;
      const float gf = 2.f * (L.K[u][l] + gam * yh + bet - L.V[u][l]) * gam;
      const float el = (gf - wave_sum(gf) * RD - yh * (wave_sum(gf * yh) * RD)) / sg;
      if (w == 0) {
        L.YH[u][l] = yh;
        L.GF[u][l] = gf;
        L.E[u][l] = el;
        if (l == 0) L.SIG[u] = sg;
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float e = readlane(el, 8 * w + m);
        s4 = axpy(s4, e, w2b[m]);
        if (step) a2[m] = axpy(a2[m], -et * e, av4);
      }
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float e = 2.f * (wave_sum(dot4(w2b[m], av4)) - L.V[u][8 * w + m]);
        if (l == m) L.E[u][8 * w + m] = e;
        s4 = axpy(s4, e, w2b[m]);
        if (step) a2[m] = axpy(a2[m], -et * e, av4);
      }
    }
    st4(&L.red1[w][4 * l], s4);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int j = 32 * w + 4 * r + g;
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < NW; ++v) s += L.red1[v][j];
      const float gg = s * gp[r];
      if (li == 0) {
        L.S[u][j] = s;
        L.G[u][j] = gg;
      }
      if (step) a1[r] = axpy(a1[r], -et * gg, k4);
    }
    __syncthreads();
  };

  // ---- pass 1: forward from W0, the state at every mini-batch start to the workspace ----
  for (int n = 0; n < nb; ++n) {
    float* ck = wsc + static_cast<int64_t>(n) * 2 * st_sz;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      w1b[r] = a1[r];
      w2b[r] = a2[r];
      st4(ck + off1(r), w1b[r]);
      st4(ck + st_sz + off2(r), w2b[r]);
    }
    if (n == nb - 1) break;  // the last mini-batch's steps are not needed
    const int t0 = n * b, nt = min(b, T - t0);
    __syncthreads();  // the previous mini-batch's tiles are consumed
    stage(t0, nt);
    __syncthreads();
    for (int u = 0; u < nt; ++u) forward_token(u, true);
  }

  // ---- pass 2: the mini-batches in reverse ----
  const int64_t cs = static_cast<int64_t>(chain) * st_sz;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    a1[r] = a.dW1f ? ld4(a.dW1f + cs + off1(r)) : make_float4(0.f, 0.f, 0.f, 0.f);
    a2[r] = a.dW2f ? ld4(a.dW2f + cs + off2(r)) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int n = nb - 1; n >= 0; --n) {
    const float* ck = wsc + static_cast<int64_t>(n) * 2 * st_sz;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      w1b[r] = ld4(ck + off1(r));
      w2b[r] = ld4(ck + st_sz + off2(r));
    }
    const int t0 = n * b, nt = min(b, T - t0);
    __syncthreads();
    stage(t0, nt);
    __syncthreads();
    for (int u = 0; u < nt; ++u) forward_token(u, false);
    // k_s . q_t and e_s . dz_t for s <= t
    {
      const int p = tid & 255, s = p >> 4, t = p & 15;
      if (s <= t && t < nt) {
        const float* x = tid < 256 ? L.K[s] : L.E[s];
        const float* y = tid < 256 ? L.Q[t] : L.DZ[t];
        float acc = 0.f;
        for (int c = 0; c < D; ++c) acc = fmaf(x[c], y[c], acc);
        (tid < 256 ? L.KQ : L.ED)[s][t] = acc;
      }
    }
    __syncthreads();

    for (int t = nt - 1; t >= 0; --t) {
      const size_t o = (static_cast<size_t>(t0) + t) * D;
      const float et = L.ET[t];
      const float4 q4 = ld4(&L.Q[t][4 * li]);
      const float4 k4 = ld4(&L.K[t][4 * li]);
      // 1. u = W1_t q, c = GELU(u), c' = GELU'(u)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int j = 32 * w + 4 * r + g;
        float u = sum16(dot4(w1b[r], q4));
        for (int s = 0; s <= t; ++s) u = fmaf(-L.ET[s] * L.KQ[s][t], L.G[s][j], u);
        float c, cp, cpp;
        gelu3(u, c, cp, cpp);
        if (li == 0) {
          L.CV[j] = c;
          L.CPV[j] = cp;
        }
      }
      __syncthreads();
      // LN, output side: y_z = W2_t c (rows 8w + m), then the gradient at it
      // (dz_l in lane l) and e_s . dy_z for the W2_t^T correction
      float dzl = 0.f;
      if constexpr (LN) {
        const float4 c4 = ld4(&L.CV[4 * l]);
        float yz[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) yz[m] = wave_sum(dot4(w2b[m], c4));
        for (int s = 0; s <= t; ++s) {
          const float f = -L.ET[s] * wave_sum(dot4(ld4(&L.A[s][4 * l]), c4));
#pragma unroll
          for (int m = 0; m < 8; ++m) yz[m] = fmaf(f, L.E[s][8 * w + m], yz[m]);
        }
#pragma unroll
        for (int m = 0; m < 8; ++m)
          if (l == m) L.YB[8 * w + m] = yz[m];
        __syncthreads();
        const float y = L.YB[l];
        const float dv = y - wave_sum(y) * RD;
        const float sg = sqrtf(wave_sum(dv * dv) * RD + a.eps);
        const float yh = dv / sg;
        const float dz = L.DZ[t][l];
        const float dyh = dz * gam;
        dzl = (dyh - wave_sum(dyh) * RD - yh * (wave_sum(dyh * yh) * RD)) / sg;
        if (w == 0) {
          dgam = fmaf(dz, yh, dgam);
          dbet += dz;
        }
        for (int s = 0; s <= t; ++s) {
          const float v = wave_sum(L.E[s][l] * dzl);
          if (w == 0 && l == 0) L.EDT[s] = v;
        }
      }
      // 2. A2 += dz c^T; partials of W2b^T dz   (LN: dy_z for dz)
      {
        const float4 c4 = ld4(&L.CV[4 * l]);
        float4 p4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float dzv = LN ? readlane(dzl, 8 * w + m) : L.DZ[t][8 * w + m];
          a2[m] = axpy(a2[m], dzv, c4);
          p4 = axpy(p4, dzv, w2b[m]);
        }
        st4(&L.red1[w][4 * l], p4);
      }
      __syncthreads();
      // 3. du = (W2_t^T dz) * GELU'(u); the dots g_s . du (wave 0)
      if (w == 0) {
        float du[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int c = 4 * l + x;
          float wz = 0.f;
#pragma unroll
          for (int v = 0; v < NW; ++v) wz += L.red1[v][c];
          for (int s = 0; s <= t; ++s) wz = fmaf(-L.ET[s] * (LN ? L.EDT[s] : L.ED[s][t]), L.A[s][c], wz);
          du[x] = wz * L.CPV[c];
        }
        st4(&L.DU[4 * l], make_float4(du[0], du[1], du[2], du[3]));
        for (int s = 0; s <= t; ++s) {
          const float part = wave_sum(dot4(ld4(&L.G[s][4 * l]), make_float4(du[0], du[1], du[2], du[3])));
          if (l == 0) L.GD[s] = part;
        }
      }
      __syncthreads();
      // 4. A1 += du q^T and the products with A1, A2 at token t
      float de1[8];
      {
        float4 x4 = make_float4(0.f, 0.f, 0.f, 0.f), y4 = x4;
        float pe = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int j = 32 * w + 4 * r + g;
          const float du = L.DU[j];
          a1[r] = axpy(a1[r], du, q4);
          x4 = axpy(x4, du, w1b[r]);                 // W1b^T du
          const float ak = sum16(dot4(a1[r], k4));   // (A1 k)_j
          const float gv = L.G[t][j];
          y4 = axpy(y4, gv, a1[r]);                  // A1^T g
          float ga, gp, gpp;
          gelu3(L.H[t][j], ga, gp, gpp);
          const float dg = -et * ak;
          if (li == 0) {
            L.DH1[j] = dg * L.S[t][j] * gpp;
            L.DS[t][j] = dg * gp;
            pe = fmaf(gv, ak, pe);
          }
        }
        x4 = rows4(x4);
        y4 = rows4(y4);
        if (g == 0) {
          st4(&L.red2[w][4 * li], x4);
          st4(&L.red2b[w][4 * li], y4);
        }
        pe = wave_sum(pe);
        if (l == 0) L.reta[0][w] = pe;
        const float4 av4 = ld4(&L.A[t][4 * l]);
        float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
        float pe2 = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float a2a = wave_sum(dot4(a2[m], av4));  // (A2 a)_i
          const float ev = L.E[t][8 * w + m];
          de1[m] = -et * a2a;
          pe2 = fmaf(ev, a2a, pe2);
          z4 = axpy(z4, ev, a2[m]);                      // A2^T e
        }
        st4(&L.red1b[w][4 * l], z4);
        if (l == 0) L.reta[1][w] = pe2;
      }
      __syncthreads();
      // 5. dq, deta; de = -eta A2 a + W2b ds, dy, dv; partials of W2b^T dy
      if (w == 0 && g == 0) {
        float4 dq = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int v = 0; v < NW; ++v) {
          const float4 x = ld4(&L.red2[v][4 * li]);
          dq = make_float4(dq.x + x.x, dq.y + x.y, dq.z + x.z, dq.w + x.w);
        }
        for (int s = 0; s <= t; ++s) dq = axpy(dq, -L.ET[s] * L.GD[s], ld4(&L.K[s][4 * li]));
        if constexpr (LN) {  // the residual of z = q + LN(...)
          const float4 r = ld4(&L.DZ[t][4 * li]);
          dq = make_float4(dq.x + r.x, dq.y + r.y, dq.z + r.z, dq.w + r.w);
        }
        st4(a.dQ + base + o + 4 * li, dq);
      }
      if (tid == 0) {
        float sum = 0.f;
        for (int v = 0; v < NW; ++v) sum += L.reta[0][v] + L.reta[1][v];
        a.deta[static_cast<size_t>(chain) * T + t0 + t] = -sum;
      }
      if constexpr (LN) {
        const float4 ds4 = ld4(&L.DS[t][4 * l]);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float de = de1[m] + wave_sum(dot4(w2b[m], ds4));
          if (l == m) L.DEB[8 * w + m] = de;
        }
        __syncthreads();
        // the K side's layer norm backward, output l in lane l
        const float del = L.DEB[l], yh = L.YH[t][l], gf = L.GF[t][l], sg = L.SIG[t];
        const float mdey = wave_sum(del * yh) * RD;
        const float dgl = (del - wave_sum(del) * RD - yh * mdey) / sg;
        const float dyh = fmaf(2.f * gam * gam, dgl, -(wave_sum(gf * yh) * RD * del + mdey * gf) / sg);
        const float dsg = -wave_sum(del * L.E[t][l]) / sg;
        const float dyl = (dyh - wave_sum(dyh) * RD - yh * (wave_sum(dyh * yh) * RD)) / sg + dsg * RD * yh;
        if (w == 0) {
          L.DY[t][l] = dyl;
          a.dV[base + o + l] = -2.f * gam * dgl;
          L.DKR[l] = 2.f * gam * dgl;
          const float fv = L.K[t][l] + gam * yh + bet - L.V[t][l];
          dgam = fmaf(dgl, 2.f * fv + 2.f * gam * yh, dgam);
          dbet = fmaf(2.f * gam, dgl, dbet);
        }
        float4 q4b = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int m = 0; m < 8; ++m) q4b = axpy(q4b, readlane(dyl, 8 * w + m), w2b[m]);  // W2b^T dy
        st4(&L.red1[w][4 * l], q4b);
      } else {
        const float4 ds4 = ld4(&L.DS[t][4 * l]);
        float4 q4b = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float de = de1[m] + wave_sum(dot4(w2b[m], ds4));
          const float dy = 2.f * de;
          if (l == m) {
            L.DY[t][8 * w + m] = dy;
            a.dV[base + o + 8 * w + m] = -dy;
          }
          q4b = axpy(q4b, dy, w2b[m]);                   // W2b^T dy
        }
        st4(&L.red1[w][4 * l], q4b);
      }
      __syncthreads();
      // 6. da = -eta A2^T e + W2b^T dy (wave 0)
      if (w == 0) {
        float da[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int c = 4 * l + x;
          float s1 = 0.f, s2 = 0.f;
#pragma unroll
          for (int v = 0; v < NW; ++v) {
            s1 += L.red1b[v][c];
            s2 += L.red1[v][c];
          }
          da[x] = fmaf(-et, s1, s2);
        }
        st4(&L.DA[4 * l], make_float4(da[0], da[1], da[2], da[3]));
      }
      __syncthreads();
      // 7. dh; partials of W1b^T dh
      {
        float4 v4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int j = 32 * w + 4 * r + g;
          float ga, gp, gpp;
          gelu3(L.H[t][j], ga, gp, gpp);
          const float dh = fmaf(L.DA[j], gp, L.DH1[j]);
          if (li == 0) L.DH_[t][j] = dh;
          v4 = axpy(v4, dh, w1b[r]);
        }
        v4 = rows4(v4);
        if (g == 0) st4(&L.red2c[w][4 * li], v4);
      }
      __syncthreads();
      // 8. dk = -eta A1^T g + W1b^T dh
      if (w == 0 && g == 0) {
        float4 dk = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int v = 0; v < NW; ++v) {
          const float4 x = ld4(&L.red2b[v][4 * li]), y = ld4(&L.red2c[v][4 * li]);
          dk = make_float4(fmaf(-et, x.x, dk.x + y.x), fmaf(-et, x.y, dk.y + y.y), fmaf(-et, x.z, dk.z + y.z),
                           fmaf(-et, x.w, dk.w + y.w));
        }
        if constexpr (LN) {  // k's own part of f(k) = k + LN(...) in the loss
          const float4 r = ld4(&L.DKR[4 * li]);
          dk = make_float4(dk.x + r.x, dk.y + r.y, dk.z + r.z, dk.w + r.w);
        }
        st4(a.dK + base + o + 4 * li, dk);
      }
    }
    // the mini-batch start: A1 += sum dh k^T, A2 += sum (e ds^T + dy a^T)
    for (int t = 0; t < nt; ++t) {
      const float4 k4 = ld4(&L.K[t][4 * li]);
      const float4 ds4 = ld4(&L.DS[t][4 * l]);
      const float4 av4 = ld4(&L.A[t][4 * l]);
#pragma unroll
      for (int r = 0; r < 8; ++r) a1[r] = axpy(a1[r], L.DH_[t][32 * w + 4 * r + g], k4);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        a2[m] = axpy(a2[m], L.E[t][8 * w + m], ds4);
        a2[m] = axpy(a2[m], L.DY[t][8 * w + m], av4);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    st4(a.dW1 + static_cast<int64_t>(chain) * st_sz + off1(r), a1[r]);
    st4(a.dW2 + static_cast<int64_t>(chain) * st_sz + off2(r), a2[r]);
  }
  if constexpr (LN) {
    if (w == 0) {
      a.dgamma[static_cast<int64_t>(chain) * D + l] = dgam;
      a.dbeta[static_cast<int64_t>(chain) * D + l] = dbet;
    }
  }
}

}  // namespace

bool mlp_bwd_supported(int d, int dh, int b) { return d == D && dh == DH && b >= 1 && b <= BT; }

hipError_t launch_mlp_bwd(const MlpBwdArgs& a, hipStream_t s) {
  dim3 grid(a.B * a.H), block(NT);
  if (a.gamma) {
    if (a.in_dtype == 0)
      hipLaunchKernelGGL((ttt_mlp_bwd_d64h256<float, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((ttt_mlp_bwd_d64h256<uint16_t, true>), grid, block, 0, s, a);
  } else if (a.in_dtype == 0) {
    hipLaunchKernelGGL((ttt_mlp_bwd_d64h256<float, false>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((ttt_mlp_bwd_d64h256<uint16_t, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace ttt
