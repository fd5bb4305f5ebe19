// Portable fp32 TTT-Linear backward (dual form).
//
// Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
// (aharts.cn / itmax.cn), part 03 §4 (the layer is trained end to end), §6
// (mini-batch GD), §7 (dual form), §9 (TTT-Linear).
//
// One workgroup per (sequence, head) walks the mini-batches from last to
// first with W and its adjoint A in LDS; every contraction is a plain fp32
// FMA loop.  Per mini-batch (token-major rows; W row i = output i; eta_s per
// token; the saved E[s][i] = (W k_s - v_s)[i] at the mini-batch-start W):
//   S[s][t]  = k_s . q_t                                     (s <= t)
//   P[s][i]  = sum_c A[i][c] K[s][c]
//   dE[s][i] = -2 eta_s (sum_{t >= s} S[s][t] dZ[t][i] + P[s][i]),  dV = -dE
//   W[i][c] += 2 sum_s eta_s E[s][i] K[s][c]      (back to the mini-batch start)
//   Y[s][t]  = -2 e_s . dz_t                                 (s <= t)
//   dQ[t][c] = sum_i dZ[t][i] W[i][c] + sum_s eta_s Y[s][t] K[s][c]
//   dK[s][c] = sum_i (dE[s][i] W[i][c] - 2 eta_s E[s][i] A[i][c]) + eta_s sum_t Y[s][t] Q[t][c]
//   deta_s   = sum_t Y[s][t] S[s][t] - 2 sum_i E[s][i] P[s][i]
//   A[i][c] += sum_t dZ[t][i] Q[t][c] + sum_s dE[s][i] K[s][c]
#include "args_bwd.h"

namespace ttt {
namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ float load_val(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_val<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_val<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_bits_to_f32(p[i]);
}

template <typename T>
__device__ __forceinline__ void store_val(T* p, size_t i, float x);
template <>
__device__ __forceinline__ void store_val<float>(float* p, size_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void store_val<uint16_t>(uint16_t* p, size_t i, float x) {
  p[i] = f32_to_bf16_bits(x);
}

template <int D, int BMAX, typename InT, typename GT>
__global__ __launch_bounds__(kThreads) void ttt_linear_bwd_generic_kernel(BwdArgs a) {
  __shared__ float W[D][D + 1];
  __shared__ float A[D][D + 1];
  __shared__ float Ks[BMAX][D + 1];
  __shared__ float Qs[BMAX][D + 1];
  __shared__ float Es[BMAX][D + 1];
  __shared__ float Zs[BMAX][D + 1];   // dZ
  __shared__ float dEs[BMAX][D + 1];
  __shared__ float Ps[BMAX][D + 1];
  __shared__ float Ss[BMAX][BMAX + 1];
  __shared__ float Ys[BMAX][BMAX + 1];
  __shared__ float et[BMAX];

  const int tid = threadIdx.x;
  const int chain = blockIdx.x;
  const int bi = chain / a.H;
  const int h = chain - bi * a.H;
  const int b = a.b;

  const float* wf = a.Wf + static_cast<int64_t>(chain) * D * D;
  const float* af = a.dWf ? a.dWf + static_cast<int64_t>(chain) * D * D : nullptr;
  for (int x = tid; x < D * D; x += kThreads) {
    W[x / D][x % D] = wf[x];
    A[x / D][x % D] = af ? af[x] : 0.f;
  }

  const size_t base = static_cast<size_t>(chain) * a.T * D;
  const InT* Qg = static_cast<const InT*>(a.Q) + base;
  const InT* Kg = static_cast<const InT*>(a.K) + base;
  const float* Eg = a.E + base;
  const GT* Zg = static_cast<const GT*>(a.dZ) + base;
  GT* dQg = static_cast<GT*>(a.dQ) + base;
  GT* dKg = static_cast<GT*>(a.dK) + base;
  GT* dVg = static_cast<GT*>(a.dV) + base;
  float* detag = a.deta + static_cast<size_t>(chain) * a.T;
  const float* eg = a.eta + bi * a.esb + h * a.esh;

  const int nb = a.T / b;
  for (int n = nb - 1; n >= 0; --n) {
    const int t0 = n * b;
    __syncthreads();  // previous mini-batch finished with the tiles, W and A
    for (int x = tid; x < b * D; x += kThreads) {
      const int t = x / D, c = x % D;
      const size_t o = static_cast<size_t>(t0) * D + x;
      Ks[t][c] = load_val<InT>(Kg, o);
      Qs[t][c] = load_val<InT>(Qg, o);
      Es[t][c] = Eg[o];
      Zs[t][c] = load_val<GT>(Zg, o);
    }
    for (int t = tid; t < b; t += kThreads) et[t] = eg[static_cast<int64_t>(t0 + t) * a.est];
    __syncthreads();

    // S (masked) and Y = -2 e_s . dz_t (masked)
    for (int x = tid; x < b * b; x += kThreads) {
      const int s = x / b, t = x % b;
      float sv = 0.f, yv = 0.f;
      if (s <= t) {
        for (int c = 0; c < D; ++c) {
          sv = fmaf(Ks[s][c], Qs[t][c], sv);
          yv = fmaf(Es[s][c], Zs[t][c], yv);
        }
        yv *= -2.f;
      }
      Ss[s][t] = sv;
      Ys[s][t] = yv;
    }
    // P = K A^T at the mini-batch-end adjoint
    for (int x = tid; x < b * D; x += kThreads) {
      const int s = x / D, i = x % D;
      float pv = 0.f;
      for (int c = 0; c < D; ++c) pv = fmaf(A[i][c], Ks[s][c], pv);
      Ps[s][i] = pv;
    }
    __syncthreads();

    // dE, dV
    for (int x = tid; x < b * D; x += kThreads) {
      const int s = x / D, i = x % D;
      float acc = Ps[s][i];
      for (int t = s; t < b; ++t) acc = fmaf(Ss[s][t], Zs[t][i], acc);
      const float de = -2.f * et[s] * acc;
      dEs[s][i] = de;
      store_val<GT>(dVg, static_cast<size_t>(t0) * D + x, -de);
    }
    // deta
    for (int s = tid; s < b; s += kThreads) {
      float acc = 0.f;
      for (int t = s; t < b; ++t) acc = fmaf(Ys[s][t], Ss[s][t], acc);
      float ep = 0.f;
      for (int i = 0; i < D; ++i) ep = fmaf(Es[s][i], Ps[s][i], ep);
      detag[t0 + s] = acc - 2.f * ep;
    }
    // back to the mini-batch-start state
    for (int x = tid; x < D * D; x += kThreads) {
      const int i = x / D, c = x % D;
      float wv = W[i][c];
      for (int s = 0; s < b; ++s) wv = fmaf(2.f * et[s] * Es[s][i], Ks[s][c], wv);
      W[i][c] = wv;
    }
    __syncthreads();

    // dQ, dK (A still the mini-batch-end adjoint)
    for (int x = tid; x < b * D; x += kThreads) {
      const int s = x / D, c = x % D;  // s is the token (t for dQ)
      float q = 0.f, k = 0.f, ea = 0.f;
      for (int i = 0; i < D; ++i) {
        q = fmaf(Zs[s][i], W[i][c], q);
        k = fmaf(dEs[s][i], W[i][c], k);
        ea = fmaf(Es[s][i], A[i][c], ea);
      }
      float qy = 0.f, ky = 0.f;
      for (int u = 0; u <= s; ++u) qy = fmaf(et[u] * Ys[u][s], Ks[u][c], qy);  // u <= t
      for (int u = s; u < b; ++u) ky = fmaf(Ys[s][u], Qs[u][c], ky);           // u >= s
      k = k - 2.f * et[s] * ea + et[s] * ky;
      store_val<GT>(dQg, static_cast<size_t>(t0) * D + x, q + qy);
      store_val<GT>(dKg, static_cast<size_t>(t0) * D + x, k);
    }
    __syncthreads();

    // adjoint of the mini-batch-start state
    for (int x = tid; x < D * D; x += kThreads) {
      const int i = x / D, c = x % D;
      float av = A[i][c];
      for (int t = 0; t < b; ++t) {
        av = fmaf(Zs[t][i], Qs[t][c], av);
        av = fmaf(dEs[t][i], Ks[t][c], av);
      }
      A[i][c] = av;
    }
  }
  __syncthreads();
  float* dw = a.dW0 + static_cast<int64_t>(chain) * D * D;
  for (int x = tid; x < D * D; x += kThreads) dw[x] = A[x / D][x % D];
}

template <int D, int BMAX>
hipError_t launch_d(const BwdArgs& a, hipStream_t s) {
  dim3 grid(a.B * a.H), block(kThreads);
  if (a.in_dtype == 0 && a.out_dtype == 0)
    hipLaunchKernelGGL((ttt_linear_bwd_generic_kernel<D, BMAX, float, float>), grid, block, 0, s, a);
  else if (a.in_dtype == 0)
    hipLaunchKernelGGL((ttt_linear_bwd_generic_kernel<D, BMAX, float, uint16_t>), grid, block, 0, s, a);
  else if (a.out_dtype == 0)
    hipLaunchKernelGGL((ttt_linear_bwd_generic_kernel<D, BMAX, uint16_t, float>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_linear_bwd_generic_kernel<D, BMAX, uint16_t, uint16_t>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool linear_bwd_generic_supported(int d, int b) {
  if (b < 1) return false;
  if (d == 16) return b <= 64;
  if (d == 32) return b <= 32;
  if (d == 64) return b <= 16;
  return false;
}

const char* linear_bwd_generic_name(int d) {
  switch (d) {
    case 16: return "ttt_linear_bwd_generic_kernel<16>";
    case 32: return "ttt_linear_bwd_generic_kernel<32>";
    case 64: return "ttt_linear_bwd_generic_kernel<64>";
    default: return nullptr;
  }
}

hipError_t launch_linear_bwd_generic(const BwdArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_d<16, 64>(a, s);
    case 32: return launch_d<32, 32>(a, s);
    case 64: return launch_d<64, 16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ttt
