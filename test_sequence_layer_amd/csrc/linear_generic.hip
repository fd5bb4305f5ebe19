// Portable fp32 TTT-Linear dual-form kernel.
//
// Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
// (aharts.cn / itmax.cn), part 03 §6 (mini-batch GD) and §7 (dual form).
//
// One workgroup per (sequence, head) walks the mini-batches in order.  The
// d x d state lives in LDS; every contraction is a plain fp32 FMA loop.  This
// is the kernel for fp32 inputs and small head dims, and a second GPU
// implementation against which the MFMA kernel is cross-checked.
//
// Per mini-batch of b tokens (token-major rows; W row i = output i):
//   E[t][i]  = sum_c W[i][c] K[t][c] - V[t][i]   (also written out when saved for the backward)
//   L[t][s]  = 2 eta_s (q_t . k_s)           for s <= t, else 0
//   Z[t][i]  = sum_c W[i][c] Q[t][c] - sum_s L[t][s] E[s][i]
//   W[i][c] -= sum_s 2 eta_s E[s][i] K[s][c]
#include "args_linear.h"

namespace ttt {
namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ float load_in(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_in<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_in<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_bits_to_f32(p[i]);
}

template <typename T>
__device__ __forceinline__ void store_out(T* p, size_t i, float x);
template <>
__device__ __forceinline__ void store_out<float>(float* p, size_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, size_t i, float x) {
  p[i] = f32_to_bf16_bits(x);
}

template <int D, int BMAX, typename InT, typename OutT>
__global__ __launch_bounds__(kThreads) void ttt_linear_generic_kernel(LinearArgs a) {
  constexpr int ITEMS = (BMAX * D + kThreads - 1) / kThreads;
  __shared__ float W[D][D + 1];
  __shared__ float Ks[BMAX][D + 1];
  __shared__ float Qs[BMAX][D + 1];
  __shared__ float Es[BMAX][D + 1];  // holds V, then E = W K - V
  __shared__ float Ls[BMAX][BMAX + 1];
  __shared__ float et[BMAX];

  const int tid = threadIdx.x;
  const int chain = blockIdx.x;
  const int bi = chain / a.H;
  const int h = chain - bi * a.H;
  const int b = a.b;

  const float* w0 = a.W0 + bi * a.w0_bstride + static_cast<int64_t>(h) * D * D;
  for (int x = tid; x < D * D; x += kThreads) W[x / D][x % D] = w0[x];

  const size_t base = static_cast<size_t>(chain) * a.T * D;
  const InT* Qg = static_cast<const InT*>(a.Q) + base;
  const InT* Kg = static_cast<const InT*>(a.K) + base;
  const InT* Vg = static_cast<const InT*>(a.V) + base;
  OutT* Zg = static_cast<OutT*>(a.Z) + base;
  const float* eg = a.eta + bi * a.esb + h * a.esh;

  const int nb = a.T / b;
  for (int n = 0; n < nb; ++n) {
    const int t0 = n * b;
    __syncthreads();  // previous mini-batch finished with the tiles and W
    for (int x = tid; x < b * D; x += kThreads) {
      const int t = x / D, c = x % D;
      const size_t g = static_cast<size_t>(t0) * D + x;
      Ks[t][c] = load_in<InT>(Kg, g);
      Qs[t][c] = load_in<InT>(Qg, g);
      Es[t][c] = load_in<InT>(Vg, g);
    }
    for (int t = tid; t < b; t += kThreads) et[t] = eg[static_cast<int64_t>(t0 + t) * a.est];
    __syncthreads();

    // W K - V (in place over V) and W Q (kept in registers)
    float zq[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int x = tid + j * kThreads;
      zq[j] = 0.f;
      if (x < b * D) {
        const int t = x / D, i = x % D;
        float pk = 0.f, pq = 0.f;
#pragma unroll 8
        for (int c = 0; c < D; ++c) {
          pk = fmaf(W[i][c], Ks[t][c], pk);
          pq = fmaf(W[i][c], Qs[t][c], pq);
        }
        Es[t][i] = pk - Es[t][i];
        if (a.Esave) a.Esave[base + static_cast<size_t>(t0) * D + x] = Es[t][i];
        zq[j] = pq;
      }
    }
    // masked, eta-scaled scores; the diagonal (s == t) is included
    for (int x = tid; x < b * b; x += kThreads) {
      const int t = x / b, s = x % b;
      float acc = 0.f;
      if (s <= t) {
        for (int c = 0; c < D; ++c) acc = fmaf(Qs[t][c], Ks[s][c], acc);
        acc *= 2.f * et[s];
      }
      Ls[t][s] = acc;
    }
    __syncthreads();

#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int x = tid + j * kThreads;
      if (x < b * D) {
        const int t = x / D, i = x % D;
        float z = zq[j];
        for (int s = 0; s <= t; ++s) z = fmaf(-Ls[t][s], Es[s][i], z);
        store_out<OutT>(Zg, static_cast<size_t>(t0) * D + x, z);
      }
    }
    // rank-b state update with the gradients taken at the mini-batch start
    for (int x = tid; x < D * D; x += kThreads) {
      const int i = x / D, c = x % D;
      float w = W[i][c];
      for (int s = 0; s < b; ++s) w = fmaf(-2.f * et[s] * Es[s][i], Ks[s][c], w);
      W[i][c] = w;
    }
  }
  __syncthreads();
  float* wf = a.Wf + static_cast<int64_t>(chain) * D * D;
  for (int x = tid; x < D * D; x += kThreads) wf[x] = W[x / D][x % D];
}

template <int D, int BMAX>
hipError_t launch_d(const LinearArgs& a, hipStream_t s) {
  dim3 grid(a.B * a.H), block(kThreads);
  if (a.in_dtype == 0 && a.out_dtype == 0)
    hipLaunchKernelGGL((ttt_linear_generic_kernel<D, BMAX, float, float>), grid, block, 0, s, a);
  else if (a.in_dtype == 0)
    hipLaunchKernelGGL((ttt_linear_generic_kernel<D, BMAX, float, uint16_t>), grid, block, 0, s, a);
  else if (a.out_dtype == 0)
    hipLaunchKernelGGL((ttt_linear_generic_kernel<D, BMAX, uint16_t, float>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_linear_generic_kernel<D, BMAX, uint16_t, uint16_t>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool linear_generic_supported(int d, int b) {
  if (b < 1) return false;
  if (d == 16 || d == 32) return b <= 64;
  if (d == 64) return b <= 32;
  return false;
}

const char* linear_generic_name(int d) {
  switch (d) {
    case 16: return "ttt_linear_generic_kernel<16>";
    case 32: return "ttt_linear_generic_kernel<32>";
    case 64: return "ttt_linear_generic_kernel<64>";
    default: return nullptr;
  }
}

hipError_t launch_linear_generic(const LinearArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_d<16, 64>(a, s);
    case 32: return launch_d<32, 64>(a, s);
    case 64: return launch_d<64, 32>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ttt
