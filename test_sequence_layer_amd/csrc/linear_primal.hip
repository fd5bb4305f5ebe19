// TTT-Linear in the primal form: one token at a time, on the GPU.
//
// Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
// (aharts.cn / itmax.cn), part 03 §6 (mini-batch GD) and §7 (the naive form
// the dual form replaces: b rank-one gradients applied one after another), and
// part 04 §3 (generation is sequential, so decoding uses the primal form).
//
// Per token t at absolute position p (gradient at the mini-batch-start state Wb):
//   if p % b == 0:  Wb <- W
//   e   = Wb k_t - v_t
//   W  <- W - 2 eta_t e k_t^T
//   z_t = W q_t
// One workgroup of 4D threads per (sequence, head): thread (i = tid / 4,
// quarter = tid % 4) owns W[i][quarter*D/4 .. +D/4) and the same slice of Wb in
// registers; the two dot products per token are finished with a 4-lane
// shuffle reduction.  Tokens are staged 16 at a time through LDS as fp32.
//
// The same kernel serves two entry points: the full forward (state from W0,
// written to W_final) and decode (state W and Wb read and written in place,
// continuing from position `pos`).
#include "ttt_internal.h"

namespace ttt {
namespace {

constexpr int TB = 16;  // tokens staged per block

template <typename T>
__device__ __forceinline__ float ld_in(const T* p, size_t i);
template <>
__device__ __forceinline__ float ld_in<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_in<uint16_t>(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }

template <typename T>
__device__ __forceinline__ void st_out(T* p, size_t i, float x);
template <>
__device__ __forceinline__ void st_out<float>(float* p, size_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void st_out<uint16_t>(uint16_t* p, size_t i, float x) { p[i] = f32_to_bf16_bits(x); }

// Sum over the 4 lanes of a quad (the 4 threads of one state row): two DPP
// quad_perm moves ([1,0,3,2], then [2,3,0,1]) fused into the adds, instead of
// shuffles through the LDS crossbar, which sit on the per-token serial chain.
// Every lane of the quad gets the same (commutative) sums as with the shuffles.
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, true));
  return x;
}

template <int D, typename InT, typename OutT>
__global__ __launch_bounds__(4 * D) void ttt_linear_primal_kernel(PrimalArgs a) {
  constexpr int NT = 4 * D;
  constexpr int CQ = D / 4;  // columns per thread
  __shared__ float ks[TB][D], qs[TB][D], vs[TB][D], zs[TB][D + 1];
  __shared__ float es[TB];

  const int tid = threadIdx.x;
  const int i = tid >> 2, qd = tid & 3;
  const int chain = blockIdx.x;
  const int bi = chain / a.H, h = chain - bi * a.H;

  // The state slice of this thread is 16-byte aligned (CQ is a multiple of 4):
  // moved with 16-byte accesses.  Wb is read only if the first token does not
  // start a mini-batch itself (then Wb <- W before any use).
  float W[CQ], Wb[CQ];
  {
    const int64_t off = bi * a.w_in_bstride + static_cast<int64_t>(h) * D * D + i * D + qd * CQ;
    const float4* w = reinterpret_cast<const float4*>(a.W_in + off);
#pragma unroll
    for (int c = 0; c < CQ / 4; ++c) {
      const float4 x = w[c];
      W[4 * c] = x.x, W[4 * c + 1] = x.y, W[4 * c + 2] = x.z, W[4 * c + 3] = x.w;
    }
    if (a.pos % a.b != 0) {
      const float4* wb = reinterpret_cast<const float4*>(a.Wb_in + off);
#pragma unroll
      for (int c = 0; c < CQ / 4; ++c) {
        const float4 x = wb[c];
        Wb[4 * c] = x.x, Wb[4 * c + 1] = x.y, Wb[4 * c + 2] = x.z, Wb[4 * c + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int c = 0; c < CQ; ++c) Wb[c] = W[c];
    }
  }
  bool wb_moved = false;  // Wb was re-snapshotted during this call
  const size_t base = static_cast<size_t>(chain) * a.T * D;
  const InT* Qg = static_cast<const InT*>(a.Q) + base;
  const InT* Kg = static_cast<const InT*>(a.K) + base;
  const InT* Vg = static_cast<const InT*>(a.V) + base;
  OutT* Zg = static_cast<OutT*>(a.Z) + base;
  const float* eg = a.eta + bi * a.esb + h * a.esh;

  for (int t0 = 0; t0 < a.T; t0 += TB) {
    const int nt = min(TB, a.T - t0);
    __syncthreads();  // previous block's tiles and outputs consumed
    for (int x = tid; x < nt * D; x += NT) {
      const size_t gidx = static_cast<size_t>(t0) * D + x;
      ks[x / D][x % D] = ld_in<InT>(Kg, gidx);
      qs[x / D][x % D] = ld_in<InT>(Qg, gidx);
      vs[x / D][x % D] = ld_in<InT>(Vg, gidx);
    }
    if (tid < nt) es[tid] = eg[static_cast<int64_t>(t0 + tid) * a.est];
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
      if ((a.pos + t0 + t) % a.b == 0) {
#pragma unroll
        for (int c = 0; c < CQ; ++c) Wb[c] = W[c];
        wb_moved = true;
      }
      float e = 0.f;
#pragma unroll
      for (int c = 0; c < CQ; ++c) e = fmaf(Wb[c], ks[t][qd * CQ + c], e);
      e = quad_sum(e) - vs[t][i];
      const float ge = -2.f * es[t] * e;
      float z = 0.f;
#pragma unroll
      for (int c = 0; c < CQ; ++c) {
        W[c] = fmaf(ge, ks[t][qd * CQ + c], W[c]);
        z = fmaf(W[c], qs[t][qd * CQ + c], z);
      }
      z = quad_sum(z);
      if (qd == 0) zs[t][i] = z;
    }
    __syncthreads();
    for (int x = tid; x < nt * D; x += NT) st_out<OutT>(Zg, static_cast<size_t>(t0) * D + x, zs[x / D][x % D]);
  }

  float4* w = reinterpret_cast<float4*>(a.W_out + static_cast<int64_t>(chain) * D * D + i * D + qd * CQ);
#pragma unroll
  for (int c = 0; c < CQ / 4; ++c) w[c] = make_float4(W[4 * c], W[4 * c + 1], W[4 * c + 2], W[4 * c + 3]);
  // an in-place Wb that no token re-snapshotted already holds these values
  if (a.Wb_out && (wb_moved || a.Wb_out != a.Wb_in)) {
    float4* wb = reinterpret_cast<float4*>(a.Wb_out + static_cast<int64_t>(chain) * D * D + i * D + qd * CQ);
#pragma unroll
    for (int c = 0; c < CQ / 4; ++c) wb[c] = make_float4(Wb[4 * c], Wb[4 * c + 1], Wb[4 * c + 2], Wb[4 * c + 3]);
  }
}

template <int D>
hipError_t launch_d(const PrimalArgs& a, hipStream_t s) {
  dim3 grid(a.B * a.H), block(4 * D);
  if (a.in_dtype == 0 && a.out_dtype == 0)
    hipLaunchKernelGGL((ttt_linear_primal_kernel<D, float, float>), grid, block, 0, s, a);
  else if (a.in_dtype == 0)
    hipLaunchKernelGGL((ttt_linear_primal_kernel<D, float, uint16_t>), grid, block, 0, s, a);
  else if (a.out_dtype == 0)
    hipLaunchKernelGGL((ttt_linear_primal_kernel<D, uint16_t, float>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_linear_primal_kernel<D, uint16_t, uint16_t>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool linear_primal_supported(int d) { return d == 16 || d == 32 || d == 64; }

const char* linear_primal_name(int d) {
  switch (d) {
    case 16: return "ttt_linear_primal_kernel<16>";
    case 32: return "ttt_linear_primal_kernel<32>";
    case 64: return "ttt_linear_primal_kernel<64>";
    default: return nullptr;
  }
}

hipError_t launch_linear_primal(const PrimalArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_d<16>(a, s);
    case 32: return launch_d<32>(a, s);
    case 64: return launch_d<64>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ttt
