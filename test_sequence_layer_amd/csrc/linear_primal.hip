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
// DPP reduction.  Tokens are staged TB at a time through LDS as fp32; while one
// block is processed, the next full block is already loading into registers
// (pieces of 4 consecutive elements of K, Q and V per thread).
//
// The same kernel serves two entry points: the full forward (state from W0,
// written to W_final) and decode (state W and Wb read and written in place,
// continuing from position `pos`).
//
// With layer norm and residual inside f (part 03 §9: f(x) = x + LN(W x), LN
// over the d outputs with per-head gamma, beta), ttt_linear_ln_primal_kernel
// takes per token
//   y = Wb k_t,  yh = (y - mean y) / sqrt(var y + eps),  g = gamma (k_t + gamma yh + beta - v_t)
//   delta = (g - mean g - yh mean(g yh)) / sqrt(var y + eps)   (half the gradient at y)
//   W <- W - 2 eta_t delta k_t^T
//   z_t = q_t + LN(W q_t)
// The means run over the whole workgroup: each row's value goes to LDS, and
// after one barrier every thread sums the quarter of the d values matching its
// state columns and finishes with the quad sum (mean and centred variance in
// two passes over the same registers).  Three barriers per token: the
// statistics of Wb k, the two sums of the LN backward, the statistics of W q.
#include "args_primal.h"

namespace ttt {
namespace {

#ifndef TTT_PRIMAL_TB
#define TTT_PRIMAL_TB 32
#endif
constexpr int TB = TTT_PRIMAL_TB;  // tokens staged per block
constexpr int TU = 16;             // tokens per unrolled run piece
static_assert(TB % TU == 0 && TU % 4 == 0, "block holds whole unrolled pieces");
// Calls of at most TS tokens (decode) take an instantiation of their own with
// TS-token tiles and no prefetch path: fewer registers and less LDS per
// workgroup, so more of the state loads of different sequences are in flight
// per CU.  Its arithmetic is that of the short branch of the full kernel.
constexpr int TS = 8;
static_assert(TS < TB, "short calls are a special case of the short branch");

template <typename T>
__device__ __forceinline__ float ld_in(const T* p, size_t i);
template <>
__device__ __forceinline__ float ld_in<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_in<uint16_t>(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }

// Four consecutive inputs starting at element i (i a multiple of 4; the
// sequences are 16-byte aligned, so these are 16- or 8-byte loads).
template <typename T>
__device__ __forceinline__ float4 ld_in4(const T* p, size_t i);
template <>
__device__ __forceinline__ float4 ld_in4<float>(const float* p, size_t i) {
  return *reinterpret_cast<const float4*>(p + i);
}
template <>
__device__ __forceinline__ float4 ld_in4<uint16_t>(const uint16_t* p, size_t i) {
  const uint2 x = *reinterpret_cast<const uint2*>(p + i);
  return make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                     __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u));
}

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

template <int D, bool LN, bool SHORT, typename InT, typename OutT>
__device__ __forceinline__ void primal_body(const PrimalArgs& a) {
  constexpr int NT = 4 * D;
  constexpr int CQ = D / 4;  // columns per thread
  constexpr int TK = SHORT ? TS : TB;  // tokens per tile
  __shared__ float ks[TK][D], qs[TK][D], vs[TK][D], zs[TK][D + 1];
  __shared__ float es[TK];
  // layer-norm exchange: one value (ys, ys2) or pair (pr) per state row
  __shared__ __align__(16) float ys[D], ys2[D];
  __shared__ __align__(16) float2 pr[D];
  const int tid = threadIdx.x;
  const int i = tid >> 2, qd = tid & 3;
  const int chain = blockIdx.x;
  const int bi = chain / a.H, h = chain - bi * a.H;
  float gam = 0.f, bet = 0.f;
  if constexpr (LN) gam = a.gamma[h * D + i], bet = a.beta[h * D + i];

  // Position of the next token within its mini-batch, carried as a counter
  // (a 64-bit modulo per token would cost more than the token's arithmetic).
  int ph = static_cast<int>(a.pos % a.b);

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
    if (ph != 0) {
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
  // Full blocks go in unrolled TU-token pieces when mini-batch starts fall only
  // on piece boundaries (then ph stays a multiple of TU at every full block).
  const bool pieces = a.b % TU == 0 && ph % TU == 0;
  const size_t base = static_cast<size_t>(chain) * a.T * D;
  const InT* Qg = static_cast<const InT*>(a.Q) + base;
  const InT* Kg = static_cast<const InT*>(a.K) + base;
  const InT* Vg = static_cast<const InT*>(a.V) + base;
  OutT* Zg = static_cast<OutT*>(a.Z) + base;
  const float* eg = a.eta + bi * a.esb + h * a.esh;

  // A full block is TB*D elements per input, NT = 4D threads: thread tid holds
  // the 4-element pieces p*NT + tid (p < NP) of it, i.e. element 4 (p NT + tid)
  // at row 4 (p NT + tid) / D.
  constexpr int NP = TB * D / (4 * NT);
  static_assert(NP * 4 * NT == TB * D, "whole 4-element pieces per thread and input");
  float4 kr[NP], qr[NP], vr[NP];
  float er = 0.f;
  auto fetch = [&](int t0) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const size_t g = static_cast<size_t>(t0) * D + 4 * (p * NT + tid);
      kr[p] = ld_in4<InT>(Kg, g);
      qr[p] = ld_in4<InT>(Qg, g);
      vr[p] = ld_in4<InT>(Vg, g);
    }
    if (tid < TB) er = eg[static_cast<int64_t>(t0 + tid) * a.est];
  };

  // Mean and 1/sqrt(var + eps) of the d values in y[] (written by the rows
  // before a barrier): thread (i, qd) sums y[qd CQ .. qd CQ + CQ), the quad
  // sum completes it; the variance is centred, from the same registers.
  auto stats = [&](const float* y, float& mu, float& rs) {
    float r[CQ];
#pragma unroll
    for (int c = 0; c < CQ / 4; ++c) {
      const float4 x = *reinterpret_cast<const float4*>(y + qd * CQ + 4 * c);
      r[4 * c] = x.x, r[4 * c + 1] = x.y, r[4 * c + 2] = x.z, r[4 * c + 3] = x.w;
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CQ; ++c) s += r[c];
    mu = quad_sum(s) * (1.f / D);
    float s2 = 0.f;
#pragma unroll
    for (int c = 0; c < CQ; ++c) {
      const float u = r[c] - mu;
      s2 = fmaf(u, u, s2);
    }
    rs = rsqrtf(fmaf(quad_sum(s2), 1.f / D, a.eps));
  };

  auto step = [&](int t) {
    float e = 0.f;
#pragma unroll
    for (int c = 0; c < CQ; ++c) e = fmaf(Wb[c], ks[t][qd * CQ + c], e);
    e = quad_sum(e);
    if constexpr (LN) {
      if (qd == 0) ys[i] = e;
      __syncthreads();
      float mu, rs;
      stats(ys, mu, rs);
      const float yh = (e - mu) * rs;
      const float g = gam * (fmaf(gam, yh, bet) + ks[t][i] - vs[t][i]);
      if (qd == 0) pr[i] = make_float2(g, g * yh);
      __syncthreads();
      float s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int c = 0; c < CQ / 2; ++c) {
        const float4 x = *reinterpret_cast<const float4*>(pr + qd * CQ + 2 * c);
        s1 += x.x + x.z;
        s2 += x.y + x.w;
      }
      const float m1 = quad_sum(s1) * (1.f / D), m2 = quad_sum(s2) * (1.f / D);
      e = rs * (g - m1 - yh * m2);
    } else {
      e -= vs[t][i];
    }
    const float ge = es[t] * e;  // es holds -2 eta (exact scaling)
    float z = 0.f;
#pragma unroll
    for (int c = 0; c < CQ; ++c) {
      W[c] = fmaf(ge, ks[t][qd * CQ + c], W[c]);
      z = fmaf(W[c], qs[t][qd * CQ + c], z);
    }
    z = quad_sum(z);
    if constexpr (LN) {
      if (qd == 0) ys2[i] = z;
      __syncthreads();
      float mu, rs;
      stats(ys2, mu, rs);
      z = qs[t][i] + fmaf(gam, (z - mu) * rs, bet);
    }
    return z;
  };

  // Tokens [t0, t0 + nt) of a block that is not full: loaded element by element.
  auto stage_part = [&](int t0, int nt) {
    for (int x = tid; x < nt * D; x += NT) {
      const size_t gidx = static_cast<size_t>(t0) * D + x;
      ks[x / D][x % D] = ld_in<InT>(Kg, gidx);
      qs[x / D][x % D] = ld_in<InT>(Qg, gidx);
      vs[x / D][x % D] = ld_in<InT>(Vg, gidx);
    }
    if (tid < nt) es[tid] = -2.f * eg[static_cast<int64_t>(t0 + tid) * a.est];
  };
  // Token by token, with the mini-batch-start test at every token.
  auto tokens_each = [&](int nt) {
    for (int u = 0; u < nt; ++u) {
      if (ph == 0) {
#pragma unroll
        for (int j = 0; j < CQ; ++j) Wb[j] = W[j];
        wb_moved = true;
      }
      const float z = step(u);
      if (qd == 0) zs[u][i] = z;
      if (++ph == a.b) ph = 0;
    }
  };
  auto store_z = [&](int t0, int nt) {
    for (int x = tid; x < nt * D; x += NT) st_out<OutT>(Zg, static_cast<size_t>(t0) * D + x, zs[x / D][x % D]);
  };

  if (SHORT || a.T < TB) {
    // One short block (decode): no prefetch, and the state loads stay in flight
    // while the tokens load.
    stage_part(0, a.T);
    __syncthreads();
    tokens_each(a.T);
    __syncthreads();
    store_z(0, a.T);
  } else if constexpr (!SHORT) {
    // Retire the state loads first (s_waitcnt vmcnt(0)): otherwise the
    // compiler's wait counting cannot tell them from the prefetch loads and
    // waits for the whole prefetch at the first token of every block.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    fetch(0);
    for (int t0 = 0; t0 < a.T; t0 += TB) {
      const int nt = min(TB, a.T - t0);
      __syncthreads();  // previous block's tiles and outputs consumed
      if (nt == TB) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int x = 4 * (p * NT + tid);
          *reinterpret_cast<float4*>(&ks[x / D][x % D]) = kr[p];
          *reinterpret_cast<float4*>(&qs[x / D][x % D]) = qr[p];
          *reinterpret_cast<float4*>(&vs[x / D][x % D]) = vr[p];
        }
        if (tid < TB) es[tid] = -2.f * er;
        if (t0 + 2 * TB <= a.T) fetch(t0 + TB);  // the next block is full too
      } else {
        stage_part(t0, nt);
      }
      __syncthreads();
      if (nt == TB && pieces) {
        // TU-token pieces never straddle a mini-batch start: the snapshot test
        // is made once per piece, and the unrolled tokens of a piece form one
        // basic block.  The z of token u is kept by lane qd = u % 4 of its row
        // (a select, not a masked store).
#pragma unroll
        for (int c = 0; c < TB / TU; ++c) {
          if (ph == 0) {
#pragma unroll
            for (int j = 0; j < CQ; ++j) Wb[j] = W[j];
            wb_moved = true;
          }
          float zr[TU / 4];
#pragma unroll
          for (int u = 0; u < TU; ++u) {
            const float z = step(c * TU + u);
            if (qd == (u & 3)) zr[u >> 2] = z;
          }
#pragma unroll
          for (int j = 0; j < TU / 4; ++j) zs[c * TU + 4 * j + qd][i] = zr[j];
          ph += TU;
          if (ph == a.b) ph = 0;
        }
      } else {
        tokens_each(nt);
      }
      __syncthreads();
      store_z(t0, nt);
    }
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

template <int D, bool SHORT, typename InT, typename OutT>
__global__ __launch_bounds__(4 * D) void ttt_linear_primal_kernel(PrimalArgs a) {
  primal_body<D, false, SHORT, InT, OutT>(a);
}

template <int D, bool SHORT, typename InT, typename OutT>
__global__ __launch_bounds__(4 * D) void ttt_linear_ln_primal_kernel(PrimalArgs a) {
  primal_body<D, true, SHORT, InT, OutT>(a);
}

template <int D, bool LN, bool SHORT, typename InT, typename OutT>
void launch_s(const PrimalArgs& a, hipStream_t s) {
  dim3 grid(a.B * a.H), block(4 * D);
  if constexpr (LN)
    hipLaunchKernelGGL((ttt_linear_ln_primal_kernel<D, SHORT, InT, OutT>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_linear_primal_kernel<D, SHORT, InT, OutT>), grid, block, 0, s, a);
}

template <int D, bool LN, typename InT, typename OutT>
void launch_t(const PrimalArgs& a, hipStream_t s) {
  if (a.T <= TS)
    launch_s<D, LN, true, InT, OutT>(a, s);
  else
    launch_s<D, LN, false, InT, OutT>(a, s);
}

template <int D, bool LN>
hipError_t launch_d(const PrimalArgs& a, hipStream_t s) {
  if (a.in_dtype == 0 && a.out_dtype == 0)
    launch_t<D, LN, float, float>(a, s);
  else if (a.in_dtype == 0)
    launch_t<D, LN, float, uint16_t>(a, s);
  else if (a.out_dtype == 0)
    launch_t<D, LN, uint16_t, float>(a, s);
  else
    launch_t<D, LN, uint16_t, uint16_t>(a, s);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dl(const PrimalArgs& a, hipStream_t s) {
  return a.gamma ? launch_d<D, true>(a, s) : launch_d<D, false>(a, s);
}

}  // namespace

bool linear_primal_supported(int d) { return d == 16 || d == 32 || d == 64; }

const char* linear_primal_name(int d, bool ln) {
  switch (d) {
    case 16: return ln ? "ttt_linear_ln_primal_kernel<16>" : "ttt_linear_primal_kernel<16>";
    case 32: return ln ? "ttt_linear_ln_primal_kernel<32>" : "ttt_linear_primal_kernel<32>";
    case 64: return ln ? "ttt_linear_ln_primal_kernel<64>" : "ttt_linear_primal_kernel<64>";
    default: return nullptr;
  }
}

hipError_t launch_linear_primal(const PrimalArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_dl<16>(a, s);
    case 32: return launch_dl<32>(a, s);
    case 64: return launch_dl<64>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ttt
