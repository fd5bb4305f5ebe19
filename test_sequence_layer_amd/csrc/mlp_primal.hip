// TTT-MLP in the primal form: one token at a time, on the GPU.
//
// Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
// (aharts.cn / itmax.cn), part 03 §6 (mini-batch GD: every gradient of a
// mini-batch is taken at its start state), §7 (the naive token-by-token form),
// §9 (TTT-MLP: f(x) = W2 GELU(W1 x), hidden width 4d), and part 04 §3
// (generation is sequential and uses the primal form; Fig 15 compares
// TTT-MLP generation with TTT-Linear).
//
// Per token t at absolute position p (W1b, W2b the mini-batch-start state):
//   if p % b == 0:  W1b <- W1, W2b <- W2
//   h = W1b k,  a = GELU(h),  e = 2 (W2b a - v)
//   s = W2b^T e,  delta = s * GELU'(h)
//   W2 <- W2 - eta e a^T,   W1 <- W1 - eta delta k^T
//   z = W2 GELU(W1 q)       (the updated state)
// with W1 [dh][d] (h = W1 k) and W2 [d][dh] row-major, d = 64, dh = 256.
//
// One workgroup of 8 waves per (sequence, head) holds W1, W2, W1b, W2b in
// registers for the whole call (128 floats per lane), so a decode call reads
// and writes each state once and a full-length primal forward reads W0 once.
// Layouts (w = wave, l = lane, g = l / 16, li = l % 16):
//   W1 row j = 32 w + 4 r + g, columns 4 li .. 4 li + 3   (r = 0..7): a 1 KB
//      contiguous block per (wave, r), and h_j a sum over the 16 lanes of a
//      DPP row;
//   W2 row i = 8 w + m, columns 4 l .. 4 l + 3            (m = 0..7): one 1 KB
//      row per (wave, m), and y_i a sum over the whole wave.
// The hidden activations cross from the W1 layout to the W2 layout through
// LDS (ak, aq), and the partial sums of W2b^T e over each wave's 8 rows back
// through LDS (sp): three barriers per token.  W1 q of the updated state is
// taken as W1 q - eta delta (k . q), from the W1 q of the state before the
// step, which the W1 pass computes together with W1b k.
//
// With layer norm and residual inside f (part 03 §9: f(x) = x + LN(W2 GELU(W1 x)),
// LN over the d outputs with per-head gamma, beta), ttt_mlp_ln_primal_d64h256
// replaces e by the loss gradient at the pre-norm output y = W2b a:
//   yh = (y - mean y) / sqrt(var y + eps),  g = gamma (k + gamma yh + beta - v)
//   e = 2 (g - mean g - yh mean(g yh)) / sqrt(var y + eps)
// and writes z = q + LN(W2 GELU(W1 q)).  Each wave's 8 pre-norm outputs go
// to LDS; after one barrier every wave holds all 64, one per lane, takes the
// statistics and the two LN-backward means as wave sums, and reads the e of
// its own 8 rows from the lanes that hold them.  The output's pre-norm values
// take the same way, and wave 0 normalises them: five barriers per token.
#include "gelu.h"
#include "args_primal.h"
#include "mfma_common.h"

namespace ttt {
namespace {

using mfma::sum16;
using mfma::sum_rows;

constexpr int D = 64;
constexpr int DH = 256;
constexpr int NW = 8;
constexpr int NT = 64 * NW;
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

__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return fmaf(a.x, b.x, fmaf(a.y, b.y, fmaf(a.z, b.z, a.w * b.w)));
}
// x - c * y, elementwise
__device__ __forceinline__ float4 sub_scaled(float4 x, float c, float4 y) {
  return make_float4(fmaf(-c, y.x, x.x), fmaf(-c, y.y, x.y), fmaf(-c, y.z, x.z), fmaf(-c, y.w, x.w));
}

// The sum over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ float wave_sum(float x) { return sum_rows(sum16(x)); }

// Mean and 1/sqrt(var + eps) of the 64 values x (one per lane), centred.
__device__ __forceinline__ void wave_stats(float x, float eps, float& mu, float& rs) {
  mu = wave_sum(x) * (1.f / D);
  const float dv = x - mu;
  rs = rsqrtf(fmaf(wave_sum(dv * dv), 1.f / D, eps));
}

template <bool LN, typename InT, typename OutT>
__device__ __forceinline__ void mlp_primal_body(const MlpPrimalArgs& a) {
  __shared__ float ks[TB][D], qs[TB][D], vs[TB][D];
  __shared__ float es[TB];
  __shared__ float zs[TB][D];
  __shared__ __align__(16) float ak[DH];  // GELU(W1b k)
  __shared__ __align__(16) float aq[DH];  // GELU(W1 q) of the updated state
  __shared__ __align__(16) float sp[NW][DH];
  __shared__ float lny[D];                // layer norm: a token's 64 pre-norm outputs

  const int tid = threadIdx.x;
  // (the layer norm's lane reads need the wave index in a scalar register)
  const int l = tid & 63, w = LN ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6, g = l >> 4, li = l & 15;
  const int chain = blockIdx.x;
  const int bi = chain / a.H, h = chain - bi * a.H;
  // layer norm: lane l handles output l
  float gam = 0.f, bet = 0.f;
  if constexpr (LN) gam = a.gamma[h * D + l], bet = a.beta[h * D + l];

  // position of the next token within its mini-batch
  int ph = static_cast<int>(a.pos % a.b);

  float4 w1[8], w1b[8], w2[8], w2b[8];
  const int64_t in_off = bi * a.w_in_bstride + static_cast<int64_t>(h) * DH * D;
  auto off1 = [&](int r) { return static_cast<int64_t>(32 * w + 4 * r + g) * D + 4 * li; };
  auto off2 = [&](int m) { return static_cast<int64_t>(8 * w + m) * DH + 4 * l; };
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    w1[r] = *reinterpret_cast<const float4*>(a.W1_in + in_off + off1(r));
    w2[r] = *reinterpret_cast<const float4*>(a.W2_in + in_off + off2(r));
  }
  // Wb is read only if the first token does not start a mini-batch itself
  if (ph != 0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      w1b[r] = *reinterpret_cast<const float4*>(a.W1b_in + in_off + off1(r));
      w2b[r] = *reinterpret_cast<const float4*>(a.W2b_in + in_off + off2(r));
    }
  } else {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      w1b[r] = w1[r];
      w2b[r] = w2[r];
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
    __syncthreads();  // the previous block's tiles and outputs are consumed
    for (int x = tid; x < nt * D; x += NT) {
      const size_t gi = static_cast<size_t>(t0) * D + x;
      ks[x / D][x % D] = ld_in<InT>(Kg, gi);
      qs[x / D][x % D] = ld_in<InT>(Qg, gi);
      vs[x / D][x % D] = ld_in<InT>(Vg, gi);
    }
    if (tid < nt) es[tid] = eg[static_cast<int64_t>(t0 + tid) * a.est];
    __syncthreads();

    for (int u = 0; u < nt; ++u) {
      if (ph == 0) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          w1b[r] = w1[r];
          w2b[r] = w2[r];
        }
        wb_moved = true;
      }
      const float4 k4 = *reinterpret_cast<const float4*>(&ks[u][4 * li]);
      const float4 q4 = *reinterpret_cast<const float4*>(&qs[u][4 * li]);
      const float et = es[u];

      // W1 pass: h = W1b k and W1 q (before the step), per DPP row
      float hk[8], hq[8], gp[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        hk[r] = sum16(dot4(w1b[r], k4));
        hq[r] = sum16(dot4(w1[r], q4));
      }
      const float kq = sum16(dot4(k4, q4));
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        float gv;
        gelu_and_prime(hk[r], gv, gp[r]);
        if (li == 0) ak[32 * w + 4 * r + g] = gv;
      }
      __syncthreads();

      // W2 pass: e = 2 (W2b a - v) over this wave's rows, the partial
      // W2b^T e, and the W2 step
      const float4 a4 = *reinterpret_cast<const float4*>(&ak[4 * l]);
      float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (LN) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float y = wave_sum(dot4(w2b[m], a4));
          if (l == m) lny[8 * w + m] = y;
        }
        __syncthreads();
        float mu, rs;
        const float yl = lny[l];
        wave_stats(yl, a.eps, mu, rs);
        const float yh = (yl - mu) * rs;
        const float gl = gam * (fmaf(gam, yh, bet) + ks[u][l] - vs[u][l]);
        const float m1 = wave_sum(gl) * (1.f / D), m2 = wave_sum(gl * yh) * (1.f / D);
        const float el = 2.f * rs * (gl - m1 - yh * m2);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float e = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(el), 8 * w + m));
          s4 = sub_scaled(s4, -e, w2b[m]);
          w2[m] = sub_scaled(w2[m], et * e, a4);
        }
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float y = sum_rows(sum16(dot4(w2b[m], a4)));
          const float e = 2.f * (y - vs[u][8 * w + m]);
          s4 = sub_scaled(s4, -e, w2b[m]);
          w2[m] = sub_scaled(w2[m], et * e, a4);
        }
      }
      *reinterpret_cast<float4*>(&sp[w][4 * l]) = s4;
      __syncthreads();

      // W1 step and the output's hidden activations
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int j = 32 * w + 4 * r + g;
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < NW; ++v) s += sp[v][j];
        const float dl = s * gp[r];
        w1[r] = sub_scaled(w1[r], et * dl, k4);
        const float hn = fmaf(-et * dl, kq, hq[r]);
        if (li == 0) aq[j] = gelu(hn);
      }
      __syncthreads();

      // z = W2 aq (the updated W2)
      const float4 a4q = *reinterpret_cast<const float4*>(&aq[4 * l]);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float z = sum_rows(sum16(dot4(w2[m], a4q)));
        if (l == m) {
          if constexpr (LN)
            lny[8 * w + m] = z;
          else
            zs[u][8 * w + m] = z;
        }
      }
      if constexpr (LN) {
        // lny's pre-norm values of W2 b were read before the sp barrier
        __syncthreads();
        if (w == 0) {
          float mu, rs;
          const float zl = lny[l];
          wave_stats(zl, a.eps, mu, rs);
          zs[u][l] = qs[u][l] + fmaf(gam, (zl - mu) * rs, bet);
        }
      }
      if (++ph == a.b) ph = 0;
    }
    __syncthreads();
    for (int x = tid; x < nt * D; x += NT) st_out<OutT>(Zg, static_cast<size_t>(t0) * D + x, zs[x / D][x % D]);
  }

  const int64_t out_off = static_cast<int64_t>(chain) * DH * D;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    *reinterpret_cast<float4*>(a.W1_out + out_off + off1(r)) = w1[r];
    *reinterpret_cast<float4*>(a.W2_out + out_off + off2(r)) = w2[r];
  }
  // an in-place Wb that no token re-snapshotted already holds these values
  if (a.W1b_out && (wb_moved || a.W1b_out != a.W1b_in)) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      *reinterpret_cast<float4*>(a.W1b_out + out_off + off1(r)) = w1b[r];
      *reinterpret_cast<float4*>(a.W2b_out + out_off + off2(r)) = w2b[r];
    }
  }
}

template <typename InT, typename OutT>
__global__ __launch_bounds__(NT) void ttt_mlp_primal_d64h256(MlpPrimalArgs a) {
  mlp_primal_body<false, InT, OutT>(a);
}

template <typename InT, typename OutT>
__global__ __launch_bounds__(NT) void ttt_mlp_ln_primal_d64h256(MlpPrimalArgs a) {
  mlp_primal_body<true, InT, OutT>(a);
}

template <typename InT, typename OutT>
void launch_io(const MlpPrimalArgs& a, hipStream_t s) {
  dim3 grid(a.B * a.H), block(NT);
  if (a.gamma)
    hipLaunchKernelGGL((ttt_mlp_ln_primal_d64h256<InT, OutT>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_mlp_primal_d64h256<InT, OutT>), grid, block, 0, s, a);
}

}  // namespace

bool mlp_primal_supported(int d, int dh) { return d == D && dh == DH; }

hipError_t launch_mlp_primal(const MlpPrimalArgs& a, hipStream_t s) {
  if (a.in_dtype == 0 && a.out_dtype == 0)
    launch_io<float, float>(a, s);
  else if (a.in_dtype == 0)
    launch_io<float, uint16_t>(a, s);
  else if (a.out_dtype == 0)
    launch_io<uint16_t, float>(a, s);
  else
    launch_io<uint16_t, uint16_t>(a, s);
  return hipGetLastError();
}

}  // namespace ttt
