// TTT-Linear dual-form forward on CDNA4 matrix cores for fp32 Q/K/V: d = 64,
// b = 16.
//
// Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
// (aharts.cn / itmax.cn), part 03 §6 (mini-batch GD), §7 (dual form), §9
// (TTT-Linear, f(x) = W x).
//
// The bf16-input kernel (linear_mfma.hip) with fp32 inputs: the per-mini-batch
// products are the same (P_K = K W^T, P_Q = Q W^T, S = K Q^T, E = P_K - V,
// G = -2 diag(eta) E, Z = P_Q + M G with M[t][s] = S[s][t] [s <= t], and the
// rank-16 update W^T += K^T G), and wave w again keeps rows 16w..16w+15 of W
// as MFMA accumulator tiles for the whole sequence.  What changes:
//   - Q and K are split into bf16 hi + lo pairs once, when a tile is staged
//     into LDS (|x - hi - lo| <= 2^-16 |x|), so every product that reads them
//     takes three passes (hi hi, hi lo, lo hi) where the bf16 kernel takes two
//     (P_K, P_Q: W is split too) or one (S: exact bf16 products);
//   - the update's 16-token contraction runs K_hi and K_lo against the same
//     [G_hi G_lo] operand, two MFMAs per 16x16 block;
//   - V stays fp32 in LDS, read as scalars in the E layout.
// 28 MFMAs per wave and mini-batch (the bf16 kernel: 16).  One workgroup of 4
// waves per (sequence, head); each 16-token tile of Q, K, V is 3 x 4 KB,
// loaded PF mini-batches ahead into registers (one 16-byte piece of each per
// thread), staged one step ahead into a double-buffered LDS slot; Z leaves
// through a double-buffered LDS tile as whole rows, one step late.
#include "args_linear.h"
#include "mfma_common.h"

namespace ttt {
namespace {

using namespace mfma;

constexpr int D = 64;
constexpr int BT = 16;
constexpr int ROW = 72;   // padded LDS row of a bf16 token tile (elements)
constexpr int VR = 68;    // padded LDS row of an fp32 tile (floats)
constexpr int kThreads = 256;

struct __align__(16) Slot32 {
  uint16_t qh[BT * ROW], ql[BT * ROW];
  uint16_t kh[BT * ROW], kl[BT * ROW];
  float v[BT * VR];
  float eta[BT];
};
static_assert(sizeof(Slot32) % 16 == 0, "slot size");

template <int PF, bool ETA_TOKEN, typename OutT>
__global__ __launch_bounds__(kThreads) void ttt_linear_mfma_f32_d64b16(LinearArgs a) {
  static_assert(PF >= 2, "a step stages its successor before it issues its own prefetch");
  __shared__ Slot32 slots[2];
  __shared__ __align__(16) float zbuf[2][BT * VR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int li = lane & 15;
  const int g = lane >> 4;

  const int chain = blockIdx.x;
  const int bi = chain / a.H;
  const int h = chain - bi * a.H;
  const int nb = a.T / BT;

  const size_t tok0 = static_cast<size_t>(chain) * a.T;
  const u32x4* Qg = reinterpret_cast<const u32x4*>(static_cast<const float*>(a.Q) + tok0 * D);
  const u32x4* Kg = reinterpret_cast<const u32x4*>(static_cast<const float*>(a.K) + tok0 * D);
  const u32x4* Vg = reinterpret_cast<const u32x4*>(static_cast<const float*>(a.V) + tok0 * D);
  OutT* Zg = static_cast<OutT*>(a.Z) + tok0 * D;
  const float* eg = a.eta + bi * a.esb + h * a.esh;

  // staging roles: thread tid moves the 16-byte piece tid of each 4 KB tile,
  // row prow = tid / 16, columns pcol .. pcol + 3; and the step size of token tid % 16
  const int prow = tid >> 4;
  const int pcol = (tid & 15) * 4;
  const float* srcE = eg + static_cast<int64_t>(tid & 15) * a.est;

  u32x4 rq[PF], rk[PF], rv[PF];
  float re[PF];
  auto load_step = [&](int n, u32x4& xq, u32x4& xk, u32x4& xv, float& xe) {
    const size_t o = static_cast<size_t>(n) * (BT * D / 4) + tid;  // 256 pieces per tile
    xq = ld_stream(Qg + o);
    xk = ld_stream(Kg + o);
    xv = ld_stream(Vg + o);
    xe = ETA_TOKEN ? srcE[static_cast<int64_t>(n) * BT * a.est] : 0.f;
  };
  auto stage = [&](int slot, const u32x4& xq, const u32x4& xk, const u32x4& xv, float xe) {
    Slot32& S = slots[slot];
    const int off = prow * ROW + pcol;
    float x[4];
    bf16x4 hi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(xq[i]);
    split4(x, hi, lo);
    *reinterpret_cast<bf16x4*>(&S.qh[off]) = hi;
    *reinterpret_cast<bf16x4*>(&S.ql[off]) = lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(xk[i]);
    split4(x, hi, lo);
    *reinterpret_cast<bf16x4*>(&S.kh[off]) = hi;
    *reinterpret_cast<bf16x4*>(&S.kl[off]) = lo;
    *reinterpret_cast<u32x4*>(&S.v[prow * VR + pcol]) = xv;
    if (ETA_TOKEN && tid < BT) S.eta[tid] = xe;
  };

  float eta_c = 0.f;
  if (!ETA_TOKEN && nb > 0) eta_c = eg[0];

  // resident state: wt[a][r] = W[16w + li][16a + 4g + r]
  float4v wt[4];
  {
    const float* w0 = a.W0 + bi * a.w0_bstride + static_cast<int64_t>(h) * D * D +
                      static_cast<int64_t>(16 * w + li) * D + 4 * g;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float4 x = *reinterpret_cast<const float4*>(w0 + 16 * t);
      wt[t] = float4v{x.x, x.y, x.z, x.w};
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) asm volatile("" : "+v"(wt[t]));
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the state loads retired before the ring prologue

  if (nb > 0) {
#pragma unroll
    for (int j = 0; j < PF; ++j) load_step(min(j, nb - 1), rq[j], rk[j], rv[j], re[j]);
    stage(0, rq[0], rk[0], rv[0], re[0]);
  }
  __syncthreads();

  // Z of mini-batch m from its staging tile: thread tid writes token tid / 16,
  // outputs 4 (tid % 16) .. +3 (whole 256-byte rows per 16 threads)
  auto flush_z = [&](int m) {
    const float4 x = *reinterpret_cast<const float4*>(&zbuf[m & 1][prow * VR + pcol]);
    OutT* zp = Zg + (static_cast<size_t>(m) * BT + prow) * D + pcol;
    if constexpr (sizeof(OutT) == 4) {
      st_stream(reinterpret_cast<u32x4*>(zp),
                u32x4{__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z), __float_as_uint(x.w)});
    } else {
      st_stream(reinterpret_cast<u32x2*>(zp),
                u32x2{static_cast<uint32_t>(f32_to_bf16_bits(x.x)) | (static_cast<uint32_t>(f32_to_bf16_bits(x.y)) << 16),
                      static_cast<uint32_t>(f32_to_bf16_bits(x.z)) | (static_cast<uint32_t>(f32_to_bf16_bits(x.w)) << 16)});
    }
  };

  auto step = [&](const int n, u32x4& xq, u32x4& xk, u32x4& xv, float& xe, const u32x4& yq, const u32x4& yk,
                  const u32x4& yv, const float ye) {
    stage((n + 1) & 1, yq, yk, yv, ye);
    load_step(min(n + PF, nb - 1), xq, xk, xv, xe);
    const Slot32& S = slots[n & 1];

    bf16x4 kxh[4], kxl[4], qxh[4], qxl[4];  // rows li, column groups 16t + 4g .. +3
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int o = li * ROW + 16 * t + 4 * g;
      kxh[t] = *reinterpret_cast<const bf16x4*>(&S.kh[o]);
      kxl[t] = *reinterpret_cast<const bf16x4*>(&S.kl[o]);
      qxh[t] = *reinterpret_cast<const bf16x4*>(&S.qh[o]);
      qxl[t] = *reinterpret_cast<const bf16x4*>(&S.ql[o]);
    }
    float et[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) et[r] = ETA_TOKEN ? S.eta[4 * g + r] : eta_c;

    // ---- P_K = K W^T, P_Q = Q W^T, S = K Q^T: three split passes each ----
    float4v pk = {0.f, 0.f, 0.f, 0.f}, pq = pk, sc = pk;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float w8[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        w8[r] = wt[2 * m][r];
        w8[4 + r] = wt[2 * m + 1][r];
      }
      bf16x4 h0, l0, h1, l1;
      split4(w8, h0, l0);
      split4(w8 + 4, h1, l1);
      const bf16x8 whi = cat(h0, h1), wlo = cat(l0, l1);
      const bf16x8 akh = cat(kxh[2 * m], kxh[2 * m + 1]), akl = cat(kxl[2 * m], kxl[2 * m + 1]);
      const bf16x8 aqh = cat(qxh[2 * m], qxh[2 * m + 1]), aql = cat(qxl[2 * m], qxl[2 * m + 1]);
      pk = mfma32(akh, whi, pk);
      pq = mfma32(aqh, whi, pq);
      sc = mfma32(akh, aqh, sc);
      pk = mfma32(akh, wlo, pk);
      pq = mfma32(aqh, wlo, pq);
      sc = mfma32(akh, aql, sc);
      pk = mfma32(akl, whi, pk);
      pq = mfma32(aql, whi, pq);
      sc = mfma32(akl, aqh, sc);
    }

    // ---- E^T[t = 4g+r][i = 16w+li] = P_K - V;  G = -2 diag(eta) E, split ----
    float gv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) gv[r] = -2.f * et[r] * (pk[r] - S.v[(4 * g + r) * VR + 16 * w + li]);
    bf16x4 bhi, blo;
    split4(gv, bhi, blo);
    const bf16x8 gb = cat(bhi, blo);

    // ---- Z = P_Q + M G, M[t][s] = S[s][t] [s <= t] ----
    float4v z = pq;
    {
      float mv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) mv[r] = (4 * g + r <= li) ? sc[r] : 0.f;
      bf16x4 mhi, mlo;
      split4(mv, mhi, mlo);
      z = mfma32(cat(mhi, mhi), gb, z);
      z = mfma32(cat(mlo, mlo), gb, z);
    }

    // ---- W^T[c][i] += sum_s K[s][c] G[s][i], K as hi and lo ----
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x4 kth = read_cols<ROW>(S.kh, 0, 16 * t, li, g);  // K[4g + r][16t + li]
      const bf16x4 ktl = read_cols<ROW>(S.kl, 0, 16 * t, li, g);
      wt[t] = mfma32(cat(kth, kth), gb, wt[t]);
      wt[t] = mfma32(cat(ktl, ktl), gb, wt[t]);
    }

    // ---- Z rows t = 4g + r, columns 16w + li into the staging tile ----
    if (n > 0) flush_z(n - 1);
    float* zb = &zbuf[n & 1][(4 * g) * VR + 16 * w + li];
#pragma unroll
    for (int r = 0; r < 4; ++r) zb[r * VR] = z[r];
    __syncthreads();
  };

  const int nfull = nb / PF * PF;
  for (int n0 = 0; n0 < nfull; n0 += PF) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int jn = (j + 1) % PF;
      step(n0 + j, rq[j], rk[j], rv[j], re[j], rq[jn], rk[jn], rv[jn], re[jn]);
    }
  }
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    const int jn = (j + 1) % PF;
    if (nfull + j < nb) step(nfull + j, rq[j], rk[j], rv[j], re[j], rq[jn], rk[jn], rv[jn], re[jn]);
  }
  if (nb > 0) flush_z(nb - 1);  // the last step's barrier made its tile visible

  float* wf = a.Wf + static_cast<int64_t>(chain) * D * D + static_cast<int64_t>(16 * w + li) * D + 4 * g;
#pragma unroll
  for (int t = 0; t < 4; ++t) *reinterpret_cast<float4*>(wf + 16 * t) = make_float4(wt[t][0], wt[t][1], wt[t][2], wt[t][3]);
}

#ifndef TTT_LINEAR_F32_PF
#define TTT_LINEAR_F32_PF 4
#endif

template <bool TOK>
hipError_t launch_tok(const LinearArgs& a, hipStream_t s) {
  dim3 grid(a.B * a.H), block(kThreads);
  if (a.out_dtype == 0)
    hipLaunchKernelGGL((ttt_linear_mfma_f32_d64b16<TTT_LINEAR_F32_PF, TOK, float>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_linear_mfma_f32_d64b16<TTT_LINEAR_F32_PF, TOK, uint16_t>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool linear_mfma_f32_supported(const LinearArgs& a) {
  return a.d == 64 && a.b == 16 && a.in_dtype == 0 && a.gamma == nullptr && a.Esave == nullptr && a.nchunk <= 1;
}

hipError_t launch_linear_mfma_f32(const LinearArgs& a, hipStream_t s) {
  return a.est != 0 ? launch_tok<true>(a, s) : launch_tok<false>(a, s);
}

}  // namespace ttt
