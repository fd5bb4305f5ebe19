// TTT-MLP backward in the dual form on CDNA4 matrix cores: d = 64, dh = 256,
// b = 16, bf16 Q/K/V.
//
// Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
// (aharts.cn / itmax.cn), part 03 §4 (the layer is trained end to end, so
// every input gets a gradient), §7 (the dual form: a mini-batch's work as
// matrix products; the pages use it for the backward as well), §9 (TTT-MLP).
//
// Column form as in the forward kernel (K, Q, V, dZ are d x b, one column per
// token; W1: dh x d and W2: d x dh are the state at the mini-batch start):
//   H_K = W1 K, A_K = GELU(H_K), E = 2 (W2 A_K - V), S = W2^T E, G = S * GELU'(H_K),
//   U = W1 Q - G L1, C = GELU(U), Z = W2 C - E L2,
//   L1 = diag(eta) triu(K^T Q), L2 = diag(eta) triu(A_K^T C)   ([s][t], s <= t kept),
//   W1' = W1 - G diag(eta) K^T, W2' = W2 - E diag(eta) A_K^T.
// Backward of one mini-batch, A1 = dL/dW1' and A2 = dL/dW2' coming in from the
// later mini-batches, with S1 = K^T Q, P = A_K^T C, ED = E^T dZ, GQ = G^T dH_Q,
// M2 = -diag(eta) triu(ED), M1 = -diag(eta) triu(GQ):
//   dH_Q = (W2^T dZ + A_K M2) * GELU'(U)
//   dG   = -(dH_Q triu(S1)^T + A1 K) diag(eta),     dS = dG * GELU'(H_K)
//   dE   = -(dZ triu(P)^T + A2 A_K) diag(eta) + W2 dS,   dY = 2 dE,  dV = -dY
//   dA_K = C M2^T - A2^T E diag(eta) + W2^T dY
//   dH_K = dA_K * GELU'(H_K) + dG * S * GELU''(H_K)
//   dQ   = W1^T dH_Q + K M1,   dK = W1^T dH_K - A1^T G diag(eta) + Q M1^T
//   deta_s = -sum_{t >= s} (ED P + GQ S1)[s][t] - e_s . (A2 a_s) - g_s . (A1 k_s)
//   then A1 += dH_Q Q^T + dH_K K^T and A2 += dZ C^T + E dS^T + dY A_K^T
//   (the gradients with respect to the mini-batch-start state).
// The mini-batch-start states come from the checkpoint pass (the forward
// kernel in checkpoint mode writes them to the workspace); the mini-batches
// run last to first.
//
// Work decomposition: one 512-thread workgroup (8 waves) per (sequence,
// head); wave w owns hidden units 32w .. 32w + 31 of W1, W2, A1, A2 (in
// registers) and of every dh x b activation.  Products over the hidden
// dimension are summed across waves through per-wave partials in LDS (a fixed
// order: the results are deterministic).
//
// Tiles.  Every matrix in registers is a set of 16 x 16 accumulator tiles:
// lane l (li = l % 16, g = l / 16) holds X[4g + r][li], r = 0..3.  Such a
// tile is an operand contracted over its rows: two tiles give the 8 k-slots
// of one v_mfma_f32_16x16x32_bf16 (rows 4g + r of the first, then of the
// second), and the product's rows are the first operand's columns, its
// columns the second's.  fp32 operands enter as bf16 hi + lo (3 passes: hi hi,
// hi lo, lo hi; bf16 inputs are exact and take 2); 16-token contractions put
// two passes into one instruction.  A state matrix contracted over its other
// index is transposed on the matrix cores (its split tiles times an identity
// operand: exact), a dh x b activation through a per-wave LDS buffer.
#include "args_mlp_bwd.h"
#include "gelu.h"
#include "mfma_common.h"

namespace ttt {
namespace {

using namespace mfma;

constexpr int D = 64;
constexpr int DH = 256;
constexpr int BT = 16;
constexpr int NW = 8;
constexpr int NT = NW * 64;
constexpr int ROW = 72;    // padded bf16 row of a token tile [t][c]
constexpr int KTROW = 20;  // padded bf16 row of a transposed token tile [c][t]
constexpr int PROW = 68;   // padded fp32 row of [t][i] buffers
constexpr int SROW = 20;   // padded fp32 row of [s][t] buffers
constexpr int XR = 20;     // padded fp32 row of the per-wave transpose buffer [j][t]
constexpr int64_t ST = static_cast<int64_t>(DH) * D;  // elements of one state matrix

struct __align__(16) Smem {
  uint16_t q[BT * ROW], k[BT * ROW], v[BT * ROW];  // bf16 token rows [t][c]
  uint16_t qt[D * KTROW], kt[D * KTROW];           // the same transposed [c][t]
  float dz[BT * PROW];                             // dZ [t][i]
  float e[BT * PROW];                              // E [t][i]
  float dy[BT * PROW];                             // dY [t][i]
  float eta[BT];
  float p[BT * SROW], gq[BT * SROW], s1[BT * SROW], ed[BT * SROW];  // [s][t]
  float pa[NW][BT * PROW];  // per-wave partials [t][i]: W2 A_K, then dE, then dQ
  float pb[NW][BT * PROW];  // per-wave partials of dK [t][c]
  float pp[NW][BT * SROW];  // per-wave partials of P
  float pg[NW][BT * SROW];  // per-wave partials of GQ
  float de2[NW][BT], de4[NW][BT];  // per-wave parts of deta
  float xs[NW][32 * XR];    // per-wave transposes [j][t]
};

struct Op8 {
  bf16x8 hi, lo;
};
__device__ __forceinline__ Op8 split8(float4v a, float4v b) {
  bf16x4 ah, al, bh, bl;
  split4(a, ah, al);
  split4(b, bh, bl);
  return Op8{cat(ah, bh), cat(al, bl)};
}
// C += A B, both split: hi hi + hi lo + lo hi
__device__ __forceinline__ float4v mfma3(const Op8& a, const Op8& b, float4v c) {
  c = mfma32(a.hi, b.hi, c);
  c = mfma32(a.hi, b.lo, c);
  c = mfma32(a.lo, b.hi, c);
  return c;
}
// C += A B over one 16-row tile pair, both split, in two instructions
__device__ __forceinline__ float4v mfma3_16(float4v a, float4v b, float4v c) {
  bf16x4 ah, al, bh, bl;
  split4(a, ah, al);
  split4(b, bh, bl);
  const bf16x4 z = {};
  c = mfma32(cat(ah, ah), cat(bh, bl), c);
  c = mfma32(cat(al, z), cat(bh, z), c);
  return c;
}
__device__ __forceinline__ float4v ld4(const float* p) { return *reinterpret_cast<const float4v*>(p); }
__device__ __forceinline__ void st4(float* p, float4v x) { *reinterpret_cast<float4v*>(p) = x; }
__device__ __forceinline__ float4v ld4nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const float4v*>(p));
}
__device__ __forceinline__ float bf(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }

// GELU(x) = x Phi(x), GELU'(x) = Phi(x) + x phi(x), GELU''(x) = phi(x) (2 - x^2) of
// the 8 values of two tiles.  Phi comes from phi_poly (the CDF polynomial of
// the forward kernels) while every |x| in the wave is below sqrt 2, else from
// erff for all 8 (a wave-uniform test); phi(x) = exp(-x^2 / 2) / sqrt(2 pi).
__device__ __forceinline__ void gelu_tiles(const float4v x[2], float4v g[2], float4v gp[2], float4v gpp[2]) {
  bool big = false;
#pragma unroll
  for (int k = 0; k < 8; ++k) big |= !(x[k >> 2][k & 3] * x[k >> 2][k & 3] < 2.f);
  const bool poly = __builtin_amdgcn_ballot_w64(big) == 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float v = x[k >> 2][k & 3], u = v * v;
    const float cdf = poly ? phi_poly(v, u) : 0.5f * (1.f + erff(v * 0.70710678118654752f));
    const float pdf = 0.39894228040143268f * __builtin_amdgcn_exp2f(u * -0.72134752044448170f);
    g[k >> 2][k & 3] = v * cdf;
    gp[k >> 2][k & 3] = fmaf(v, pdf, cdf);
    gpp[k >> 2][k & 3] = pdf * (2.f - u);
  }
}

// The transposes (as bf16 hi and lo, exact) of the two tiles x0, x1: out[q]
// holds x_q^T, i.e. lane l gets x_q[li][4g + r].
__device__ __forceinline__ void transpose2(float4v x0, float4v x1, const bf16x8 ident[2], bf16x4 oh[2],
                                           bf16x4 ol[2]) {
  const Op8 x = split8(x0, x1);
  const float4v z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    oh[q] = __builtin_convertvector(mfma32(x.hi, ident[q], z), bf16x4);
    ol[q] = __builtin_convertvector(mfma32(x.lo, ident[q], z), bf16x4);
  }
}

__global__ __launch_bounds__(NT) void ttt_mlp_bwd_d64h256b16(MlpBwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar address parts
  const int li = lane & 15;
  const int g = lane >> 4;
  const int chain = blockIdx.x;
  const int bi = chain / a.H;
  const int h = chain - bi * a.H;
  const int T = a.T;
  const int nb = T / BT;

  const size_t base = static_cast<size_t>(chain) * T * D;
  const uint16_t* Qg = static_cast<const uint16_t*>(a.Q) + base;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.K) + base;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.V) + base;
  const float* DZg = a.dZ + base;
  float* dQg = a.dQ + base;
  float* dKg = a.dK + base;
  float* dVg = a.dV + base;
  float* detag = a.deta + static_cast<size_t>(chain) * T;
  const float* eg = a.eta + bi * a.esb + h * a.esh;

  // identity operands: split tiles (k-slots = the rows of two tiles) times
  // ident[q] give tile q transposed
  bf16x8 ident[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int sl = 0; sl < 8; ++sl)
      ident[q][sl] = static_cast<__bf16>((sl / 4 == q && 4 * g + (sl & 3) == li) ? 1.f : 0.f);

  // adjoints; layouts as the states below:
  // a1[jt][c4] : A1[j = 32w + 16jt + li][c = 16c4 + 4g + r]   (tile rows c, columns j)
  // a2[it][jt] : A2[i = 16it + li][j = 32w + 16jt + 4g + r]   (tile rows j, columns i)
  float4v a1[2][4], a2[4][2];
  {
    const int64_t cs = static_cast<int64_t>(chain) * ST;
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4)
        a1[jt][c4] = a.dW1f ? ld4(a.dW1f + cs + (32 * w + 16 * jt + li) * D + 16 * c4 + 4 * g) : zero4v();
#pragma unroll
      for (int it = 0; it < 4; ++it)
        a2[it][jt] = a.dW2f ? ld4(a.dW2f + cs + (16 * it + li) * DH + 32 * w + 16 * jt + 4 * g) : zero4v();
    }
  }

  float* xs = sm.xs[w];
  // [j][t] tiles (rows j = 16jt + 4g + r, columns t = li) -> [t][j] tiles (lane: X[j = 16jt + li][t = 4g + r])
  auto jt2tj = [&](const float4v x[2], float4v y[2]) {
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r) xs[(16 * jt + 4 * g + r) * XR + li] = x[jt][r];
    // one wave writes and reads its own buffer: its LDS accesses run in order
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) y[jt] = ld4(&xs[(16 * jt + li) * XR + 4 * g]);
  };

  // The state at the start of mini-batch n (the checkpoint):
  // W1 tile (jt, c4) : W1[j = 32w + 16jt + li][c = 16c4 + 4g + r]   (tile rows c, columns j)
  // W2 tile (it, jt) : W2[i = 16it + li][j = 32w + 16jt + 4g + r]   (tile rows j, columns i)
  float4v w1t[2][4], w2n[4][2];
  auto load_state = [&](int n) {
    const float* ck = a.ws + (static_cast<int64_t>(chain) * nb + n) * (2 * ST);
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) w1t[jt][c4] = ld4(ck + (32 * w + 16 * jt + li) * D + 16 * c4 + 4 * g);
#pragma unroll
      for (int it = 0; it < 4; ++it) w2n[it][jt] = ld4(ck + ST + (16 * it + li) * DH + 32 * w + 16 * jt + 4 * g);
    }
  };

  for (int n = nb - 1; n >= 0; --n) {
    const int t0 = n * BT;
    __syncthreads();  // the previous mini-batch's LDS reads are done
    // ---- stage the tokens ----
    {
      const int within = tid & 255, srow = within >> 4, scol = (within & 15) * 4;
      const uint16_t* src = (tid < 256 ? Qg : Kg) + static_cast<size_t>(t0 + srow) * D + scol;
      const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
      uint16_t* rows = tid < 256 ? sm.q : sm.k;
      uint16_t* cols = tid < 256 ? sm.qt : sm.kt;
      *reinterpret_cast<u32x2*>(&rows[srow * ROW + scol]) = x;
      cols[(scol + 0) * KTROW + srow] = static_cast<uint16_t>(x.x & 0xffffu);
      cols[(scol + 1) * KTROW + srow] = static_cast<uint16_t>(x.x >> 16);
      cols[(scol + 2) * KTROW + srow] = static_cast<uint16_t>(x.y & 0xffffu);
      cols[(scol + 3) * KTROW + srow] = static_cast<uint16_t>(x.y >> 16);
      const int vr = tid >> 5, vc = (tid & 31) * 2;
      *reinterpret_cast<uint32_t*>(&sm.v[vr * ROW + vc]) =
          __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(Vg + static_cast<size_t>(t0 + vr) * D + vc));
      *reinterpret_cast<float2v*>(&sm.dz[vr * PROW + vc]) =
          __builtin_nontemporal_load(reinterpret_cast<const float2v*>(DZg + static_cast<size_t>(t0 + vr) * D + vc));
      if (tid < BT) sm.eta[tid] = eg[static_cast<int64_t>(t0 + tid) * a.est];
    }
    // the state tiles again (from the caches) where a transpose is needed
    const float* ck = a.ws + (static_cast<int64_t>(chain) * nb + n) * (2 * ST);
    auto w1_tile = [&](int jt, int c4) { return ld4(ck + (32 * w + 16 * jt + li) * D + 16 * c4 + 4 * g); };
    auto w2_tile = [&](int it, int jt) { return ld4(ck + ST + (16 * it + li) * DH + 32 * w + 16 * jt + 4 * g); };
    float4v hk[2], hq[2], s1 = zero4v(), s1t = zero4v();
    load_state(n);
    {
      __syncthreads();

      // token rows: kx[c4] = K[t = li][16c4 + 4g .. +3] (tile rows c, columns t)
      bf16x4 kx[4], qx[4];
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        kx[c4] = *reinterpret_cast<const bf16x4*>(&sm.k[li * ROW + 16 * c4 + 4 * g]);
        qx[c4] = *reinterpret_cast<const bf16x4*>(&sm.q[li * ROW + 16 * c4 + 4 * g]);
      }
      // ---- A1: H_K, W1 Q ([j][t] tiles), S1 = K^T Q ----
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        hk[jt] = zero4v();
        hq[jt] = zero4v();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const Op8 wj = split8(w1t[jt][2 * m], w1t[jt][2 * m + 1]);
          const bf16x8 kb = cat(kx[2 * m], kx[2 * m + 1]);
          const bf16x8 qb = cat(qx[2 * m], qx[2 * m + 1]);
          hk[jt] = mfma32(wj.hi, kb, hk[jt]);
          hk[jt] = mfma32(wj.lo, kb, hk[jt]);
          hq[jt] = mfma32(wj.hi, qb, hq[jt]);
          hq[jt] = mfma32(wj.lo, qb, hq[jt]);
        }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const bf16x8 kb = cat(kx[2 * m], kx[2 * m + 1]), qb = cat(qx[2 * m], qx[2 * m + 1]);
        s1 = mfma32(kb, qb, s1);    // S1[s = 4g + r][t = li]
        s1t = mfma32(qb, kb, s1t);  // S1[s = li][t = 4g + r]
      }
    }
    float et_row[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) et_row[r] = sm.eta[4 * g + r];  // eta of token 4g + r (tile rows)
    const float et_col = sm.eta[li];                               // eta of token li (tile columns)

    // ---- A1 (cont.): GELU, partials of W2 A_K ----
    float4v ak[2], gk1[2], gk2[2];
    gelu_tiles(hk, ak, gk1, gk2);
    {
      const Op8 akop = split8(ak[0], ak[1]);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const float4v y = mfma3(split8(w2n[it][0], w2n[it][1]), akop, zero4v());  // [i = 16it + 4g + r][t = li]
        st4(&sm.pa[w][li * PROW + 16 * it + 4 * g], y);
      }
    }
    if (w == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.s1[(4 * g + r) * SROW + li] = s1[r];
    }
    __syncthreads();  // #1

    // ---- A2: E = 2 (W2 A_K - V), [t][i] ----
    {
      const int e0 = 2 * tid, t = e0 >> 6, i = e0 & 63;
      float y0 = 0.f, y1 = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        y0 += sm.pa[ww][t * PROW + i];
        y1 += sm.pa[ww][t * PROW + i + 1];
      }
      const uint32_t vv = *reinterpret_cast<const uint32_t*>(&sm.v[t * ROW + i]);
      sm.e[t * PROW + i] = 2.f * (y0 - __uint_as_float(vv << 16));
      sm.e[t * PROW + i + 1] = 2.f * (y1 - __uint_as_float(vv & 0xffff0000u));
    }
    __syncthreads();  // #2

    // ---- A3 ----
    // E, dZ tiles of a pair of i blocks: [i = 32m + 16hf + 4g + r][t = li]   (tile rows i, columns t)
    auto e_tile = [&](int it) { return ld4(&sm.e[li * PROW + 16 * it + 4 * g]); };
    auto dz_tile = [&](int it) { return ld4(&sm.dz[li * PROW + 16 * it + 4 * g]); };
    // S = W2^T E and W2^T dZ ([j][t]), ED = E^T dZ ([s][t]) and its transpose
    float4v sv[2] = {zero4v(), zero4v()}, wz[2] = {zero4v(), zero4v()};
    float4v m2, m2t;  // M2 [s = 4g + r][t = li] and M2 [s = li][t = 4g + r]
    {
      float4v ed = zero4v(), edt = zero4v();
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        // th[hf][jt] = W2[16(2m + hf) + 4g + r][32w + 16jt + li]
        bf16x4 th[2][2], tl[2][2];
        transpose2(w2n[2 * m][0], w2n[2 * m][1], ident, th[0], tl[0]);
        transpose2(w2n[2 * m + 1][0], w2n[2 * m + 1][1], ident, th[1], tl[1]);
        const Op8 eo = split8(e_tile(2 * m), e_tile(2 * m + 1)), zo = split8(dz_tile(2 * m), dz_tile(2 * m + 1));
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          const Op8 A{cat(th[0][jt], th[1][jt]), cat(tl[0][jt], tl[1][jt])};
          sv[jt] = mfma3(A, eo, sv[jt]);
          wz[jt] = mfma3(A, zo, wz[jt]);
        }
        ed = mfma3(eo, zo, ed);    // [s = 4g + r][t = li]
        edt = mfma3(zo, eo, edt);  // [t = 4g + r][s = li]
      }
      if (w == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.ed[(4 * g + r) * SROW + li] = ed[r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        m2[r] = (4 * g + r <= li) ? -et_row[r] * ed[r] : 0.f;
        m2t[r] = (li <= 4 * g + r) ? -et_col * edt[r] : 0.f;
      }
    }
    float4v gg[2];  // G [j][t]
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r) gg[jt][r] = sv[jt][r] * gk1[jt][r];
    // U = W1 Q - G L1, C = GELU(U)
    float4v cq[2], gu1[2];
    {
      float4v ggt[2];
      jt2tj(gg, ggt);
      float4v nl1;  // -L1 [s = 4g + r][t = li]
#pragma unroll
      for (int r = 0; r < 4; ++r) nl1[r] = (4 * g + r <= li) ? -et_row[r] * s1[r] : 0.f;
      float4v u[2], unused[2];
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) u[jt] = mfma3_16(ggt[jt], nl1, hq[jt]);
      gelu_tiles(u, cq, gu1, unused);
    }
    // P partial = A_K^T C over this wave's hidden units
    {
      const float4v pv = mfma3(split8(ak[0], ak[1]), split8(cq[0], cq[1]), zero4v());  // [s = 4g + r][t = li]
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.pp[w][(4 * g + r) * SROW + li] = pv[r];
    }
    // dH_Q = (W2^T dZ + A_K M2) * GELU'(U)
    float4v akt[2], dhq[2];
    jt2tj(ak, akt);
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      const float4v dc = mfma3_16(akt[jt], m2, wz[jt]);
#pragma unroll
      for (int r = 0; r < 4; ++r) dhq[jt][r] = dc[r] * gu1[jt][r];
    }
    // dG = -(dH_Q triu(S1)^T + A1 K) diag(eta); the deta part -g_s . (A1 k_s)
    float4v dg[2];
    {
      float4v dhqt[2];
      jt2tj(dhq, dhqt);
      float4v s1m;  // S1[s = li][t = 4g + r], s <= t
#pragma unroll
      for (int r = 0; r < 4; ++r) s1m[r] = (li <= 4 * g + r) ? s1t[r] : 0.f;
      float pe = 0.f;
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const float4v x1 = mfma3_16(dhqt[jt], s1m, zero4v());
        float4v x2 = zero4v();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const Op8 ao = split8(a1[jt][2 * m], a1[jt][2 * m + 1]);
          const bf16x8 kb = cat(*reinterpret_cast<const bf16x4*>(&sm.k[li * ROW + 32 * m + 4 * g]),
                                *reinterpret_cast<const bf16x4*>(&sm.k[li * ROW + 32 * m + 16 + 4 * g]));
          x2 = mfma32(ao.hi, kb, x2);
          x2 = mfma32(ao.lo, kb, x2);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          dg[jt][r] = -et_col * (x1[r] + x2[r]);
          pe = fmaf(gg[jt][r], x2[r], pe);
        }
      }
      pe = sum_rows(pe);
      if (g == 0) sm.de4[w][li] = -pe;
    }
    // GQ partial = G^T dH_Q
    {
      const float4v gqv = mfma3(split8(gg[0], gg[1]), split8(dhq[0], dhq[1]), zero4v());
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.pg[w][(4 * g + r) * SROW + li] = gqv[r];
    }
    // dS, and the GELU'' part of dH_K
    float4v ds[2], dhk1[2];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ds[jt][r] = dg[jt][r] * gk1[jt][r];
        dhk1[jt][r] = dg[jt][r] * sv[jt][r] * gk2[jt][r];
      }
    // dE partial = W2 dS - (A2 A_K) diag(eta), [s][i]; the deta part -e_s . (A2 a_s)
    {
      const Op8 dso = split8(ds[0], ds[1]), ako = split8(ak[0], ak[1]);
      float pe = 0.f;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const float4v wd = mfma3(split8(w2_tile(it, 0), w2_tile(it, 1)), dso, zero4v());
        const float4v aa = mfma3(split8(a2[it][0], a2[it][1]), ako, zero4v());
        const float4v ev = e_tile(it);
        float4v pv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pv[r] = wd[r] - et_col * aa[r];
          pe = fmaf(ev[r], aa[r], pe);
        }
        st4(&sm.pa[w][li * PROW + 16 * it + 4 * g], pv);
      }
      pe = sum_rows(pe);
      if (g == 0) sm.de2[w][li] = -pe;
    }
    // dA_K so far: C M2^T - (A2^T E) diag(eta)  (W2^T dY is added once dY is known)
    float4v dak[2];
    float4v cqt[2], dst[2];
    jt2tj(cq, cqt);
    jt2tj(ds, dst);
    {
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) dak[jt] = mfma3_16(cqt[jt], m2t, zero4v());
      float4v ae[2] = {zero4v(), zero4v()};
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        // A2 transposed: ah[hf][jt] = A2[16(2m + hf) + 4g + r][32w + 16jt + li]
        bf16x4 ah[2][2], al[2][2];
        transpose2(a2[2 * m][0], a2[2 * m][1], ident, ah[0], al[0]);
        transpose2(a2[2 * m + 1][0], a2[2 * m + 1][1], ident, ah[1], al[1]);
        const Op8 eo = split8(e_tile(2 * m), e_tile(2 * m + 1));
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) ae[jt] = mfma3(Op8{cat(ah[0][jt], ah[1][jt]), cat(al[0][jt], al[1][jt])}, eo, ae[jt]);
      }
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) dak[jt][r] -= et_col * ae[jt][r];
    }
    // the dK partial's -(A1^T G) diag(eta) ([c][t] tiles, to pb; W1^T dH_K is added later)
    {
      const Op8 go = split8(gg[0], gg[1]);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bf16x4 a1jh[2][2], a1jl[2][2];  // [jt][q] = A1[32w + 16jt + 4g + r][16(2m + q) + li]
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) transpose2(a1[jt][2 * m], a1[jt][2 * m + 1], ident, a1jh[jt], a1jl[jt]);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float4v ag = mfma3(Op8{cat(a1jh[0][q], a1jh[1][q]), cat(a1jl[0][q], a1jl[1][q])}, go, zero4v());
          float4v kv;
#pragma unroll
          for (int r = 0; r < 4; ++r) kv[r] = -et_col * ag[r];
          st4(&sm.pb[w][li * PROW + 16 * (2 * m + q) + 4 * g], kv);
        }
      }
    }
    // A1 and A2 are no longer read as the incoming adjoints: the first terms of
    // the mini-batch-start adjoints, A1 += dH_Q Q^T, A2 += dZ C^T + E dS^T
    {
      float4v dhqt[2];
      jt2tj(dhq, dhqt);
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        bf16x4 qh, ql;
        split4(dhqt[jt], qh, ql);
        const bf16x8 qb = cat(qh, ql);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const bf16x4 qt4 = *reinterpret_cast<const bf16x4*>(&sm.qt[(16 * c4 + li) * KTROW + 4 * g]);
          a1[jt][c4] = mfma32(cat(qt4, qt4), qb, a1[jt][c4]);
        }
      }
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        float4v zt, et4;  // [t = 4g + r][i = 16it + li]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          zt[r] = sm.dz[(4 * g + r) * PROW + 16 * it + li];
          et4[r] = sm.e[(4 * g + r) * PROW + 16 * it + li];
        }
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          float4v x = a2[it][jt];
          x = mfma3_16(cqt[jt], zt, x);
          x = mfma3_16(dst[jt], et4, x);
          a2[it][jt] = x;
        }
      }
    }
    __syncthreads();  // #3

    // ---- R-A: P and GQ summed over the waves ----
    {
      const int s = (tid & 255) >> 4, t = tid & 15;
      float acc = 0.f;
      if (tid < 256) {
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) acc += sm.pp[ww][s * SROW + t];
        sm.p[s * SROW + t] = acc;
      } else {
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) acc += sm.pg[ww][s * SROW + t];
        sm.gq[s * SROW + t] = acc;
      }
    }
    __syncthreads();  // #4

    // ---- R-B: dE = (the partials) - (dZ triu(P)^T) diag(eta) -> dY (LDS), dV; deta ----
    if (w < 4) {
      const int it = w;  // outputs i = 16it .. 16it + 15
      // dZ [t = 4g + r][i = 16it + li] and P'[s = li][t = 4g + r] = eta_s P[s][t] (t >= s)
      float4v zt, pt;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * g + r;
        zt[r] = sm.dz[t * PROW + 16 * it + li];
        pt[r] = (t >= li) ? et_col * sm.p[li * SROW + t] : 0.f;
      }
      float4v acc = mfma3_16(zt, pt, zero4v());  // [i = 16it + 4g + r][s = li] = sum_t dZ[t][i] P'[s][t]
      float4v sum = zero4v();
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) sum += ld4(&sm.pa[ww][li * PROW + 16 * it + 4 * g]);
      const float4v dy = 2.f * (sum - acc);
      st4(&sm.dy[li * PROW + 16 * it + 4 * g], dy);
      *reinterpret_cast<float4v*>(dVg + static_cast<size_t>(t0 + li) * D + 16 * it + 4 * g) = -dy;
    } else if (w == 4 && lane < BT) {
      const int s = lane;
      float acc = 0.f;
      for (int t = s; t < BT; ++t)
        acc += sm.ed[s * SROW + t] * sm.p[s * SROW + t] + sm.gq[s * SROW + t] * sm.s1[s * SROW + t];
      float part = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) part += sm.de2[ww][s] + sm.de4[ww][s];
      detag[t0 + s] = part - acc;
    }
    __syncthreads();  // #5

    // ---- A5: dA_K, dH_K, partials of dQ and dK ----
    float4v dhk[2];
    {
      // dA_K += W2^T dY
      float4v wy[2] = {zero4v(), zero4v()};
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bf16x4 th[2][2], tl[2][2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) transpose2(w2_tile(2 * m + hf, 0), w2_tile(2 * m + hf, 1), ident, th[hf], tl[hf]);
        // dY [i = 32m + 16hf + 4g + r][s = li]
        const Op8 yo = split8(ld4(&sm.dy[li * PROW + 32 * m + 4 * g]), ld4(&sm.dy[li * PROW + 32 * m + 16 + 4 * g]));
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) wy[jt] = mfma3(Op8{cat(th[0][jt], th[1][jt]), cat(tl[0][jt], tl[1][jt])}, yo, wy[jt]);
      }
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) dhk[jt][r] = fmaf(dak[jt][r] + wy[jt][r], gk1[jt][r], dhk1[jt][r]);
      // dQ partial = W1^T dH_Q (to pa), dK partial += W1^T dH_K (pb)   ([c][t] tiles)
      const Op8 dqo = split8(dhq[0], dhq[1]), dko = split8(dhk[0], dhk[1]);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bf16x4 w1jh[2][2], w1jl[2][2];  // [jt][q] = W1[32w + 16jt + 4g + r][16(2m + q) + li]
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
          transpose2(w1_tile(jt, 2 * m), w1_tile(jt, 2 * m + 1), ident, w1jh[jt], w1jl[jt]);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int c4 = 2 * m + q;
          const Op8 W{cat(w1jh[0][q], w1jh[1][q]), cat(w1jl[0][q], w1jl[1][q])};
          const float4v pq = mfma3(W, dqo, zero4v());  // [c = 16c4 + 4g + r][t = li]
          float* kp = &sm.pb[w][li * PROW + 16 * c4 + 4 * g];
          const float4v pk = mfma3(W, dko, ld4(kp));
          st4(&sm.pa[w][li * PROW + 16 * c4 + 4 * g], pq);
          st4(kp, pk);
        }
      }
    }
    __syncthreads();  // #6


    // ---- R-C: dQ = (the partials) + K M1, dK = (the partials) + Q M1^T; waves 0-3 dQ, 4-7 dK ----
    {
      const bool isq = w < 4;
      const int c4 = w & 3;  // columns c = 16c4 .. 16c4 + 15
      // M1[s][t] = -eta_s GQ[s][t] (s <= t): dQ takes it with rows s (lane: s = 4g + r, t = li),
      // dK with rows t (lane: s = li, t = 4g + r)
      float4v m1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = isq ? 4 * g + r : li, t = isq ? li : 4 * g + r;
        m1[r] = (s <= t) ? -sm.eta[s] * sm.gq[s * SROW + t] : 0.f;
      }
      bf16x4 mh, ml;
      split4(m1, mh, ml);
      // K [s = 4g + r][c = 16c4 + li] or Q [t = 4g + r][c]: bf16, exact
      const bf16x4 x4 = *reinterpret_cast<const bf16x4*>(&(isq ? sm.kt : sm.qt)[(16 * c4 + li) * KTROW + 4 * g]);
      float4v acc = mfma32(cat(x4, x4), cat(mh, ml), zero4v());  // [c = 16c4 + 4g + r][t = li]
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) acc += ld4(&(isq ? sm.pa[ww] : sm.pb[ww])[li * PROW + 16 * c4 + 4 * g]);
      *reinterpret_cast<float4v*>((isq ? dQg : dKg) + static_cast<size_t>(t0 + li) * D + 16 * c4 + 4 * g) = acc;
    }

    // ---- A6: the rest of the mini-batch-start adjoints: A1 += dH_K K^T, A2 += dY A_K^T ----
    {
      float4v dhkt[2];
      jt2tj(dhk, dhkt);
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        bf16x4 kh, kl;
        split4(dhkt[jt], kh, kl);
        const bf16x8 kb = cat(kh, kl);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const bf16x4 kt4 = *reinterpret_cast<const bf16x4*>(&sm.kt[(16 * c4 + li) * KTROW + 4 * g]);
          a1[jt][c4] = mfma32(cat(kt4, kt4), kb, a1[jt][c4]);
        }
      }
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        float4v yt;  // dY [t = 4g + r][i = 16it + li]
#pragma unroll
        for (int r = 0; r < 4; ++r) yt[r] = sm.dy[(4 * g + r) * PROW + 16 * it + li];
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) a2[it][jt] = mfma3_16(akt[jt], yt, a2[it][jt]);
      }
    }
  }

  const int64_t cs = static_cast<int64_t>(chain) * ST;
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) st4(a.dW1 + cs + (32 * w + 16 * jt + li) * D + 16 * c4 + 4 * g, a1[jt][c4]);
#pragma unroll
    for (int it = 0; it < 4; ++it) st4(a.dW2 + cs + (16 * it + li) * DH + 32 * w + 16 * jt + 4 * g, a2[it][jt]);
  }
}

}  // namespace

bool mlp_bwd_mfma_supported(int d, int dh, int b, int in_dtype, int T) {
  return d == D && dh == DH && b == BT && in_dtype == 1 && T % BT == 0;
}

hipError_t launch_mlp_bwd_mfma(const MlpBwdArgs& a, hipStream_t s) {
  const size_t smem = sizeof(Smem);
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ttt_mlp_bwd_d64h256b16),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ttt_mlp_bwd_d64h256b16, dim3(a.B * a.H), dim3(NT), smem, s, a);
  return hipGetLastError();
}

}  // namespace ttt
