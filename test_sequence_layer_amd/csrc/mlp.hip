// TTT-MLP dual-form forward on CDNA4 matrix cores: d = 64, dh = 256, b = 16, bf16 Q/K/V.
//
// Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
// (aharts.cn / itmax.cn), part 03 §9 (TTT-MLP: two layers, hidden width 4x,
// GELU), with the update/output rules of 03 §1, §5, §6 and the dual form of
// 03 §7 applied layer by layer.
//
// The model is f(x) = W2 GELU(W1 x), W1: dh x d, W2: d x dh.  Per mini-batch of
// 16 tokens (columns; W1, W2 = the state before the mini-batch, eta_s per token):
//   H_K = W1 K,  A_K = GELU(H_K),  E = 2 (W2 A_K - V)                  (d x b)
//   D   = (W2^T E) * GELU'(H_K)                                        (dh x b)
//   H_Q = W1 Q - D L1,      L1[s][t] = eta_s (k_s . q_t) [s <= t]
//   A_Q = GELU(H_Q),   Z = W2 A_Q - E L2,  L2[s][t] = eta_s (a_K,s . a_Q,t) [s <= t]
//   W1 -= D diag(eta) K^T,  W2 -= E diag(eta) A_K^T
// (the gradient of |W2 GELU(W1 k) - v|^2 is E A^T for W2 and (W2^T E * GELU') k^T
// for W1; the output z_t uses the state after token t's own step).
//
// Work decomposition.  One 512-thread workgroup (8 waves) per (sequence, head),
// one workgroup per CU (the 128 KB state per chain lives in registers).  Wave w
// owns hidden units J_w = [32w, 32w+32): rows J_w of W1 and columns J_w of W2.
// Products over the hidden dimension (W2 A_K, W2 A_Q, A_K^T A_Q) are summed
// across the 8 waves through per-wave partial buffers in LDS (a fixed order, so
// results are deterministic).
//
// MFMA layouts (v_mfma_f32_16x16x32_bf16 only).  An accumulator tile holds
// X[m][n] at lane (n = l%16, m = 4(l/16) + r); an operand holds its free index at
// l%16 and its contraction index in the k-slots of lane group l/16.  A tile can
// therefore be contracted only over the index it keeps at 4(l/16)+r.  W2 is
// contracted over hidden units (W2 A) and over outputs (W2^T E).  The state
// keeps the first orientation; the second is made each mini-batch by
// multiplying the split W2 operand by an identity operand on the matrix cores
// (D = X I moves X's k-slot index to l%16; bf16 x 1 is exact).  Activations
// needed in the other orientation (A_K for the W2 update, GELU'(H_K) for the
// backward product) go through per-wave LDS tiles; A_K is stored already split
// and read back with transposing loads.  Every run of matrix-core instructions
// is issued at raised wave priority (wave_prio.h): -3.6% at the TTT-MLP shape,
// -9.3% with the layer norm.  As in the TTT-Linear kernel, fp32 operands enter as bf16
// hi + lo pairs (3 passes when both are fp32; 16-token contractions put two
// passes into the 8 k-slots of one instruction).
#include "gelu.h"
#include "args_mlp.h"
#include "mfma_common.h"
#include "wave_prio.h"

namespace ttt {
namespace {

using namespace mfma;

constexpr int D = 64;       // model dim
constexpr int DH = 256;     // hidden width
constexpr int BT = 16;      // mini-batch
constexpr int NW = 8;       // waves per workgroup
constexpr int JW = DH / NW; // hidden units per wave (32)
constexpr int kThreads = NW * 64;
constexpr int ROW = 72;     // padded bf16 row of a token tile (row reads conflict-free)
constexpr int EROW = 80;    // padded bf16 row of the -eta E tiles (column reads conflict-free)
constexpr int AROW = 48;    // padded bf16 row of the per-wave A_K tiles [t][j] (column reads conflict-free)
constexpr int KTROW = 20;   // padded bf16 row of the transposed K tile
constexpr int TROW = 20;    // padded fp32 row of the per-wave transpose buffer [j][t]
constexpr int PROW = 68;    // padded fp32 row of [t][i] buffers
constexpr int SROW = 20;    // padded fp32 row of [s][t] buffers

struct __align__(16) Slot {
  uint16_t q[BT * ROW];
  uint16_t k[BT * ROW];
  uint16_t v[BT * ROW];
  uint16_t kt[D * KTROW];
  float eta[BT];
};

// Every fp32 operand that several waves (or several products) use is split into
// bf16 hi + lo once, where it is made, and kept split: E and -eta E by the
// threads that form them, A_K by the wave that owns its hidden units.
struct __align__(16) Smem {
  Slot slots[2];
  uint16_t akh[NW][BT * AROW];  // A_K of each wave, bf16 hi, [t][j]
  uint16_t akl[NW][BT * AROW];  //   and lo
  float gk_t[NW][JW * TROW];    // GELU'(H_K) of each wave, [j][t]
  float part[NW][BT * PROW];    // per-wave partial of W2 A (over the wave's hidden units), [t][i]
  float s2p[NW][BT * SROW];     // per-wave partial of A_K^T A_Q, [s][t]
  uint16_t eh[BT * ROW];        // E, bf16 hi, [t][i]
  uint16_t el[BT * ROW];        //   and lo
  uint16_t enh[BT * EROW];      // -eta_t E, bf16 hi, [t][i]
  uint16_t enl[BT * EROW];      //   and lo
  float zr[BT * PROW];          // W2 A_Q summed over waves, [t][i]
  float s2[BT * SROW];          // A_K^T A_Q summed over waves, [s][t]
};

// a pair of 4-wide tiles split into 8-slot hi and lo operands
struct Op8 {
  bf16x8 hi, lo;
};
__device__ __forceinline__ Op8 split8(float4v a, float4v b) {
  bf16x4 ah, al, bh, bl;
  split4(a, ah, al);
  split4(b, bh, bl);
  return Op8{cat(ah, bh), cat(al, bl)};
}

// C += A B with both operands split: hi*hi + hi*lo + lo*hi
__device__ __forceinline__ float4v mfma3(const Op8& a, const Op8& b, float4v c) {
  c = mfma32(a.hi, b.hi, c);
  c = mfma32(a.hi, b.lo, c);
  c = mfma32(a.lo, b.hi, c);
  return c;
}

// 16-slot contraction of two split operands (4 values each): the 3 passes
// hi*hi + hi*lo + lo*hi in 2 instructions
__device__ __forceinline__ float4v mfma3_16(bf16x4 ah, bf16x4 al, bf16x4 bh, bf16x4 bl, float4v c) {
  const bf16x4 z = {};
  c = mfma32(cat(ah, ah), cat(bh, bl), c);
  c = mfma32(cat(al, z), cat(bh, z), c);
  return c;
}

// Sum over the 32 lanes of a half wave (lanes 0-31 or 32-63): DPP inside each
// 16-lane row, then the neighbouring row.
__device__ __forceinline__ float sum32(float x) {
  return sum_row_pairs(sum16(x));
}

__device__ __forceinline__ float4v ld4(const float* p) { return *reinterpret_cast<const float4v*>(p); }
__device__ __forceinline__ void st4(float* p, float4v x) { *reinterpret_cast<float4v*>(p) = x; }
// checkpoints are read back only after the whole forward: keep them out of the caches
__device__ __forceinline__ void st4nt(float* p, float4v x) { __builtin_nontemporal_store(x, reinterpret_cast<float4v*>(p)); }

// LN: f(x) = x + LN(W2 GELU(W1 x)) (layer norm over the d outputs, per-head
// gamma and beta, and a residual).  The loss gradient with respect to the
// pre-norm output, Delta = J_LN^T (2 (f(k) - v) * gamma), takes the place of
// E = 2 (W2 A_K - V); everything downstream is unchanged, and the output is
// Z = Q + LN(W2 A_Q - Delta (diag(eta) triu(A_K^T A_Q))).
//
// CKPT: the first pass of the backward.  The state at the start of every
// mini-batch goes to a.ckpt (W1 then W2, row-major fp32, per chain and
// mini-batch) and the output side (H_Q, A_Q, Z, the final state) is skipped.
template <bool ETA_TOKEN, bool LN, bool CKPT>
__global__ __launch_bounds__(kThreads) void ttt_mlp_fwd_d64h256b16(MlpArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);

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
  const u32x2* Qg = reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.Q) + tok0 * D);
  const u32x2* Kg = reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.K) + tok0 * D);
  const uint32_t* Vg = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.V) + tok0 * D);
  float* Zg = static_cast<float*>(a.Z) + tok0 * D;
  const float* eg = a.eta + bi * a.esb + h * a.esh;

  // staging: 8 B of Q (tid < 256) or K (tid >= 256), 4 B of V, eta of token tid & 15
  const int within = tid & 255;
  const u32x2* srcA = (tid < 256 ? Qg : Kg) + within;
  const uint32_t* srcB = Vg + tid;
  const int srow = within >> 4, scol = (within & 15) * 4;
  const int vrow = tid >> 5, vcol = (tid & 31) * 2;
  const float* srcE = eg + static_cast<int64_t>(tid & 15) * a.est;

  // Mini-batches of look-ahead in the load ring.  Measured at the TTT-MLP shape:
  // the plain scalar-eta form runs 1.055 / 1.013 / 1.010 / 1.180 ms with 2 / 3 /
  // 4 / 6 (6 spills inside the loop); the layer-norm form is fastest with 2
  // (1.144 ms against 1.148 with 3 or 4), and with 4 the per-token-eta forms
  // spill 81-121 registers, so they keep 2.
  constexpr int PF = (ETA_TOKEN || LN) ? 2 : 4;
  u32x2 ra[PF];
  uint32_t rb[PF];
  float re[PF];
  auto load_step = [&](int n, u32x2& xa, uint32_t& xb, float& xe) {
    xa = __builtin_nontemporal_load(srcA + static_cast<size_t>(n) * (BT * D / 4));
    xb = __builtin_nontemporal_load(srcB + static_cast<size_t>(n) * (BT * D / 2));
    xe = ETA_TOKEN ? srcE[static_cast<int64_t>(n) * BT * a.est] : 0.f;
  };
  auto stage = [&](int slot, const u32x2& xa, uint32_t xb, float xe) {
    Slot& S = sm.slots[slot];
    *reinterpret_cast<uint32_t*>(&S.v[vrow * ROW + vcol]) = xb;
    if (tid < 256) {
      *reinterpret_cast<u32x2*>(&S.q[srow * ROW + scol]) = xa;
    } else {
      *reinterpret_cast<u32x2*>(&S.k[srow * ROW + scol]) = xa;
      S.kt[(scol + 0) * KTROW + srow] = static_cast<uint16_t>(xa.x & 0xffffu);
      S.kt[(scol + 1) * KTROW + srow] = static_cast<uint16_t>(xa.x >> 16);
      S.kt[(scol + 2) * KTROW + srow] = static_cast<uint16_t>(xa.y & 0xffffu);
      S.kt[(scol + 3) * KTROW + srow] = static_cast<uint16_t>(xa.y >> 16);
    }
    if (ETA_TOKEN && tid < BT) S.eta[tid] = xe;
  };

  float eta_c = 0.f;
  if (!ETA_TOKEN && nb > 0) eta_c = eg[0];

  // layer norm scale and shift of outputs i, i + 1 of token tid / 32: the
  // thread's role in both layer norms (the phase-2 sums and the output)
  float lg[2] = {0.f, 0.f}, lb[2] = {0.f, 0.f};
  if constexpr (LN) {
    const float* gm = a.gamma + static_cast<int64_t>(h) * D;
    const float* bt = a.beta + static_cast<int64_t>(h) * D;
    const int i2 = (2 * tid) & (D - 1);
    lg[0] = gm[i2]; lg[1] = gm[i2 + 1];
    lb[0] = bt[i2]; lb[1] = bt[i2 + 1];
  }

  // ---- resident state (this wave's hidden units J_w) ----
  // w1[jt][c4]  : W1[j = 32w + 16jt + li][c = 16 c4 + 4g + r]
  // w2a[it][jt] : W2[i = 16it + li][j = 32w + 16jt + 4g + r]   (contracted over j)
  float4v w1[2][4], w2a[4][2];
  {
    const float* W1 = a.W1 + bi * a.w_bstride + static_cast<int64_t>(h) * DH * D;
    const float* W2 = a.W2 + bi * a.w_bstride + static_cast<int64_t>(h) * D * DH;
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) w1[jt][c4] = ld4(W1 + (32 * w + 16 * jt + li) * D + 16 * c4 + 4 * g);
#pragma unroll
      for (int it = 0; it < 4; ++it) w2a[it][jt] = ld4(W2 + (16 * it + li) * DH + 32 * w + 16 * jt + 4 * g);
    }
  }
  // Identity operands: X (as A, k-slots = the wave's 32 hidden units) times
  // ident[jt] returns X's columns 16jt..16jt+15 in accumulator layout, i.e. with
  // the hidden unit at l%16: the transpose of the lane roles.  bf16 x 1 products
  // are exact, so a split operand transposes exactly.
  bf16x8 ident[2];
#pragma unroll
  for (int jt = 0; jt < 2; ++jt)
#pragma unroll
    for (int sl = 0; sl < 8; ++sl)
      ident[jt][sl] = static_cast<__bf16>((sl / 4 == jt && 4 * g + (sl & 3) == li) ? 1.f : 0.f);
  // drain the state loads before the prefetch ring (see the TTT-Linear kernel)
  __builtin_amdgcn_s_waitcnt(0x0F70);

  if (nb > 0) {
#pragma unroll
    for (int j = 0; j < PF; ++j) load_step(min(j, nb - 1), ra[j], rb[j], re[j]);
    stage(0, ra[0], rb[0], re[0]);
  }
  __syncthreads();

  uint16_t* akh = sm.akh[w];
  uint16_t* akl = sm.akl[w];
  float* gkt = sm.gk_t[w];
  float* part = sm.part[w];

  auto step = [&](const int n, u32x2& xa, uint32_t& xb, float& xe, const u32x2& ya, const uint32_t yb,
                  const float ye) {
    stage((n + 1) & 1, ya, yb, ye);
    load_step(min(n + PF, nb - 1), xa, xb, xe);
    const Slot& S = sm.slots[n & 1];
    if constexpr (CKPT) {
      float* ck = a.ckpt + (static_cast<int64_t>(chain) * nb + n) * (2 * DH * D);
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) st4nt(ck + (32 * w + 16 * jt + li) * D + 16 * c4 + 4 * g, w1[jt][c4]);
#pragma unroll
        for (int it = 0; it < 4; ++it) st4nt(ck + DH * D + (16 * it + li) * DH + 32 * w + 16 * jt + 4 * g, w2a[it][jt]);
      }
    }

    // token-row operands of K and Q: row li, columns {16 c4 + 4g .. +3}
    bf16x4 kx[4], qx[4];
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      kx[c4] = *reinterpret_cast<const bf16x4*>(&S.k[li * ROW + 16 * c4 + 4 * g]);
      qx[c4] = *reinterpret_cast<const bf16x4*>(&S.q[li * ROW + 16 * c4 + 4 * g]);
    }
    float et[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) et[r] = ETA_TOKEN ? S.eta[4 * g + r] : eta_c;

    // ---- phase 1: H_K, W1 Q (layout [j][t]), S1 = K Q^T, GELU ----
    float4v hk[2], hq[2];
    float4v s1 = {0.f, 0.f, 0.f, 0.f};
    prio_mfma();
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      hk[jt] = float4v{0.f, 0.f, 0.f, 0.f};
      hq[jt] = hk[jt];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const Op8 wj = split8(w1[jt][2 * m], w1[jt][2 * m + 1]);
        const bf16x8 kb = cat(kx[2 * m], kx[2 * m + 1]);
        const bf16x8 qb = cat(qx[2 * m], qx[2 * m + 1]);
        hk[jt] = mfma32(wj.hi, kb, hk[jt]);
        hk[jt] = mfma32(wj.lo, kb, hk[jt]);
        if constexpr (!CKPT) {
          hq[jt] = mfma32(wj.hi, qb, hq[jt]);
          hq[jt] = mfma32(wj.lo, qb, hq[jt]);
        }
      }
    }
    if constexpr (!CKPT) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
        s1 = mfma32(cat(kx[2 * m], kx[2 * m + 1]), cat(qx[2 * m], qx[2 * m + 1]), s1);
    }
    prio_valu();

    float4v ak[2];
    {
      float xv[8], gv[8], gpv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) xv[k] = hk[k >> 2][k & 3];
      gelu8<true>(xv, gv, gpv);
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ak[jt][r] = gv[4 * jt + r];
          gkt[(16 * jt + 4 * g + r) * TROW + li] = gpv[4 * jt + r];  // transposed: [j = 16jt + 4g + r][t = li]
        }
      }
    }
    const Op8 akop = split8(ak[0], ak[1]);  // A_K with j in the k-slots, t at l%16
    {
      // the same split values, row t = li of the [t][j] tiles (read back transposed for the W2 update)
      const u32x4 hv = __builtin_bit_cast(u32x4, akop.hi), lv = __builtin_bit_cast(u32x4, akop.lo);
      *reinterpret_cast<u32x2*>(&akh[li * AROW + 4 * g]) = u32x2{hv.x, hv.y};
      *reinterpret_cast<u32x2*>(&akh[li * AROW + 16 + 4 * g]) = u32x2{hv.z, hv.w};
      *reinterpret_cast<u32x2*>(&akl[li * AROW + 4 * g]) = u32x2{lv.x, lv.y};
      *reinterpret_cast<u32x2*>(&akl[li * AROW + 16 + 4 * g]) = u32x2{lv.z, lv.w};
    }

    // Y partial[i][t] = sum_{j in J_w} W2[i][j] A_K[j][t]  -> part[t][i]
    prio_mfma();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const float4v y = mfma3(split8(w2a[it][0], w2a[it][1]), akop, float4v{0.f, 0.f, 0.f, 0.f});
      // lane holds Y[i = 16it + 4g + r][t = li]
      st4(&part[li * PROW + 16 * it + 4 * g], y);
    }
    prio_valu();
    __syncthreads();  // #1: partials written

    // ---- phase 2: E[t][i] = 2 (sum_w part_w[t][i] - V[t][i]), stored split, and -eta_t E ----
    {
      const int e0 = 2 * tid;
      const int t = e0 >> 6, i = e0 & 63;
      float y0 = 0.f, y1 = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        y0 += sm.part[ww][t * PROW + i];
        y1 += sm.part[ww][t * PROW + i + 1];
      }
      const uint32_t vv = *reinterpret_cast<const uint32_t*>(&S.v[t * ROW + i]);
      float x0, x1;
      if constexpr (LN) {
        // 32 consecutive threads (half a wave) hold token t's 64 outputs
        const float mu = sum32(y0 + y1) * (1.f / D);
        const float d0 = y0 - mu, d1 = y1 - mu;
        const float rs = rsqrtf(sum32(d0 * d0 + d1 * d1) * (1.f / D) + a.eps);
        const float h0 = d0 * rs, h1 = d1 * rs;
        const uint32_t kk = *reinterpret_cast<const uint32_t*>(&S.k[t * ROW + i]);
        // dl/df = 2 (k + gamma yhat + beta - v), times gamma: the gradient at yhat
        const float g0 = 2.f * (__uint_as_float(kk << 16) + lg[0] * h0 + lb[0] - __uint_as_float(vv << 16)) * lg[0];
        const float g1 =
            2.f * (__uint_as_float(kk & 0xffff0000u) + lg[1] * h1 + lb[1] - __uint_as_float(vv & 0xffff0000u)) * lg[1];
        const float mg = sum32(g0 + g1) * (1.f / D);
        const float mgy = sum32(g0 * h0 + g1 * h1) * (1.f / D);
        x0 = (g0 - mg - h0 * mgy) * rs;
        x1 = (g1 - mg - h1 * mgy) * rs;
      } else {
        x0 = 2.f * (y0 - __uint_as_float(vv << 16));
        x1 = 2.f * (y1 - __uint_as_float(vv & 0xffff0000u));
      }
      const float ne = -(ETA_TOKEN ? S.eta[t] : eta_c);
      uint32_t hi, lo;
      split2(x0, x1, hi, lo);
      *reinterpret_cast<uint32_t*>(&sm.eh[t * ROW + i]) = hi;
      *reinterpret_cast<uint32_t*>(&sm.el[t * ROW + i]) = lo;
      split2(ne * x0, ne * x1, hi, lo);
      *reinterpret_cast<uint32_t*>(&sm.enh[t * EROW + i]) = hi;
      *reinterpret_cast<uint32_t*>(&sm.enl[t * EROW + i]) = lo;
    }
    __syncthreads();  // #2: E ready, partial buffer free

    // ---- phase 3: backward through W2 and GELU, H_Q, A_Q, partials, updates ----
    // E^T operand: row t = li, i in the k-slots {32m + 16 h + 4g .. +3}
    Op8 eq[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint16_t* ph = &sm.eh[li * ROW + 32 * m + 4 * g];
      const uint16_t* pl = &sm.el[li * ROW + 32 * m + 4 * g];
      eq[m] = Op8{cat(*reinterpret_cast<const bf16x4*>(ph), *reinterpret_cast<const bf16x4*>(ph + 16)),
                  cat(*reinterpret_cast<const bf16x4*>(pl), *reinterpret_cast<const bf16x4*>(pl + 16))};
    }
    // W2 with the hidden unit at l%16 (contraction over i): the split W2 operands
    // times the identity give W2[i = 16it + 4g + r][j = 16jt + li], exact bf16 values.
    Op8 w2s[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) w2s[it] = split8(w2a[it][0], w2a[it][1]);
    // G[j][s] = -eta_s GELU'(H_K)[j][s] sum_i E[i][s] W2[i][j]   (s = 4g + r, j = 16jt + li),
    // i.e. -eta_s D[j][s]; split once, it serves the H_Q correction and the W1 gradient
    bf16x4 gdh[2], gdl[2];
    prio_mfma();
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const float4v z4 = {0.f, 0.f, 0.f, 0.f};
        const bf16x4 h0 = __builtin_convertvector(mfma32(w2s[2 * m].hi, ident[jt], z4), bf16x4);
        const bf16x4 h1 = __builtin_convertvector(mfma32(w2s[2 * m + 1].hi, ident[jt], z4), bf16x4);
        const bf16x4 l0 = __builtin_convertvector(mfma32(w2s[2 * m].lo, ident[jt], z4), bf16x4);
        const bf16x4 l1v = __builtin_convertvector(mfma32(w2s[2 * m + 1].lo, ident[jt], z4), bf16x4);
        acc = mfma3(eq[m], Op8{cat(h0, h1), cat(l0, l1v)}, acc);
      }
      const float4v gp = ld4(&gkt[(16 * jt + li) * TROW + 4 * g]);
      float4v gd;
#pragma unroll
      for (int r = 0; r < 4; ++r) gd[r] = -et[r] * (acc[r] * gp[r]);
      split4(gd, gdh[jt], gdl[jt]);
    }
    prio_valu();
    // H_Q[j][t] += sum_s G[j][s] S1[s][t] [s <= t]   (= - D diag(eta) triu(K^T Q))
    if constexpr (!CKPT) {
    bf16x4 s1h, s1l;
    {
      float4v s1m;
#pragma unroll
      for (int r = 0; r < 4; ++r) s1m[r] = (4 * g + r <= li) ? s1[r] : 0.f;
      split4(s1m, s1h, s1l);
    }
    float4v aq[2];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) hq[jt] = mfma3_16(gdh[jt], gdl[jt], s1h, s1l, hq[jt]);
    {
      float xv[8], gv[8], unused[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) xv[k] = hq[k >> 2][k & 3];
      gelu8<false>(xv, gv, unused);
#pragma unroll
      for (int k = 0; k < 8; ++k) aq[k >> 2][k & 3] = gv[k];
    }
    const Op8 aqop = split8(aq[0], aq[1]);
    // S2 partial[s][t] = sum_{j in J_w} A_K[j][s] A_Q[j][t]   (s = 4g + r, t = li)
    prio_mfma();
    {
      const float4v s2 = mfma3(akop, aqop, float4v{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.s2p[w][(4 * g + r) * SROW + li] = s2[r];
    }
    // W2 A_Q partial -> part[t][i]
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const float4v y = mfma3(w2s[it], aqop, float4v{0.f, 0.f, 0.f, 0.f});
      st4(&part[li * PROW + 16 * it + 4 * g], y);
    }
    prio_valu();
    }  // !CKPT

    // ---- state updates (gradients at the mini-batch-start state) ----
    // W1^T[c][j] += sum_s K[s][c] G[j][s]
    prio_mfma();
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      const bf16x8 gb = cat(gdh[jt], gdl[jt]);
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const bf16x4 kt = *reinterpret_cast<const bf16x4*>(&S.kt[(16 * c4 + li) * KTROW + 4 * g]);
        w1[jt][c4] = mfma32(cat(kt, kt), gb, w1[jt][c4]);
      }
    }
    // W2[i][j] += sum_s A_K[j][s] (-eta_s E[i][s])   (tile: j = 16jt + 4g + r, i = 16it + li),
    // both operands read back split: A_K[j = 16jt + li][s = 4g + r], -eta_s E[i = 16it + li][s = 4g + r]
    bf16x4 gah[2], gal[2];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      gah[jt] = read_cols<AROW>(akh, 0, 16 * jt, li, g);
      gal[jt] = read_cols<AROW>(akl, 0, 16 * jt, li, g);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const bf16x4 eh = read_cols<EROW>(sm.enh, 0, 16 * it, li, g);
      const bf16x4 el = read_cols<EROW>(sm.enl, 0, 16 * it, li, g);
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) w2a[it][jt] = mfma3_16(gah[jt], gal[jt], eh, el, w2a[it][jt]);
    }
    prio_valu();
    __syncthreads();  // #3: S2 and W2 A_Q partials written
    if constexpr (CKPT) return;  // (the next mini-batch may restage this slot only after #3)

    // ---- phase 4: sum the partials ----
    if (tid < BT * BT) {
      const int s = tid >> 4, t = tid & 15;
      float acc = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) acc += sm.s2p[ww][s * SROW + t];
      sm.s2[s * SROW + t] = acc;
    }
    {
      const int e0 = 2 * tid;
      const int t = e0 >> 6, i = e0 & 63;
      float y0 = 0.f, y1 = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        y0 += sm.part[ww][t * PROW + i];
        y1 += sm.part[ww][t * PROW + i + 1];
      }
      sm.zr[t * PROW + i] = y0;
      sm.zr[t * PROW + i + 1] = y1;
    }
    __syncthreads();  // #4

    // ---- phase 5: Z[t][i] = (W2 A_Q)[i][t] + sum_s (-eta_s E[i][s]) S2[s][t] [s <= t], waves 0..3 ----
    // (with the layer norm: Z = Q + LN of that, over the 64 outputs of each token)
    if (w < 4) {
      const int it = w;
      bf16x4 s2h, s2l;
      {
        float4v s2m;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = 4 * g + r;
          s2m[r] = (s <= li) ? sm.s2[s * SROW + li] : 0.f;
        }
        split4(s2m, s2h, s2l);
      }
      // A: -eta_s E[i = 16it + li][s = 4g + r] (valid until the next mini-batch's barrier #1)
      const bf16x4 eh = read_cols<EROW>(sm.enh, 0, 16 * it, li, g);
      const bf16x4 el = read_cols<EROW>(sm.enl, 0, 16 * it, li, g);
      // C: (W2 A_Q)[i = 16it + 4g + r][t = li]
      float4v z = ld4(&sm.zr[li * PROW + 16 * it + 4 * g]);
      z = mfma3_16(eh, el, s2h, s2l, z);
      if constexpr (LN) {
        st4(&sm.zr[li * PROW + 16 * it + 4 * g], z);  // back in place: the pre-norm rows for the output LN
      } else {
        float* zp = Zg + (static_cast<size_t>(n) * BT + li) * D + 16 * w + 4 * g;
        *reinterpret_cast<float4v*>(zp) = z;  // 64-byte pieces of a row per wave, merged in the L2
      }
    }
    if constexpr (LN) {
      // The output layer norm in the phase-2 role: every thread takes token
      // tid / 32, outputs i, i + 1, so the 64 outputs of a token are in 32
      // consecutive threads (half-wave sums) and the 32 threads write its whole
      // Z row.  Q for the residual is read before the barrier, after which
      // other waves may restage this slot.
      const int t = tid >> 5, i = (2 * tid) & (D - 1);
      const uint32_t qq = *reinterpret_cast<const uint32_t*>(&S.q[t * ROW + i]);
      __syncthreads();  // #5: the pre-norm rows of all output waves
      const float2 y = *reinterpret_cast<const float2*>(&sm.zr[t * PROW + i]);
      const float mu = sum32(y.x + y.y) * (1.f / D);
      const float d0 = y.x - mu, d1 = y.y - mu;
      const float rs = rsqrtf(sum32(d0 * d0 + d1 * d1) * (1.f / D) + a.eps);
      const float q0 = __uint_as_float(qq << 16), q1 = __uint_as_float(qq & 0xffff0000u);
      float* zp = Zg + (static_cast<size_t>(n) * BT + t) * D + i;
      *reinterpret_cast<float2*>(zp) = make_float2(q0 + lg[0] * (d0 * rs) + lb[0], q1 + lg[1] * (d1 * rs) + lb[1]);
    }
  };

  const int nfull = nb / PF * PF;
  for (int n0 = 0; n0 < nfull; n0 += PF) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int jn = (j + 1) % PF;
      step(n0 + j, ra[j], rb[j], re[j], ra[jn], rb[jn], re[jn]);
    }
  }
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    const int jn = (j + 1) % PF;
    if (nfull + j < nb) step(nfull + j, ra[j], rb[j], re[j], ra[jn], rb[jn], re[jn]);
  }

  // ---- final state ----
  if constexpr (CKPT) return;
  float* W1f = a.W1f + static_cast<int64_t>(chain) * DH * D;
  float* W2f = a.W2f + static_cast<int64_t>(chain) * D * DH;
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) st4(W1f + (32 * w + 16 * jt + li) * D + 16 * c4 + 4 * g, w1[jt][c4]);
#pragma unroll
    for (int it = 0; it < 4; ++it) st4(W2f + (16 * it + li) * DH + 32 * w + 16 * jt + 4 * g, w2a[it][jt]);
  }
}

template <bool TOK, bool LN, bool CKPT = false>
hipError_t launch_tok(const MlpArgs& a, hipStream_t s) {
  const size_t smem = sizeof(Smem);
  // the dynamic LDS limit is raised on every launch (a host-side attribute, no
  // stream work), so the library keeps no state between calls
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ttt_mlp_fwd_d64h256b16<TOK, LN, CKPT>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((ttt_mlp_fwd_d64h256b16<TOK, LN, CKPT>), dim3(a.B * a.H), dim3(kThreads), smem, s, a);
  return hipGetLastError();
}

}  // namespace

bool mlp_supported(const MlpArgs& a) {
  return a.d == D && a.dh == DH && a.b == BT && a.in_dtype == 1 && a.out_dtype == 0;
}

const char* mlp_name(const MlpArgs& a) {
  return a.gamma ? "ttt_mlp_fwd_d64h256b16 (layer norm)" : "ttt_mlp_fwd_d64h256b16";
}

hipError_t launch_mlp(const MlpArgs& a, hipStream_t s) {
  if (a.gamma) return a.est != 0 ? launch_tok<true, true>(a, s) : launch_tok<false, true>(a, s);
  return a.est != 0 ? launch_tok<true, false>(a, s) : launch_tok<false, false>(a, s);
}

hipError_t launch_mlp_ckpt(const MlpArgs& a, hipStream_t s) {
  return a.est != 0 ? launch_tok<true, false, true>(a, s) : launch_tok<false, false, true>(a, s);
}

}  // namespace ttt
