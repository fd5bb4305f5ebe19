// TTT-Linear backward (dual form) on CDNA4 matrix cores: d = 64, b = 16, bf16 Q/K.
//
// Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
// (aharts.cn / itmax.cn), part 03 §4 (the TTT layer is trained end to end like
// any other layer, so it needs a backward), §6 (mini-batch GD), §7 (the dual
// form serves the forward and the backward alike), §9 (TTT-Linear, f(x) = W x).
//
// The forward of one mini-batch (tokens s, t of the mini-batch, columns of
// K, Q, V, Z are tokens, W the state at the mini-batch start, eta_s per token):
//   E  = W K - V,   S[s][t] = k_s . q_t,   M[s][t] = eta_s S[s][t] [s <= t]
//   Z  = W Q - 2 E M,        W' = W - 2 E diag(eta) K^T
// Given the adjoints dZ and A = dL/dW', its backward is
//   P  = A K                                   (d x b)
//   dE = -2 dZ M^T - 2 P diag(eta),   dV = -dE
//   Y[s][t] = e_s . dz_t,   Y'[s][t] = -2 eta_s Y[s][t] [s <= t]
//   dQ = W^T dZ + K Y'
//   dK = W^T dE - 2 A^T E diag(eta) + Q Y'^T
//   deta_s = -2 sum_{t >= s} S[s][t] Y[s][t] - 2 e_s . p_s
//   dL/dW = A + dZ Q^T + dE K^T                 (the adjoint carried backward)
// The mini-batch-start state is rebuilt backward from the final state with the
// saved E: W = W' + 2 E diag(eta) K^T, so nothing but E (one fp32 value per
// token and output) is kept from the forward.
//
// Work decomposition: one workgroup (4 waves) per (sequence, head) walks the
// mini-batches from last to first.  Two products contract over the state's
// columns (P = A K) and four over its rows (W^T dE, W^T dZ, A^T E and the
// updates), so the state is held in two MFMA layouts:
//   F1 (row-owned)    wave w holds rows i = 16w..16w+15, all columns, as
//                     accumulator tiles a1[a][r] = A[16w + li][16a + 4g + r]
//                     -- the B operand of a contraction over columns;
//   F2 (column-owned) wave w holds columns c = 16w..16w+15, all rows:
//                     w2[b][r] = W[16b + 4g + r][16w + li],
//                     a2[b][r] = A[16b + 4g + r][16w + li]
//                     -- the B operand of a contraction over rows.
// A is kept in both (its two copies are updated with the same terms); W only
// in F2.  Each wave then owns dE, dV and P for its 16 rows and dQ, dK for its
// 16 columns; dE crosses the waves once per mini-batch through LDS (one
// barrier), and the per-token deta partials ride on the same barrier.
//
// Precision: every fp32 operand enters the bf16 matrix cores as a hi + lo
// pair (|x - hi - lo| <= 2^-16 |x|); products of two fp32 operands take three
// passes (hi hi, hi lo, lo hi), products with bf16 inputs two.
//
// Staging: each 16-token tile is loaded PF mini-batches ahead into registers
// and, one step ahead, written to a double-buffered LDS slot already split:
// E and dZ as bf16 hi / lo tiles, and the state-rebuilding term
// R = 2 diag(eta) E as the negated split of the forward's own -2 eta e, so the
// rebuilt state subtracts exactly the operands the forward added.  The waves
// read every operand in the layout its product wants: rows with 8-byte
// loads, columns with the transposing LDS load (ds_read_b64_tr_b16).
#include "args_bwd.h"
#include "mfma_common.h"
#include "wave_prio.h"

namespace ttt {
namespace {

using namespace mfma;

constexpr int D = 64;       // head dim
constexpr int BT = 16;      // mini-batch (tokens)
constexpr int ROW = 68;     // padded LDS row of a bf16 token tile (elements, 136 B: 8-byte aligned rows)
constexpr int kThreads = 256;

typedef uint16_t Tile[BT * ROW];

struct __align__(16) BSlot {
  Tile q, k;        // inputs (bf16)
  Tile eh, el;      // E = W K - V, split
  Tile rh, rl;      // R = 2 diag(eta) E (the negated forward update factor), split
  Tile zh, zl;      // dZ, split
  float eta[BT];
};
static_assert(sizeof(BSlot) % 16 == 0, "slot size");

template <int PF, bool ETA_TOKEN, typename GT>
__global__ __launch_bounds__(kThreads) void ttt_linear_bwd_d64b16(BwdArgs a) {
  static_assert(PF >= 2, "a step stages its successor before it issues its own prefetch");
  __shared__ BSlot slots[2];
  __shared__ Tile deh, del;  // dE of all rows, split
  __shared__ float part[4][BT];

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

  typedef typename GradLoad<GT>::type GLoad;
  const u32x4* Qg = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.Q) + tok0 * D);
  const u32x4* Kg = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.K) + tok0 * D);
  const u32x4* Eg = reinterpret_cast<const u32x4*>(a.E + tok0 * D);
  const GLoad* Zg = reinterpret_cast<const GLoad*>(static_cast<const GT*>(a.dZ) + tok0 * D);
  GT* dQg = static_cast<GT*>(a.dQ) + tok0 * D;
  GT* dKg = static_cast<GT*>(a.dK) + tok0 * D;
  GT* dVg = static_cast<GT*>(a.dV) + tok0 * D;
  float* detag = a.deta + tok0;
  const float* eg = a.eta + bi * a.esb + h * a.esh;

  // staging roles: 16 B of Q (tid < 128) or K (tid >= 128) at row srow, columns
  // scol..scol+7; 4 values of E and of dZ at row frow = tid / 16, columns
  // fcol..fcol+3, and the step size of token frow
  const int within = tid & 127;
  const u32x4* srcA = (tid < 128 ? Qg : Kg) + within;
  const u32x4* srcE = Eg + tid;
  const GLoad* srcZ = Zg + tid;
  const int srow = within >> 3;
  const int scol = (within & 7) * 8;
  const int frow = tid >> 4;
  const int fcol = (tid & 15) * 4;
  const float* srcEta = eg + static_cast<int64_t>(frow) * a.est;

  u32x4 ra[PF], re[PF];
  GLoad rz[PF];
  float rt[PF];

  float eta_c = 0.f;
  if (!ETA_TOKEN && nb > 0) eta_c = eg[0];

  auto load_step = [&](int n, u32x4& xa, u32x4& xe, GLoad& xz, float& xt) {
    xa = ld_stream(srcA + static_cast<size_t>(n) * (BT * D / 8));
    xe = ld_stream(srcE + static_cast<size_t>(n) * (BT * D / 4));
    xz = ld_stream(srcZ + static_cast<size_t>(n) * (BT * D / 4));
    xt = ETA_TOKEN ? srcEta[static_cast<int64_t>(n) * BT * a.est] : 0.f;
  };
  auto stage = [&](int slot, const u32x4& xa, const u32x4& xe, const GLoad& xz, float xt) {
    BSlot& S = slots[slot];
    {
      // two 8-byte stores: a 136-byte row keeps 8-byte, not 16-byte, alignment
      u32x2* dst = reinterpret_cast<u32x2*>(tid < 128 ? &S.q[srow * ROW + scol] : &S.k[srow * ROW + scol]);
      dst[0] = u32x2{xa[0], xa[1]};
      dst[1] = u32x2{xa[2], xa[3]};
    }
    const float et = ETA_TOKEN ? xt : eta_c;
    float e[4], r[4], z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[i] = __uint_as_float(xe[i]);
      r[i] = -(-2.f * et * e[i]);  // the forward's update factor, negated (exact)
    }
    GradLoad<GT>::get(xz, z);
    const int off = frow * ROW + fcol;
    bf16x4 hi, lo;
    split4(e, hi, lo);
    put4(S.eh, off, hi);
    put4(S.el, off, lo);
    split4(r, hi, lo);
    put4(S.rh, off, hi);
    put4(S.rl, off, lo);
    split4(z, hi, lo);
    put4(S.zh, off, hi);
    put4(S.zl, off, lo);
    if (ETA_TOKEN && (tid & 15) == 0) S.eta[frow] = xt;
  };

  // state: W (F2) from the final state, A (F1 and F2) from dL/dW_final
  float4v w2[4], a2[4], a1[4];
  {
    const float* wf = a.Wf + static_cast<int64_t>(chain) * D * D;
    const float* af = a.dWf ? a.dWf + static_cast<int64_t>(chain) * D * D : nullptr;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = (16 * b + 4 * g + r) * D + 16 * w + li;
        w2[b][r] = wf[o];
        a2[b][r] = af ? af[o] : 0.f;
      }
      if (af) {
        const float4 x = *reinterpret_cast<const float4*>(af + (16 * w + li) * D + 16 * b + 4 * g);
        a1[b] = float4v{x.x, x.y, x.z, x.w};
      } else {
        a1[b] = zero4v();
      }
    }
  }
  // identity operand for transposing an accumulator tile: B[k][n] = [k == n],
  // slots 0-3 and 4-7 of lane group g both cover k = 4g .. 4g + 3
  bf16x8 ident;
#pragma unroll
  for (int j = 0; j < 8; ++j) ident[j] = (4 * g + (j & 3) == li) ? static_cast<__bf16>(1.f) : static_cast<__bf16>(0.f);

  // drain the state loads before the ring prologue (vmcnt = 0)
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // mini-batches are visited last to first: step j handles mini-batch nb - 1 - j
  if (nb > 0) {
#pragma unroll
    for (int j = 0; j < PF; ++j) load_step(max(nb - 1 - j, 0), ra[j], re[j], rz[j], rt[j]);
    stage(0, ra[0], re[0], rz[0], rt[0]);
  }
  __syncthreads();

  auto step = [&](const int j, u32x4& xa, u32x4& xe, GLoad& xz, float& xt, const u32x4& ya, const u32x4& ye,
                  const GLoad& yz, const float yt) {
    const int n = nb - 1 - j;
    stage((j + 1) & 1, ya, ye, yz, yt);
    load_step(max(n - PF, 0), xa, xe, xz, xt);
    const BSlot& S = slots[j & 1];

    float et[4], eta_li;
#pragma unroll
    for (int r = 0; r < 4; ++r) et[r] = ETA_TOKEN ? S.eta[4 * g + r] : eta_c;
    eta_li = ETA_TOKEN ? S.eta[li] : eta_c;

    // ---- S = K Q^T (s = 4g+r, t = li) and S^T (t = 4g+r, s = li): exact ----
    bf16x4 kx[4], qx[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      kx[t] = *reinterpret_cast<const bf16x4*>(&S.k[li * ROW + 16 * t + 4 * g]);
      qx[t] = *reinterpret_cast<const bf16x4*>(&S.q[li * ROW + 16 * t + 4 * g]);
    }
    float4v sc = zero4v(), st = zero4v(), p = zero4v();
    prio_mfma();  // the step's first run of matrix-core work: -1.0% at the 1.3B shape (raised for the later runs too: no gain)
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const bf16x8 ak = cat(kx[2 * m], kx[2 * m + 1]);
      const bf16x8 aq = cat(qx[2 * m], qx[2 * m + 1]);
      sc = mfma32(ak, aq, sc);
      st = mfma32(aq, ak, st);
      // ---- P[s][i] = sum_c K[s][c] A[i][c], rows i of this wave (F1) ----
      bf16x4 h0, l0, h1, l1;
      split4(a1[2 * m], h0, l0);
      split4(a1[2 * m + 1], h1, l1);
      p = mfma32(ak, cat(h0, h1), p);
      p = mfma32(ak, cat(l0, l1), p);
    }

    // ---- Y = E dZ^T (s = 4g+r, t = li), contraction over all 64 outputs ----
    bf16x4 erh[4], erl[4], zrh[4], zrl[4];
    rows4<ROW>(S.eh, li, g, erh);
    rows4<ROW>(S.el, li, g, erl);
    rows4<ROW>(S.zh, li, g, zrh);
    rows4<ROW>(S.zl, li, g, zrl);
    const float4v y = rows_x_f2(erh, erl, zrh, zrl, zero4v());
    prio_valu();

    // ---- dE = -2 dZ M^T - 2 P diag(eta), rows i of this wave ----
    const bf16x4 zwh = read_cols<ROW>(S.zh, 0, 16 * w, li, g);  // dZ[t = 4g+r][16w + li]
    const bf16x4 zwl = read_cols<ROW>(S.zl, 0, 16 * w, li, g);
    float4v mdz;
    {
      // A operand M[s = li][t = 4g+r] from S^T, causal mask s <= t, scale eta_s
      float mv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) mv[r] = (li <= 4 * g + r) ? eta_li * st[r] : 0.f;
      bf16x4 mh, ml;
      split4(mv, mh, ml);
      const bf16x4 z4 = {};
      mdz = mfma32(cat(mh, mh), cat(zwh, zwl), zero4v());
      mdz = mfma32(cat(ml, z4), cat(zwh, z4), mdz);
    }
    float de[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) de[r] = -2.f * mdz[r] - 2.f * et[r] * p[r];
    bf16x4 dh, dl;
    split4(de, dh, dl);
    {
      GT* vp = dVg + (static_cast<size_t>(n) * BT + 4 * g) * D + 16 * w + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        store_merged<GT>(vp + r * D, -de[r]);
        const int o = (4 * g + r) * ROW + 16 * w + li;
        deh[o] = bf16_bits(dh, r);
        del[o] = bf16_bits(dl, r);
      }
    }

    // ---- deta partials: -2 sum_t S Y [s <= t] (wave 0) - 2 sum_i E P (rows of this wave) ----
    {
      const bf16x4 ewh = read_cols<ROW>(S.eh, 0, 16 * w, li, g);  // E[4g + r][16w + li]
      const bf16x4 ewl = read_cols<ROW>(S.el, 0, 16 * w, li, g);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = (static_cast<float>(ewh[r]) + static_cast<float>(ewl[r])) * p[r];
        if (w == 0) x += (4 * g + r <= li) ? sc[r] * y[r] : 0.f;
        x = sum16(x);
        if (li == 0) part[w][4 * g + r] = -2.f * x;
      }
    }

    // ---- Y' = -2 eta_s Y [s <= t]; dQ = K Y' and dK = Q Y'^T parts ----
    const bf16x4 kw = read_cols<ROW>(S.k, 0, 16 * w, li, g);  // K[4g + r][16w + li]
    const bf16x4 qw = read_cols<ROW>(S.q, 0, 16 * w, li, g);  // Q[4g + r][16w + li]
    float4v dq, dk;
    {
      float yp[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) yp[r] = (4 * g + r <= li) ? -2.f * et[r] * y[r] : 0.f;
      bf16x4 yh, yl;
      split4(yp, yh, yl);
      const bf16x8 ya8 = cat(yh, yl);
      dq = mfma32(ya8, cat(kw, kw), zero4v());
      const float4v ypt = mfma32(ya8, ident, zero4v());  // Y'^T (t = 4g+r, s = li)
      bf16x4 th, tl;
      split4(ypt, th, tl);
      dk = mfma32(cat(th, tl), cat(qw, qw), zero4v());
    }

    // ---- A (F1, rows of this wave) += dZ Q^T + dE K^T, after P used it ----
    {
      const bf16x8 bz = cat(zwh, zwl), bd = cat(dh, dl);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x4 qt = read_cols<ROW>(S.q, 0, 16 * t, li, g);
        const bf16x4 kt = read_cols<ROW>(S.k, 0, 16 * t, li, g);
        a1[t] = mfma32(cat(qt, qt), bz, a1[t]);
        a1[t] = mfma32(cat(kt, kt), bd, a1[t]);
      }
    }

    // ---- rebuild the mini-batch-start state: W += R^T K, R = 2 diag(eta) E ----
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const bf16x4 rh = read_cols<ROW>(S.rh, 0, 16 * b, li, g);  // R[s = 4g+r][16b + li]
      const bf16x4 rl = read_cols<ROW>(S.rl, 0, 16 * b, li, g);
      w2[b] = mfma32(cat(rh, rl), cat(kw, kw), w2[b]);
    }
    bf16x4 wh[4], wl[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) split4(w2[b], wh[b], wl[b]);

    // ---- dQ += dZ W (contraction over the 64 rows of W) ----
    dq = rows_x_f2(zrh, zrl, wh, wl, dq);

    // ---- dK += -2 diag(eta) E A (A before this mini-batch's update, F2) ----
    {
      bf16x4 ah[4], al[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) split4(a2[b], ah[b], al[b]);
      const float4v ea = rows_x_f2(erh, erl, ah, al, zero4v());
#pragma unroll
      for (int r = 0; r < 4; ++r) dk[r] += -2.f * et[r] * ea[r];
    }

    __syncthreads();  // dE of all rows and the deta partials are in LDS

    // ---- dK += dE W ----
    {
      bf16x4 drh[4], drl[4];
      rows4<ROW>(deh, li, g, drh);
      rows4<ROW>(del, li, g, drl);
      dk = rows_x_f2(drh, drl, wh, wl, dk);
    }

    // ---- A (F2, columns of this wave) += dZ Q^T + dE K^T ----
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const bf16x4 zbh = read_cols<ROW>(S.zh, 0, 16 * b, li, g);
      const bf16x4 zbl = read_cols<ROW>(S.zl, 0, 16 * b, li, g);
      const bf16x4 dbh = read_cols<ROW>(deh, 0, 16 * b, li, g);
      const bf16x4 dbl = read_cols<ROW>(del, 0, 16 * b, li, g);
      a2[b] = mfma32(cat(zbh, zbl), cat(qw, qw), a2[b]);
      a2[b] = mfma32(cat(dbh, dbl), cat(kw, kw), a2[b]);
    }

    // ---- stores: dQ, dK rows 4g + r, columns 16w + li (64-byte pieces of a row
    // per wave, merged in the L2); deta ----
    {
      const size_t o = (static_cast<size_t>(n) * BT + 4 * g) * D + 16 * w + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        store_merged<GT>(dQg + o + r * D, dq[r]);
        store_merged<GT>(dKg + o + r * D, dk[r]);
      }
    }
    if (tid < BT) detag[n * BT + tid] = part[0][tid] + part[1][tid] + part[2][tid] + part[3][tid];

    __syncthreads();
  };

  const int nfull = nb / PF * PF;
  for (int j0 = 0; j0 < nfull; j0 += PF) {
#pragma unroll
    for (int jj = 0; jj < PF; ++jj) {
      const int jn = (jj + 1) % PF;
      step(j0 + jj, ra[jj], re[jj], rz[jj], rt[jj], ra[jn], re[jn], rz[jn], rt[jn]);
    }
  }
#pragma unroll
  for (int jj = 0; jj < PF; ++jj) {
    const int jn = (jj + 1) % PF;
    if (nfull + jj < nb) step(nfull + jj, ra[jj], re[jj], rz[jj], rt[jj], ra[jn], re[jn], rz[jn], rt[jn]);
  }

  // dL/dW0 = the adjoint of the first mini-batch's start state (F1 copy)
  float* dw = a.dW0 + static_cast<int64_t>(chain) * D * D + static_cast<int64_t>(16 * w + li) * D + 4 * g;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    *reinterpret_cast<float4*>(dw + 16 * t) = make_float4(a1[t][0], a1[t][1], a1[t][2], a1[t][3]);
}

// Prefetch ring depth (mini-batches in flight per thread; at least 2): 2
// measured 1.3% faster than 3 at the 1.3B shape and 4.4% at 64 sequences x 32K
// tokens (228 against 244 VGPRs), bit-identical results.
#ifndef TTT_BWD_PF
#define TTT_BWD_PF 2
#endif
constexpr int kPF = TTT_BWD_PF;

template <bool TOK>
hipError_t launch_tok(const BwdArgs& a, hipStream_t s) {
  dim3 grid(a.B * a.H), block(kThreads);
  if (a.out_dtype == 0)
    hipLaunchKernelGGL((ttt_linear_bwd_d64b16<kPF, TOK, float>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_linear_bwd_d64b16<kPF, TOK, uint16_t>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool linear_bwd_mfma_supported(const BwdArgs& a) { return a.d == 64 && a.b == 16 && a.in_dtype == 1; }

hipError_t launch_linear_bwd_mfma(const BwdArgs& a, hipStream_t s) {
  return a.est != 0 ? launch_tok<true>(a, s) : launch_tok<false>(a, s);
}

}  // namespace ttt
