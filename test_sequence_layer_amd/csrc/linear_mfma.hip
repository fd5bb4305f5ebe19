// TTT-Linear dual-form forward on CDNA4 matrix cores: d = 64, b = 16, bf16 Q/K/V.
//
// Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
// (aharts.cn / itmax.cn), part 03 §6 (mini-batch GD: every gradient of a
// mini-batch is taken at the state before it), §7 (dual form: never build the
// b per-token d x d gradients; get the mini-batch-end state and the b outputs
// from matrix products), §9 (TTT-Linear, f(x) = W x).
//
// Work decomposition
//   The 4 waves of a (sequence, head) walk its T/16 mini-batches in order.
//   Rows of W are independent (row i of the next state and of Z needs only
//   row i of W, column i of V and all of K, Q, eta), so wave w owns rows
//   [16w, 16w+16) of W and never talks to the other waves except through the
//   shared input tiles.  The 4 waves form one workgroup (RB = 1), or RB = 2 or
//   4 workgroups of 4 / RB waves (row blocks) when there are too few
//   sequences x heads to fill the chip; each row block then stages the whole
//   K and Q tiles itself (they are read from the L2 it shares with the
//   chain's other row blocks) and only its own columns of V.
//
// State layout (the key trick)
//   Wave w keeps W^T[c][i] (c = 0..63, i = 16w..16w+15) as four 16x16 fp32
//   MFMA accumulator tiles: lane l holds W[16w + l%16][16a + 4(l/16) + r] in
//   wt[a][r].  That is exactly the B-operand layout (k = c, n = i) the
//   projections K W^T and Q W^T need, so the state is fed back into the
//   matrix cores with no transpose and no LDS round trip, and the rank-16
//   update accumulates straight into it.
//
// Per mini-batch, per wave (M = 16 tokens, N = 16 rows of W):
//   P_K = K W^T, P_Q = Q W^T    v_mfma_f32_16x16x32_bf16, W split hi+lo bf16
//   S   = K Q^T (s x t)         v_mfma_f32_16x16x32_bf16, exact bf16 products
//   E   = P_K - V               registers (E^T layout: lane = (t = 4g+r, i))
//   G   = -2 diag(eta) E        registers (same layout as E)
//   Z   = P_Q + M G,  M[t][s] = S[s][t] [s <= t]
//                               v_mfma_f32_16x16x32_bf16 x2 (4 split passes)
//   W^T += K^T G                v_mfma_f32_16x16x32_bf16, [K^T K^T] x [G_hi G_lo]
//   Only the native gfx950 K=32 bf16 MFMA is used: a 16-token contraction
//   puts two split passes into its 8 k-slots per lane group.
//   The S accumulator layout (s = 4g+r, t = l%16) is the A-operand layout of
//   M, and the E accumulator layout is the B-operand layout of both the Z
//   correction and the update: the causal mask and the eta scaling are
//   applied in registers between the products, and G is split once for both.
//
// Precision: fp32 operands enter the bf16 matrix cores as hi + lo bf16 pairs,
// each rounded to nearest (bf16 keeps 8 significant bits, so |x - hi| <= 2^-8 |x|
// and |x - hi - lo| <= 2^-16 |x|); bf16 x bf16 products are exact and every
// sum is fp32, so the result tracks an fp32 computation to ~1e-5.
//
// Streaming: a 16-token tile of Q, K, V is 3 x 2 KB contiguous.  Each step
// loads the tile PF steps ahead into registers (coalesced 16-byte loads),
// stores the tile one step ahead into a double-buffered LDS slot, and issues
// one barrier.  Z goes out through a double-buffered LDS tile as whole rows,
// one step late, so every store instruction writes contiguous 16-byte pieces.  The update's K^T operand and E's V values are column reads of
// the row-major tiles with the gfx950 transposing LDS load (ds_read_b64_tr_b16).
#include "args_linear.h"
#include "mfma_common.h"
#include "wave_prio.h"

namespace ttt {
namespace {

using namespace mfma;

constexpr int D = 64;       // head dim
constexpr int BT = 16;      // mini-batch (tokens)
constexpr int ROW = 72;     // padded LDS row of a token tile (bf16 elements, 144 B)
constexpr int ZROW = 68;    // padded fp32 row of the Z staging tile (conflict-free deposits)

struct __align__(16) Slot {
  uint16_t q[BT * ROW];
  uint16_t k[BT * ROW];
  uint16_t v[BT * ROW];
  float eta[BT];
};
static_assert(sizeof(Slot) % 16 == 0, "slot size");

// ---- layer norm: tokens split over the waves ------------------------------
// The row-split waves each hold 16 of a token's 64 outputs.  For the layer
// norm they swap roles through LDS: each wave deposits its transposed tile
// (lane l: token l%16, outputs 16w + 4(l/16) + r) as row pieces of a
// [token][output] tile, and then normalises 4 whole tokens, 4w + l/16, 4 outputs
// (4(l%16) + r) per lane, so a token's sums are 16-lane DPP reductions.
struct LnShared {
  float yk[BT * ZROW];    // W k of the mini-batch, fp32 [token][output]
  float yq[BT * ZROW];    // the pre-norm outputs W_t q, fp32 [token][output]
  uint16_t gh[BT * ROW];  // the update factor G, bf16 hi, [token][output]
  uint16_t gl[BT * ROW];  //   and lo
};

// Mean and centred values of the 64 entries a 16-lane row holds 4 at a time,
// and 1/sqrt(variance + eps): two passes, no cancellation of raw power sums.
__device__ __forceinline__ float ln_centre(const float4 y, float dv[4], float eps) {
  const float mu = sum16((y.x + y.y) + (y.z + y.w)) * (1.f / 64.f);
  dv[0] = y.x - mu;
  dv[1] = y.y - mu;
  dv[2] = y.z - mu;
  dv[3] = y.w - mu;
  float m2 = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) m2 = fmaf(dv[r], dv[r], m2);
  return rsqrtf(sum16(m2) * (1.f / 64.f) + eps);
}

// LDS of one workgroup, declared as separate arrays by each kernel (measured:
// one struct holding them made the latency-bound forward 3% slower) and handed
// to the body by reference: the double-buffered input slots, the layer norm's
// exchange tiles, and for the forward the staging tiles of Z (and of E when it
// is saved): each wave deposits its 16 outputs of every token, fp32
// [token][output] with rows padded to ZROW, and one step later every thread
// writes 16 contiguous bytes of whole rows.
template <bool ZB, bool SAVE>
struct Shm {
  Slot (&slots)[2];
  LnShared& lns;
  float (&zbuf)[ZB ? 2 : 1][ZB ? BT * ZROW : 4];
  float (&ebuf)[SAVE ? 2 : 1][SAVE ? BT * ZROW : 4];
};

// The stretch of one (sequence, head) chain a workgroup walks, and where its
// state starts and ends.
struct Unit {
  int chain;
  int rblk;              // row block (rows 64 / RB * rblk ..)
  int64_t mb0;           // first mini-batch
  int nb;                // mini-batches
  const float* w_start;  // MODE 0: start state, row-major d x d (z = W q)
  float* w_end;          // MODE 0: end state (nullptr: not kept); MODE 1: P
  float* w_end2;         // MODE 1: R
};

// First mini-batch of chunk c when nb mini-batches are split into n chunks,
// chunk 0 holding mb1 of them and the rest shared evenly (c = n: nb).
__device__ __forceinline__ int64_t chunk_begin(int64_t c, int64_t nb, int64_t n, int64_t mb1) {
  return c == 0 ? 0 : mb1 + (c - 1) * (nb - mb1) / (n - 1);
}

// MODE 0: forward (Z and the end state).  MODE 1: the two maps of one chunk of
// a chunked forward, W_end = W_start P + R: P is the state recurrence run from I
// with V = 0 and R the recurrence run from 0 with V, over the chunk, with no
// query path and no Z; every wave holds its 16 rows of both (they share the
// staged K and V tiles).
// LN: f(x) = x + LN(W x) (layer norm and residual inside f; MODE 0 only).
// SAVE: also write the backward's input of every token (MODE 0): E = W K - V,
// or with LN the update factor G = -eta delta as applied (delta the gradient
// of the token's loss with respect to W k).
// RB: row blocks (workgroups) per (sequence, head, chunk); 1, 2 or 4.
template <int PF, bool ETA_TOKEN, typename OutT, int MODE, bool LN, bool SAVE, int RB, typename SH>
__device__ __forceinline__ void linear_body(const LinearArgs& a, SH& sh, const Unit& u) {
  static_assert(PF >= 2, "a step stages its successor before it issues its own prefetch");
  static_assert(RB == 1 || RB == 2 || RB == 4, "row blocks");
  static_assert(!LN || RB == 1, "the layer norm needs all 64 outputs of a token in one workgroup");
  static_assert(!LN || MODE == 0, "the maps have no layer norm");
  static_assert(MODE == 0 || (RB == 1 && !SAVE), "the maps run in whole workgroups");
  constexpr int NWV = 4 / RB;   // waves per workgroup
  constexpr int NT = 64 * NWV;  // threads per workgroup
  constexpr int CA = 256 / NT;  // 16-byte pieces of the Q|K tiles each thread stages per step
  auto& slots = sh.slots;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int li = lane & 15;
  const int g = lane >> 4;

  const int chain = u.chain;
  const int rblk = u.rblk;
  const int wg = NWV * rblk + w;  // this wave's rows of W: [16 wg, 16 wg + 16)
  const int bi = chain / a.H;
  const int h = chain - bi * a.H;
  const int nb = u.nb;

  const size_t tok0 = static_cast<size_t>(chain) * a.T + static_cast<size_t>(u.mb0) * BT;
  const u32x4* Qg = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.Q) + tok0 * D);
  const u32x4* Kg = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.K) + tok0 * D);
  const u32x4* Vg = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.V) + tok0 * D);
  OutT* Zg = static_cast<OutT*>(a.Z) + tok0 * D;
  const float* eg = a.eta + bi * a.esb + h * a.esh + u.mb0 * BT * a.est;

  // staging roles (every load unconditional, so the ring stays in registers):
  //   CA 16-byte pieces of the Q|K tiles: piece x = tid + c NT of the 256
  //   (x < 128: Q, else K) is row (x & 127) / 8, columns 8 (x & 7) .. +7;
  //   8 B of V in this row block's columns: row vrow, columns vcol .. vcol+3;
  //   eta of token (tid & 15).
  // The maps have no query path: there V takes Q's place in the 16-byte
  // pieces and the 8-byte V loads are dropped (4 KB per step, not 6).
  const u32x4* tileA = MODE == 0 ? Qg : Vg;
  const u32x4* srcA[CA];
#pragma unroll
  for (int c = 0; c < CA; ++c) {
    const int x = tid + c * NT;
    srcA[c] = (x < 128 ? tileA : Kg) + (x & 127);
  }
  const int vrow = tid / (4 * NWV);
  const int vcol = 16 * NWV * rblk + (tid % (4 * NWV)) * 4;
  const u32x2* srcB = reinterpret_cast<const u32x2*>(Vg) + (vrow * D + vcol) / 4;
  const float* srcE = eg + static_cast<int64_t>(tid & 15) * a.est;

  u32x4 ra[PF][CA];
  u32x2 rb[PF];
  float re[PF];

  auto load_step = [&](int n, u32x4 (&xa)[CA], u32x2& xb, float& xe) {
#pragma unroll
    for (int c = 0; c < CA; ++c) xa[c] = ld_stream(srcA[c] + static_cast<size_t>(n) * (BT * D / 8));  // 128 uint4 per tile
    if constexpr (MODE == 0) xb = ld_stream(srcB + static_cast<size_t>(n) * (BT * D / 4));  // 256 uint2 per tile
    xe = ETA_TOKEN ? srcE[static_cast<int64_t>(n) * BT * a.est] : 0.f;
  };
  auto stage = [&](int slot, const u32x4 (&xa)[CA], const u32x2& xb, float xe) {
    Slot& S = slots[slot];
    if constexpr (MODE == 0) *reinterpret_cast<u32x2*>(&S.v[vrow * ROW + vcol]) = xb;
#pragma unroll
    for (int c = 0; c < CA; ++c) {
      const int x = tid + c * NT, within = x & 127;
      uint16_t* dst = x < 128 ? (MODE == 0 ? S.q : S.v) : S.k;
      *reinterpret_cast<u32x4*>(&dst[(within >> 3) * ROW + (within & 7) * 8]) = xa[c];
    }
    if (ETA_TOKEN && tid < BT) S.eta[tid] = xe;
  };

  // constant eta (scalar or per head)
  float eta_c = 0.f;
  if (!ETA_TOKEN && nb > 0) eta_c = eg[0];
  // LN scale and shift of outputs 4(l%16) + j (the token rows this lane normalises)
  float4v ln_g = {}, ln_b = {};
  if constexpr (LN) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // (gamma and beta are only 4-byte aligned)
      ln_g[j] = a.gamma[h * D + 4 * li + j];
      ln_b[j] = a.beta[h * D + 4 * li + j];
    }
  }
  [[maybe_unused]] const int tk = 4 * w + g;  // the token whose layer norms this lane takes part in
  // (layer norm: a step's output norm runs after the next step's first barrier,
  // which also publishes its pre-norm tile; qp holds that step's Q residual)
  [[maybe_unused]] bf16x4 qp = {};

  // resident state: wt[a][r] = W[16w + li][16a + 4g + r] (the maps: P in wt, R in wr)
  float4v wt[4];
  [[maybe_unused]] float4v wr[4];
  if constexpr (MODE == 0) {
    const float* w0 = u.w_start + static_cast<int64_t>(16 * wg + li) * D + 4 * g;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float4 x = *reinterpret_cast<const float4*>(w0 + 16 * t);
      wt[t] = float4v{x.x, x.y, x.z, x.w};
    }
  } else {
    // P starts from the identity, R from zero
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        wt[t][r] = (16 * wg + li == 16 * t + 4 * g + r) ? 1.f : 0.f;
        wr[t][r] = 0.f;
      }
  }

  // Drain the state / eta loads before the ring prologue: otherwise the
  // compiler's wait analysis sees them pending at the loop header and makes
  // every step wait for them, i.e. for most of the prefetch ring, which
  // serialises it.  The empty asm statements read the loaded state registers,
  // so the loads cannot sink below this point (a bare s_waitcnt does not stop
  // that) and their wait is placed here, once.  (s_waitcnt immediate: vmcnt =
  // 0, expcnt = 7, lgkmcnt = 15.)
  if constexpr (MODE == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) asm volatile("" : "+v"(wt[t]));
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);

  if (nb > 0) {
#pragma unroll
    for (int j = 0; j < PF; ++j) load_step(min(j, nb - 1), ra[j], rb[j], re[j]);
    stage(0, ra[0], rb[0], re[0]);
  }
  __syncthreads();

  // One mini-batch: stage step n+1 (ring slot jn) into LDS, prefetch step
  // min(n+PF, nb-1) into ring slot j, compute step n, barrier.  The prefetch
  // index is clamped instead of guarded so every step issues the same memory
  // operations and the compiler's wait counts stay exact.
  // Z rows of mini-batch m from the staging tile to HBM: thread tid writes
  // token tid / (4 NWV), this row block's outputs fcol .. fcol + 3.  One row
  // block writes whole 256-byte rows (non-temporal); several write a piece of
  // every row each, and the pieces merge in the L2 before they reach HBM.
  const int frow = tid / (4 * NWV);
  const int fl = (tid % (4 * NWV)) * 4;    // column in the staging tile
  const int fcol = 16 * NWV * rblk + fl;   // output column
  auto put = [](auto* p, auto x) {
    if constexpr (RB == 1) {
      st_stream(p, x);
    } else {
      *p = x;
    }
  };
  auto flush_z = [&](int m) {
    if constexpr (SAVE && !LN) {
      const float4 e4 = *reinterpret_cast<const float4*>(&sh.ebuf[m & 1][frow * ZROW + fl]);
      float* ep = a.Esave + (tok0 + static_cast<size_t>(m) * BT + frow) * D + fcol;
      put(reinterpret_cast<u32x4*>(ep),
          u32x4{__float_as_uint(e4.x), __float_as_uint(e4.y), __float_as_uint(e4.z), __float_as_uint(e4.w)});
    }
    const float4 x = *reinterpret_cast<const float4*>(&sh.zbuf[m & 1][frow * ZROW + fl]);
    OutT* zp = Zg + (static_cast<size_t>(m) * BT + frow) * D + fcol;
    if constexpr (sizeof(OutT) == 4) {
      put(reinterpret_cast<u32x4*>(zp),
          u32x4{__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z), __float_as_uint(x.w)});
    } else {
      put(reinterpret_cast<u32x2*>(zp),
          u32x2{static_cast<uint32_t>(f32_to_bf16_bits(x.x)) | (static_cast<uint32_t>(f32_to_bf16_bits(x.y)) << 16),
                static_cast<uint32_t>(f32_to_bf16_bits(x.z)) | (static_cast<uint32_t>(f32_to_bf16_bits(x.w)) << 16)});
    }
  };

  // z = q + LN(W_t q) of mini-batch m from the pre-norm [token][output] tile:
  // this lane normalises token tk, outputs 4 li .. 4 li + 3, and writes them to
  // HBM as a 16-byte piece of the token's row (16 lanes: the whole row)
  auto ln_out = [&](int m) {
    if constexpr (LN) {
      float dv[4];
      const float rs = ln_centre(*reinterpret_cast<const float4*>(&sh.lns.yq[tk * ZROW + 4 * li]), dv, a.eps);
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = static_cast<float>(qp[r]) + ln_g[r] * (dv[r] * rs) + ln_b[r];
      OutT* zp = Zg + (static_cast<size_t>(m) * BT + tk) * D + 4 * li;
      if constexpr (sizeof(OutT) == 4) {
        st_stream(reinterpret_cast<u32x4*>(zp),
                  u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])});
      } else {
        st_stream(reinterpret_cast<u32x2*>(zp),
                  u32x2{static_cast<uint32_t>(f32_to_bf16_bits(o[0])) | (static_cast<uint32_t>(f32_to_bf16_bits(o[1])) << 16),
                        static_cast<uint32_t>(f32_to_bf16_bits(o[2])) | (static_cast<uint32_t>(f32_to_bf16_bits(o[3])) << 16)});
      }
    }
  };

  auto step = [&](const int n, u32x4 (&xa)[CA], u32x2& xb, float& xe, const u32x4 (&ya)[CA], const u32x2& yb,
                  const float ye) {
    stage((n + 1) & 1, ya, yb, ye);
    load_step(min(n + PF, nb - 1), xa, xb, xe);
    const Slot& S = slots[n & 1];
    // ---- operands: token rows li, column groups {16a + 4g .. +3} ----
    bf16x4 kx[4], qx[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      kx[t] = *reinterpret_cast<const bf16x4*>(&S.k[li * ROW + 16 * t + 4 * g]);
      if constexpr (MODE == 0) qx[t] = *reinterpret_cast<const bf16x4*>(&S.q[li * ROW + 16 * t + 4 * g]);
    }
    float et[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) et[r] = ETA_TOKEN ? S.eta[4 * g + r] : eta_c;

    if constexpr (MODE != 0) {
      // ---- the maps: E_X = K X^T - V_X for X = P (V_P = 0) and R (V_R = V), and
      // X^T += K^T G_X, G_X = -2 diag(eta) E_X, on the shared K and V tiles ----
      float4v pp = {0.f, 0.f, 0.f, 0.f}, pr = pp;
      prio_mfma();  // -1.0% for the 5-chunk long workload
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const bf16x8 ak = cat(kx[2 * m], kx[2 * m + 1]);
        float p8[8], r8[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p8[r] = wt[2 * m][r];
          p8[4 + r] = wt[2 * m + 1][r];
          r8[r] = wr[2 * m][r];
          r8[4 + r] = wr[2 * m + 1][r];
        }
        bf16x4 h0, l0, h1, l1;
        split4(p8, h0, l0);
        split4(p8 + 4, h1, l1);
        pp = mfma32(ak, cat(h0, h1), pp);
        pp = mfma32(ak, cat(l0, l1), pp);
        split4(r8, h0, l0);
        split4(r8 + 4, h1, l1);
        pr = mfma32(ak, cat(h0, h1), pr);
        pr = mfma32(ak, cat(l0, l1), pr);
      }
      prio_valu();
      const bf16x4 vc = read_cols<ROW>(S.v, 0, 16 * wg, li, g);  // V[4g + r][16wg + li]
      float gp[4], gr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        gp[r] = -2.f * et[r] * pp[r];
        gr[r] = -2.f * et[r] * (pr[r] - static_cast<float>(vc[r]));
      }
      bf16x4 ph, pl, rh, rl;
      split4(gp, ph, pl);
      split4(gr, rh, rl);
      const bf16x8 gpb = cat(ph, pl), grb = cat(rh, rl);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x4 kt = read_cols<ROW>(S.k, 0, 16 * t, li, g);  // K[4g + r][16t + li]
        wt[t] = mfma32(cat(kt, kt), gpb, wt[t]);
        wr[t] = mfma32(cat(kt, kt), grb, wr[t]);
      }
      __syncthreads();
      return;
    }
    // (layer norm: the residual's Q row piece of token tk, read now, before the
    // step's last barrier)
    bf16x4 qr = {};
    if constexpr (LN) qr = *reinterpret_cast<const bf16x4*>(&S.q[tk * ROW + 4 * li]);

    // ---- P_K = K W^T, P_Q = Q W^T, S = K Q^T ----
    float4v pk = {0.f, 0.f, 0.f, 0.f}, pq = pk, sc = pk;
    prio_mfma();  // the step's long run of matrix-core work: -2.2% at the 1.3B shape, -1.9% with the layer norm
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
      const bf16x8 ak = cat(kx[2 * m], kx[2 * m + 1]);
      const bf16x8 aq = cat(qx[2 * m], qx[2 * m + 1]);
      if constexpr (LN) {
        // transposed: P_K^T[i = 16w + 4g + r][t = li] (lane li holds token li)
        pk = mfma32(whi, ak, pk);
        pq = mfma32(whi, aq, pq);
        sc = mfma32(ak, aq, sc);
        pk = mfma32(wlo, ak, pk);
        pq = mfma32(wlo, aq, pq);
      } else {
        pk = mfma32(ak, whi, pk);
        pq = mfma32(aq, whi, pq);
        sc = mfma32(ak, aq, sc);
        pk = mfma32(ak, wlo, pk);
        pq = mfma32(aq, wlo, pq);
      }
    }

    prio_valu();
    // ---- E^T[t = 4g+r][i = 16w+li] = P_K - V ----
    // ---- G[s][i] = -eta_s (dl/dy)[s][i]: the gradient factor of the rank-16
    // update, also the operand of the Z correction ----
    bf16x4 bhi, blo;
    // (layer norm: the update's K column reads are made before the G barrier,
    // the step's last, so that no read of the slot follows it)
    [[maybe_unused]] bf16x4 kc[4] = {};
    if constexpr (LN) {
#pragma unroll
      for (int t = 0; t < 4; ++t) kc[t] = read_cols<ROW>(S.k, 0, 16 * t, li, g);
      // y = W k, f(k) = k + LN(y); dl/dy back through LN at the mini-batch-start
      // state.  The wave's transposed tile goes to the [token][output] tile ...
      *reinterpret_cast<float4*>(&sh.lns.yk[li * ZROW + 16 * w + 4 * g]) = make_float4(pk[0], pk[1], pk[2], pk[3]);
      __syncthreads();
      if (n > 0) ln_out(n - 1);  // the previous step's pre-norm tile is visible too
      qp = qr;
      // ... and this lane takes token tk, outputs 4 li .. 4 li + 3
      float dv[4];
      const float rs = ln_centre(*reinterpret_cast<const float4*>(&sh.lns.yk[tk * ZROW + 4 * li]), dv, a.eps);
      const bf16x4 kr = *reinterpret_cast<const bf16x4*>(&S.k[tk * ROW + 4 * li]);
      const bf16x4 vr = *reinterpret_cast<const bf16x4*>(&S.v[tk * ROW + 4 * li]);
      float yh[4], gr[4], s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        yh[r] = dv[r] * rs;
        const float res = static_cast<float>(kr[r]) - static_cast<float>(vr[r]) + ln_b[r] + ln_g[r] * yh[r];
        gr[r] = 2.f * ln_g[r] * res;
        s1 += gr[r];
        s2 = fmaf(gr[r], yh[r], s2);
      }
      s1 = sum16(s1) * (1.f / 64.f);  // the two means over the 64 outputs
      s2 = sum16(s2) * (1.f / 64.f);
      const float sg = -(ETA_TOKEN ? S.eta[tk] : eta_c) * rs;
      float d[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) d[r] = sg * (gr[r] - s1 - yh[r] * s2);
      // G = -eta delta, split once, as [token][output] rows; read back in the
      // operand layout (lane = output 16w + l%16, slots = tokens)
      bf16x4 dh, dl;
      split4(d, dh, dl);
      if constexpr (SAVE) {
        // G exactly as the update applies it (hi + lo is exact in fp32), 16
        // lanes writing the token's row
        float* ep = a.Esave + (tok0 + static_cast<size_t>(n) * BT + tk) * D + 4 * li;
        float gs[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) gs[r] = static_cast<float>(dh[r]) + static_cast<float>(dl[r]);
        st_stream(reinterpret_cast<u32x4*>(ep),
                  u32x4{__float_as_uint(gs[0]), __float_as_uint(gs[1]), __float_as_uint(gs[2]), __float_as_uint(gs[3])});
      }
      *reinterpret_cast<bf16x4*>(&sh.lns.gh[tk * ROW + 4 * li]) = dh;
      *reinterpret_cast<bf16x4*>(&sh.lns.gl[tk * ROW + 4 * li]) = dl;
      __syncthreads();
      bhi = read_cols<ROW>(sh.lns.gh, 0, 16 * w, li, g);
      blo = read_cols<ROW>(sh.lns.gl, 0, 16 * w, li, g);
    } else {
      float gv[4];
      float e[4];
      {
        const bf16x4 vc = read_cols<ROW>(S.v, 0, 16 * wg, li, g);  // V[4g + r][16wg + li]
#pragma unroll
        for (int r = 0; r < 4; ++r) e[r] = pk[r] - static_cast<float>(vc[r]);
      }
      if constexpr (SAVE) {
        float* eb = &sh.ebuf[n & 1][(4 * g) * ZROW + 16 * w + li];
#pragma unroll
        for (int r = 0; r < 4; ++r) eb[r * ZROW] = e[r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) gv[r] = -2.f * et[r] * e[r];
      split4(gv, bhi, blo);
    }

    // ---- Z = P_Q + M G, with M[t][s] = S[s][t] [s <= t] (causal mask, diagonal
    // included), G the operand the update uses too ----
    float4v z = pq;
    if constexpr (MODE == 0) {
      float mv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) mv[r] = (4 * g + r <= li) ? sc[r] : 0.f;
      bf16x4 mhi, mlo;
      split4(mv, mhi, mlo);
      // The 16x16x32 MFMA sums 8 k-slots per lane group; a 16-token contraction
      // uses slots 0-3 and 4-7 for two passes at once: [Mhi Mhi] x [Ghi Glo] and
      // [Mlo Mlo] x [Ghi Glo] (the update's own G operand and no zero-padded
      // halves to build; the extra lo x lo product is below fp32 rounding).
      const bf16x8 gz = cat(bhi, blo);
      if constexpr (LN) {
        // transposed: Z^T = G^T M^T
        z = mfma32(gz, cat(mhi, mhi), z);
        z = mfma32(gz, cat(mlo, mlo), z);
      } else {
        z = mfma32(cat(mhi, mhi), gz, z);
        z = mfma32(cat(mlo, mlo), gz, z);
      }
    }

    // ---- W^T[c][i] += sum_s K[s][c] G[s][i] ----
    const bf16x8 gb = cat(bhi, blo);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x4 kt = LN ? kc[t] : read_cols<ROW>(S.k, 0, 16 * t, li, g);  // K[4g + r][16t + li]
      wt[t] = mfma32(cat(kt, kt), gb, wt[t]);
    }

    if constexpr (LN) {
      // the pre-norm z of this step, transposed, as row pieces of the [token][output]
      // tile: the next step's first barrier (or the one after the last step)
      // publishes it and ln_out normalises it.  No read of the slot follows the
      // G barrier (Q and K were read before it), so the next step may restage
      // the slot at once and the step needs no closing barrier.
      *reinterpret_cast<float4*>(&sh.lns.yq[li * ZROW + 16 * w + 4 * g]) = make_float4(z[0], z[1], z[2], z[3]);
    } else if constexpr (MODE == 0) {
      // ---- store Z rows t = 4g + r, columns 16w + li ----
      if (n > 0) flush_z(n - 1);
      float* zb = &sh.zbuf[n & 1][(4 * g) * ZROW + 16 * w + li];
#pragma unroll
      for (int r = 0; r < 4; ++r) zb[r * ZROW] = z[r];
    }

    if constexpr (!LN) __syncthreads();
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

  if constexpr (MODE == 0 && !LN) {
    if (nb > 0) flush_z(nb - 1);  // the last step's barrier made its tile visible
  }
  if constexpr (LN) {
    __syncthreads();  // the last step's pre-norm tile
    if (nb > 0) ln_out(nb - 1);
  }

  // end state (a chunk that is not the sequence's last keeps none) / the maps
  const int64_t off = static_cast<int64_t>(16 * wg + li) * D + 4 * g;
  if (u.w_end) {
    float* wf = u.w_end + off;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      *reinterpret_cast<float4*>(wf + 16 * t) = make_float4(wt[t][0], wt[t][1], wt[t][2], wt[t][3]);
  }
  if constexpr (MODE != 0) {
    float* wf = u.w_end2 + off;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      *reinterpret_cast<float4*>(wf + 16 * t) = make_float4(wr[t][0], wr[t][1], wr[t][2], wr[t][3]);
  }
}

// The plain forward (one unit per chain, the whole sequence from W0) and the
// last pass of a chunked forward (a.nchunk > 1: one unit per chain and chunk
// 1 .. nchunk - 1, each from its start state in a.Wstart; the last chunk writes
// W_final).
template <int PF, bool ETA_TOKEN, typename OutT, bool LN, bool SAVE, int RB>
__global__ __launch_bounds__(256 / RB) void ttt_linear_mfma_d64b16(LinearArgs a) {
  __shared__ Slot slots[2];
  __shared__ LnShared lns;
  __shared__ __align__(16) float zbuf[!LN ? 2 : 1][!LN ? BT * ZROW : 4];
  constexpr bool EB = SAVE && !LN;  // E staged like Z (the layer norm writes delta directly)
  __shared__ __align__(16) float ebuf[EB ? 2 : 1][EB ? BT * ZROW : 4];
  Shm<!LN, EB> sh{slots, lns, zbuf, ebuf};
  const int per_chain = a.nchunk > 1 ? a.nchunk - 1 : 1;
  const int units = a.B * a.H * per_chain;
  // The RB row blocks of a unit are 8 block indices apart, so the round-robin
  // dispatch of workgroups over the 8 XCDs places them on one XCD (one L2).
  // A last group of fewer than 8 units is packed the same way with its size.
  int unit = blockIdx.x, rblk = 0;
  if constexpr (RB > 1) {
    const int full = units / 8;
    const int grp = unit / (8 * RB);
    const int in = unit - grp * 8 * RB;
    const int width = grp < full ? 8 : units - full * 8;  // > 0: blockIdx.x < units * RB
    rblk = in / width;
    unit = grp * 8 + (in - rblk * width);
  }
  Unit u;
  u.chain = unit / per_chain;
  u.rblk = rblk;
  u.w_end2 = nullptr;
  const int64_t nbt = a.T / BT;
  if (a.nchunk > 1) {
    const int c = 1 + (unit - u.chain * per_chain);
    u.mb0 = chunk_begin(c, nbt, a.nchunk, a.mb1);
    u.nb = static_cast<int>(chunk_begin(c + 1, nbt, a.nchunk, a.mb1) - u.mb0);
    u.w_start = a.Wstart + (static_cast<int64_t>(u.chain) * (a.nchunk - 1) + (c - 1)) * D * D;
    u.w_end = c == a.nchunk - 1 ? a.Wf + static_cast<int64_t>(u.chain) * D * D : nullptr;
  } else {
    const int bi = u.chain / a.H, h = u.chain - bi * a.H;
    u.mb0 = 0;
    u.nb = static_cast<int>(nbt);
    u.w_start = a.W0 + bi * a.w0_bstride + static_cast<int64_t>(h) * D * D;
    u.w_end = a.Wf + static_cast<int64_t>(u.chain) * D * D;
  }
  linear_body<PF, ETA_TOKEN, OutT, 0, LN, SAVE, RB>(a, sh, u);
}

// The first pass of a chunked forward: per chain, nchunk - 1 units.  Unit 0
// runs the forward of chunk 0 from W0 (Z of its tokens, and its end state =
// the start state of chunk 1, a.Wstart[chain][0]); unit c = 1 .. nchunk - 2
// computes the maps P_c, R_c of chunk c (a.maps[chain][c - 1]).  The last
// chunk needs no map: the scan only has to reach its start state.
template <int PF, bool ETA_TOKEN, typename OutT>
__global__ __launch_bounds__(256) void ttt_linear_mfma_head_maps(LinearArgs a) {
  __shared__ Slot slots[2];
  __shared__ LnShared lns;  // (unused: no layer norm here)
  __shared__ __align__(16) float zbuf[2][BT * ZROW];
  __shared__ __align__(16) float ebuf[1][4];
  Shm<true, false> sh{slots, lns, zbuf, ebuf};
  const int per_chain = a.nchunk - 1;
  Unit u;
  u.chain = blockIdx.x / per_chain;
  const int c = blockIdx.x - u.chain * per_chain;
  u.rblk = 0;
  const int64_t nbt = a.T / BT;
  u.mb0 = chunk_begin(c, nbt, a.nchunk, a.mb1);
  u.nb = static_cast<int>(chunk_begin(c + 1, nbt, a.nchunk, a.mb1) - u.mb0);
  if (c == 0) {
    const int bi = u.chain / a.H, h = u.chain - bi * a.H;
    u.w_start = a.W0 + bi * a.w0_bstride + static_cast<int64_t>(h) * D * D;
    u.w_end = a.Wstart + static_cast<int64_t>(u.chain) * (a.nchunk - 1) * D * D;
    u.w_end2 = nullptr;
    linear_body<PF, ETA_TOKEN, OutT, 0, false, false, 1>(a, sh, u);
  } else {
    float* m = a.maps + (static_cast<int64_t>(u.chain) * (a.nchunk - 2) + (c - 1)) * 2 * D * D;
    u.w_start = nullptr;
    u.w_end = m;
    u.w_end2 = m + D * D;
    linear_body<PF, ETA_TOKEN, OutT, 1, false, false, 1>(a, sh, u);
  }
}

#ifndef TTT_LINEAR_PF
#define TTT_LINEAR_PF 6
#endif
#ifndef TTT_LINEAR_PF_LONG
#define TTT_LINEAR_PF_LONG 8
#endif
// Prefetch distance (mini-batches in flight per thread).  Measured: the plain
// forward at the 1.3B shape (512 workgroups, two per CU) runs ~1% faster with 6
// than with 8 (5 and 7 are slower), but with one workgroup or less per CU (64
// sequences x 32K tokens) 6 is 7% slower than 8, since no other workgroup hides
// a wave's memory latency; the layer-norm forward is ~1% faster with 8; the map
// pass keeps 8.  A thread of a smaller row block stages more of each tile
// (CA + 1 loads per step), so its ring is shorter; those launches are
// latency-bound (few chains), not bandwidth-bound.
template <int RB, bool LONG = false>
constexpr int pf_for() { return RB != 1 ? 4 : LONG ? TTT_LINEAR_PF_LONG : TTT_LINEAR_PF; }
constexpr int64_t kShortRingUnits = 512;  // workgroups from which the plain forward takes the short ring

template <bool TOK, bool LN, int RB, bool LONG = LN>
hipError_t launch_rb(const LinearArgs& a, hipStream_t s) {
  constexpr int PF = pf_for<RB, LONG>();
  const int64_t units = static_cast<int64_t>(a.B) * a.H * (a.nchunk > 1 ? a.nchunk - 1 : 1);
  dim3 grid(units * RB), block(256 / RB);
  if constexpr (!LN && RB == 1 && !LONG) {
    if (units < kShortRingUnits) return launch_rb<TOK, false, 1, true>(a, s);
  }
  if (a.Esave) {
    if (a.out_dtype == 0)
      hipLaunchKernelGGL((ttt_linear_mfma_d64b16<PF, TOK, float, LN, true, RB>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((ttt_linear_mfma_d64b16<PF, TOK, uint16_t, LN, true, RB>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  if (a.out_dtype == 0)
    hipLaunchKernelGGL((ttt_linear_mfma_d64b16<PF, TOK, float, LN, false, RB>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_linear_mfma_d64b16<PF, TOK, uint16_t, LN, false, RB>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <bool TOK, bool LN>
hipError_t launch_eta(const LinearArgs& a, hipStream_t s) {
  if constexpr (LN) {
    return launch_rb<TOK, true, 1>(a, s);  // the layer norm runs with one row block
  } else {
    switch (a.rb) {
      case 4: return launch_rb<TOK, false, 4>(a, s);
      case 2: return launch_rb<TOK, false, 2>(a, s);
      default: return launch_rb<TOK, false, 1>(a, s);
    }
  }
}

template <bool TOK>
hipError_t launch_head_maps_eta(const LinearArgs& a, hipStream_t s) {
  dim3 grid(a.B * a.H * (a.nchunk - 1)), block(256);
  if (a.out_dtype == 0)
    hipLaunchKernelGGL((ttt_linear_mfma_head_maps<pf_for<1, true>(), TOK, float>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((ttt_linear_mfma_head_maps<pf_for<1, true>(), TOK, uint16_t>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool linear_mfma_supported(const LinearArgs& a) { return a.d == 64 && a.b == 16 && a.in_dtype == 1; }

const char* linear_mfma_name(const LinearArgs& a) {
  if (a.gamma) return "ttt_linear_mfma_d64b16 (layer norm)";
  return a.rb == 4 ? "ttt_linear_mfma_d64b16_r4" : a.rb == 2 ? "ttt_linear_mfma_d64b16_r2" : "ttt_linear_mfma_d64b16";
}

hipError_t launch_linear_mfma(const LinearArgs& a, hipStream_t s) {
  if (a.gamma) return a.est != 0 ? launch_eta<true, true>(a, s) : launch_eta<false, true>(a, s);
  return a.est != 0 ? launch_eta<true, false>(a, s) : launch_eta<false, false>(a, s);
}

hipError_t launch_linear_mfma_head_maps(const LinearArgs& a, hipStream_t s) {
  return a.est != 0 ? launch_head_maps_eta<true>(a, s) : launch_head_maps_eta<false>(a, s);
}

}  // namespace ttt
