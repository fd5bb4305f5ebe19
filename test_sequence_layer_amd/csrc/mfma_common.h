// Device helpers shared by the gfx950 matrix-core kernels of TTT-Linear
// (forward and backward): operand types, the bf16 hi + lo split of fp32
// values, transposing LDS column reads, streaming loads and stores, and
// sums within and across 16-lane rows.
//
// MFMA v_mfma_f32_16x16x32_bf16 lane layouts (lane l, li = l % 16, g = l / 16):
//   A operand  lane l holds A[m = li][k = 8g + j],  j = 0..7
//   B operand  lane l holds B[k = 8g + j][n = li]
//   D (accum.) lane l holds D[m = 4g + r][n = li],  r = 0..3
// An accumulator tile X (lane holds X[4g + r][li]) is therefore directly an
// A operand of X^T or a B operand of X once its 16-long row index is put on
// the contraction: slots j = 0..3 of lane group g take rows 4g + j, and
// slots 4..7 take the same rows again for a second split pass.
#pragma once

#include "ttt_common.h"

namespace ttt {
namespace mfma {

typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float float2v __attribute__((__vector_size__(2 * sizeof(float))));
typedef float float4v __attribute__((__vector_size__(4 * sizeof(float))));
typedef short short4v __attribute__((__vector_size__(4 * sizeof(short))));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float4v mfma32(bf16x8 a, bf16x8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Column read of a row-major bf16 tile with row stride RS elements: lane l gets
// X[row0 + 4(l/16) + r][col0 + l%16] for r = 0..3.  ds_read_b64_tr_b16 works on
// blocks of 16 lanes: output lane i receives element r from the 8-byte chunk
// addressed by lane 4r + i/4 of its block, position i%4; so lane j of block g
// addresses row row0 + 4g + j/4, columns col0 + 4(j%4) .. +3.
template <int RS>
__device__ __forceinline__ bf16x4 read_cols(const uint16_t* tile, int row0, int col0, int li, int g) {
  const uint16_t* p = tile + (row0 + 4 * g + (li >> 2)) * RS + col0 + 4 * (li & 3);
  typedef short4v __attribute__((address_space(3))) * lds_short4v_ptr;
  const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v_ptr)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// Two fp32 values -> packed bf16 hi pair and lo pair, x ~= hi + lo.  One
// v_cvt_pk_bf16_f32 rounds both hi values (nearest even); they are widened back
// with a shift and a mask, and the exact residuals are rounded into lo.
// Rounding is symmetric, so the split of -x is exactly -hi, -lo.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const bf16x2 h = __builtin_convertvector(float2v{x0, x1}, bf16x2);
  hi = __builtin_bit_cast(uint32_t, h);
  const float h0 = __uint_as_float(hi << 16);
  const float h1 = __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{x0 - h0, x1 - h1}, bf16x2));
}

__device__ __forceinline__ void split4(const float x[4], bf16x4& hi, bf16x4& lo) {
  uint32_t h[2], l[2];
  split2(x[0], x[1], h[0], l[0]);
  split2(x[2], x[3], h[1], l[1]);
  hi = __builtin_bit_cast(bf16x4, h);
  lo = __builtin_bit_cast(bf16x4, l);
}

__device__ __forceinline__ void split4(float4v x, bf16x4& hi, bf16x4& lo) {
  const float v[4] = {x[0], x[1], x[2], x[3]};
  split4(v, hi, lo);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

#ifndef TTT_LINEAR_NT
#define TTT_LINEAR_NT 1
#endif
// Streams touched exactly once are marked non-temporal so they do not evict
// each other from the caches.
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
  if constexpr (TTT_LINEAR_NT) {
    return __builtin_nontemporal_load(p);
  } else {
    return *p;
  }
}
template <typename T>
__device__ __forceinline__ void st_stream(T* p, T x) {
  if constexpr (TTT_LINEAR_NT) {
    __builtin_nontemporal_store(x, p);
  } else {
    *p = x;
  }
}

// fp32 value to an fp32 or bf16 output element
template <typename OutT>
__device__ __forceinline__ void store_out(OutT* p, float x);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float x) { st_stream(p, x); }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float x) { st_stream(p, f32_to_bf16_bits(x)); }

// The same through the L2 (no non-temporal hint): outputs written as partial
// lines by several waves merge there before they reach HBM, where non-temporal
// partial-line stores were measured to cost 22% extra write traffic.
template <typename OutT>
__device__ __forceinline__ void store_merged(OutT* p, float x);
template <>
__device__ __forceinline__ void store_merged<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store_merged<uint16_t>(uint16_t* p, float x) { *p = f32_to_bf16_bits(x); }

// Data-parallel-primitive (DPP) lane moves inside a 16-lane row: quad_perm
// [1,0,3,2] and [2,3,0,1] exchange neighbours 1 and 2 apart; row_half_mirror
// (lane i <-> 7 - i within 8) and row_mirror (i <-> 15 - i) then fold the
// quads, so after four adds every lane of the row holds the row's sum.
// (Every source lane of these patterns lies in the row, so no lane keeps an old
// value and the move needs no zeroed destination.)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float sum16(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

// Sums across the 16-lane rows: v_permlane16_swap with both operands x
// returns x of the two rows of a pair (rows 0, 1 and rows 2, 3), and
// v_permlane32_swap x of the two halves of the wave, so each pair's sum is the
// same in every lane of it.
__device__ __forceinline__ float sum_row_pairs(float x) {  // rows 2p and 2p + 1
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_rows(float x) {  // all four rows
  x = sum_row_pairs(x);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// dZ tile loads: 4 elements per thread per mini-batch, widened to fp32
template <typename GT>
struct GradLoad;
template <>
struct GradLoad<float> {
  typedef u32x4 type;
  __device__ static void get(type x, float v[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(x[i]);
  }
};
template <>
struct GradLoad<uint16_t> {
  typedef u32x2 type;
  __device__ static void get(type x, float v[4]) {
    v[0] = __uint_as_float(x[0] << 16);
    v[1] = __uint_as_float(x[0] & 0xffff0000u);
    v[2] = __uint_as_float(x[1] << 16);
    v[3] = __uint_as_float(x[1] & 0xffff0000u);
  }
};

__device__ __forceinline__ float4v zero4v() { return float4v{0.f, 0.f, 0.f, 0.f}; }

// Raw bits of element r of a bf16x4, taken from its two 32-bit words.  (Stores
// of bit-cast __bf16 vector elements were compiled as stores of element 0 for
// every r; the word arithmetic avoids that path.)
__device__ __forceinline__ uint16_t bf16_bits(bf16x4 x, int r) {
  const u32x2 w = __builtin_bit_cast(u32x2, x);
  const uint32_t v = w[r >> 1];
  return static_cast<uint16_t>((r & 1) ? (v >> 16) : (v & 0xffffu));
}

__device__ __forceinline__ void put4(uint16_t* tile, int off, bf16x4 x) {
  *reinterpret_cast<bf16x4*>(tile + off) = x;
}

// Row li of a bf16 tile (row stride RS elements) in the row-contraction order:
// block b holds columns 16b + 4g .. 16b + 4g + 3 (the order of an F2 state's rows).
template <int RS>
__device__ __forceinline__ void rows4(const uint16_t* tile, int li, int g, bf16x4 x[4]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) x[b] = *reinterpret_cast<const bf16x4*>(tile + li * RS + 16 * b + 4 * g);
}

// The backward kernels keep a d x d state in two layouts: F1 (row-owned: wave w
// holds rows 16w..16w+15 as accumulator tiles x[a][r] = X[16w + li][16a + 4g + r])
// and F2 (column-owned: x[b][r] = X[16b + 4g + r][16w + li]).
// 64-deep contraction over the rows of an F2 state: acc += X[m = li][:] . F2[:][n = li]
// with X given as split rows (rows4) and the state tiles pre-split; three passes.
__device__ __forceinline__ float4v rows_x_f2(const bf16x4 xh[4], const bf16x4 xl[4], const bf16x4 sh[4],
                                             const bf16x4 sl[4], float4v acc) {
#pragma unroll
  for (int p = 0; p < 4; p += 2) {
    const bf16x8 ah = cat(xh[p], xh[p + 1]), al = cat(xl[p], xl[p + 1]);
    const bf16x8 bh = cat(sh[p], sh[p + 1]), bl = cat(sl[p], sl[p + 1]);
    acc = mfma32(ah, bh, acc);
    acc = mfma32(ah, bl, acc);
    acc = mfma32(al, bh, acc);
  }
  return acc;
}

}  // namespace mfma
}  // namespace ttt
