// Chunk start states of a chunked TTT-Linear forward.
//
// Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
// (aharts.cn / itmax.cn), part 03 §6-§7.  Each mini-batch of TTT-Linear maps the
// state affinely, W -> W (I - 2 K diag(eta) K^T) + 2 V diag(eta) K^T, so a chunk
// of mini-batches maps it as W -> W P + R.  The first pass of a chunked forward
// runs chunk 0 from W0 (so the start state of chunk 1 is known) and computes
// the maps P_c, R_c of chunks 1 .. n-2 in parallel; the start state of chunk
// c+1 is then Wstart[c] P_c + R_c, and this kernel runs that short sequential
// scan per chain, after which chunks 1 .. n-1 are computed in parallel from
// their start states.  Each 64 x 64 x 64 product runs on
// the fp32 matrix cores (v_mfma_f32_16x16x4_f32: fp32 products and sums, no
// bf16 splitting): wave w computes rows 16w .. 16w + 15 of W P + R, the four
// 16 x 16 column tiles accumulating over k in steps of 4.
#include "args_linear.h"

namespace ttt {
namespace {

constexpr int D = 64;
constexpr int kThreads = 256;
typedef float float4v __attribute__((__vector_size__(4 * sizeof(float))));

__global__ __launch_bounds__(kThreads) void ttt_linear_chunk_scan(LinearArgs a) {
  // row strides chosen so that the operand reads (16 rows x 4 columns of W,
  // 4 rows x 16 columns of P per instruction) hit 64 distinct banks
  __shared__ float W[D][D + 4];
  __shared__ float P[D][D + 16];
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int chain = blockIdx.x;
  // ws[c - 1]: start state of chunk c = 1 .. n-1; ws[0] was written by the first pass
  float* ws = a.Wstart + static_cast<int64_t>(chain) * (a.nchunk - 1) * D * D;
  for (int x = tid; x < D * D; x += kThreads) W[x / D][x % D] = ws[x];
  // This thread stages row pr, columns pc .. pc + 15 of the next P, and holds
  // R in the accumulator layout: acc[b][r] = R[16w + 4g + r][16b + li].  Both
  // are loaded one chunk ahead so their latency overlaps the current product.
  const int pr = tid >> 2, pc = (tid & 3) * 16;
  // maps[c - 1]: P, R of chunk c = 1 .. n-2
  const float* maps = a.maps + static_cast<int64_t>(chain) * (a.nchunk - 2) * 2 * D * D;
  float4 pn[4];
  float4v rn[4];
  auto load_maps = [&](int c) {
    const float* Pg = maps + static_cast<int64_t>(c) * 2 * D * D;
#pragma unroll
    for (int q = 0; q < 4; ++q) pn[q] = *reinterpret_cast<const float4*>(Pg + pr * D + pc + 4 * q);
    const float* Rg = Pg + D * D + (16 * w + 4 * g) * D + li;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) rn[b][r] = Rg[r * D + 16 * b];
  };
  if (a.nchunk > 2) load_maps(0);
  for (int c = 0; c + 2 < a.nchunk; ++c) {  // chunk c + 1's map: Wstart of chunk c + 2
    __syncthreads();  // W complete, previous P consumed
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<float4*>(&P[pr][pc + 4 * q]) = pn[q];
    float4v acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = rn[b];
    if (c + 3 < a.nchunk) load_maps(c + 1);
    __syncthreads();
    // acc[b] += W[16w + m][k] P[k][16b + n]: A operand W[16w + li][k0 + g],
    // B operand P[k0 + g][16b + li], k0 = 0, 4, ..., 60
#pragma unroll 4
    for (int k0 = 0; k0 < D; k0 += 4) {
      const float av = W[16 * w + li][k0 + g];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, P[k0 + g][16 * b + li], acc[b], 0, 0, 0);
    }
    __syncthreads();  // every read of W done
    float* out = ws + static_cast<int64_t>(c + 1) * D * D;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        W[16 * w + 4 * g + r][16 * b + li] = acc[b][r];
        out[(16 * w + 4 * g + r) * D + 16 * b + li] = acc[b][r];
      }
  }
}

}  // namespace

hipError_t launch_linear_chunk_scan(const LinearArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(ttt_linear_chunk_scan, dim3(a.B * a.H), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
