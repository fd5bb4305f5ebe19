// Chunk start states of a chunked TTT-Linear forward.
//
// Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer"
// (aharts.cn / itmax.cn), part 03 §6-§7.  Each mini-batch of TTT-Linear maps the
// state affinely, W -> W (I - 2 K diag(eta) K^T) + 2 V diag(eta) K^T, so a chunk
// of mini-batches maps it as W -> W P + R.  With the maps P_c, R_c of every
// chunk but the last (computed in parallel by the MFMA kernel in its map
// mode), the start state of chunk c+1 is Wstart[c] P_c + R_c; this kernel runs
// that short sequential scan per chain (fp32 FMA, the maps staged in LDS and
// fetched one chunk ahead), after which every chunk's outputs are computed in
// parallel from its start state.
#include "ttt_internal.h"

namespace ttt {
namespace {

constexpr int D = 64;
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void ttt_linear_chunk_scan(LinearArgs a) {
  __shared__ float W[D][D + 1];
  __shared__ float P[D][D + 1];
  const int tid = threadIdx.x;
  const int chain = blockIdx.x;
  const int bi = chain / a.H, h = chain - bi * a.H;
  const float* w0 = a.W0 + bi * a.w0_bstride + static_cast<int64_t>(h) * D * D;
  float* ws = a.Wstart + static_cast<int64_t>(chain) * a.nchunk * D * D;
  for (int x = tid; x < D * D; x += kThreads) {
    const float v = w0[x];
    W[x / D][x % D] = v;
    ws[x] = v;
  }
  // Thread tid owns outputs W'[i][j0 .. j0 + 15] and stages the same 16 entries
  // of P; the next chunk's P and R entries are loaded one step ahead so their
  // latency overlaps the current product.
  const int i = tid >> 2, j0 = (tid & 3) * 16;
  const float* maps = a.maps + static_cast<int64_t>(chain) * (a.nchunk - 1) * 2 * D * D;
  float4 pn[4], rn[4];
  auto load_maps = [&](int c) {
    const float* Pg = maps + static_cast<int64_t>(c) * 2 * D * D + i * D + j0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pn[q] = *reinterpret_cast<const float4*>(Pg + 4 * q);
      rn[q] = *reinterpret_cast<const float4*>(Pg + D * D + 4 * q);
    }
  };
  if (a.nchunk > 1) load_maps(0);
  for (int c = 0; c + 1 < a.nchunk; ++c) {
    __syncthreads();  // W complete, previous P consumed
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      P[i][j0 + 4 * q + 0] = pn[q].x;
      P[i][j0 + 4 * q + 1] = pn[q].y;
      P[i][j0 + 4 * q + 2] = pn[q].z;
      P[i][j0 + 4 * q + 3] = pn[q].w;
    }
    float acc[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[4 * q + 0] = rn[q].x;
      acc[4 * q + 1] = rn[q].y;
      acc[4 * q + 2] = rn[q].z;
      acc[4 * q + 3] = rn[q].w;
    }
    if (c + 2 < a.nchunk) load_maps(c + 1);
    __syncthreads();
    for (int k = 0; k < D; ++k) {
      const float wik = W[i][k];
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) acc[jj] = fmaf(wik, P[k][j0 + jj], acc[jj]);
    }
    __syncthreads();  // every read of W done
    float* out = ws + static_cast<int64_t>(c + 1) * D * D + i * D + j0;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) W[i][j0 + jj] = acc[jj];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(out + 4 * q) = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
  }
}

}  // namespace

hipError_t launch_linear_chunk_scan(const LinearArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(ttt_linear_chunk_scan, dim3(a.B * a.H), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
