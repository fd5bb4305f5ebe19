// TTT-Linear forward launches (dual form, matrix-core, portable and chunked kernels).
#pragma once
#include "ttt_common.h"

namespace ttt {

// Everything a TTT-Linear launch needs, validated on the host.
struct LinearArgs {
  int B, H, T, d, b;
  int in_dtype, out_dtype;  // 0 = fp32, 1 = bf16
  const void* Q;
  const void* K;
  const void* V;
  const float* W0;
  int64_t w0_bstride;  // elements between sequences' W0 (0 = shared)
  const float* eta;
  int64_t esb, esh, est;  // eta strides (elements)
  void* Z;
  float* Wf;
  // Chunked execution: the sequence's nb = T / 16 mini-batches are split into
  // nchunk chunks: chunk 0 holds mb1 of them, and chunk c >= 1 starts at
  // mini-batch mb1 + (c - 1) (nb - mb1) / (nchunk - 1)
  // (nchunk = 1, Wstart = maps = nullptr for a plain forward).
  int nchunk;
  int64_t mb1;
  float* Wstart;        // [chains][nchunk-1][d][d] start states of chunks 1 .. nchunk-1
  float* maps;          // [chains][nchunk-2][2][d][d] maps (P, R) of chunks 1 .. nchunk-2
  // Layer norm and residual inside f (f(x) = x + LN(W x)); gamma == nullptr: plain f(x) = W x.
  const float* gamma;   // [H][d]
  const float* beta;    // [H][d]
  float eps;
  // Forward for training: also write E[t] = W_{mini-batch start} k_t - v_t
  // (with the layer norm: the update factor G[t] = -eta_t delta_t as applied)
  // ([chains][T][d] fp32) for the backward; nullptr: not saved.
  float* Esave;
  // MFMA forward: workgroups (row blocks of 64 / rb rows of W) per
  // (sequence, head, chunk); 1, 2 or 4 (1 with a layer norm).
  int rb;
};

// Portable fp32 kernel (any supported d/b/dtype).
bool linear_generic_supported(int d, int b);
const char* linear_generic_name(int d);
hipError_t launch_linear_generic(const LinearArgs& a, hipStream_t s);

// MFMA kernel: d = 64, b = 16, bf16 Q/K/V.
bool linear_mfma_supported(const LinearArgs& a);
const char* linear_mfma_name(const LinearArgs& a);
hipError_t launch_linear_mfma(const LinearArgs& a, hipStream_t s);
// MFMA kernel for fp32 Q/K/V: d = 64, b = 16, plain forward (no layer norm, no
// saved E, not chunked).
bool linear_mfma_f32_supported(const LinearArgs& a);
hipError_t launch_linear_mfma_f32(const LinearArgs& a, hipStream_t s);
// First pass of a chunked forward: for every chain, the forward of chunk 0
// from W0 (its Z, and its end state = the start state of chunk 1), and the
// maps of chunks 1 .. nchunk-2: P = the product of the chunk's
// (I - 2 K diag(eta) K^T) and R = the state the chunk reaches from zero, so
// that W_end = W_start P + R.
hipError_t launch_linear_mfma_head_maps(const LinearArgs& a, hipStream_t s);
// Chunk start states: Wstart of chunk c+1 = (that of chunk c) P_c + R_c, c = 1 .. nchunk-2.
hipError_t launch_linear_chunk_scan(const LinearArgs& a, hipStream_t s);

}  // namespace ttt
