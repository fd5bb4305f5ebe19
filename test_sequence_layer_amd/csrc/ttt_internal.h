// Internal declarations of libttt.so (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Backward of TTT-Linear (plain f(x) = W x) from the saved E and the final state.
struct BwdArgs {
  int B, H, T, d, b;
  int in_dtype, out_dtype;   // Q/K dtype; dZ and dQ/dK/dV dtype
  const void* Q;
  const void* K;
  const float* eta;
  int64_t esb, esh, est;
  const float* Wf;           // [chains][d][d] state after the last mini-batch
  const float* E;            // [chains][T][d] saved by the forward
  const void* dZ;            // [chains][T][d]
  const float* dWf;          // [chains][d][d] or nullptr (zero)
  void* dQ;
  void* dK;
  void* dV;
  float* deta;               // [chains][T]
  float* dW0;                // [chains][d][d]
  // Layer norm and residual inside f (gamma != nullptr): E holds the saved
  // update factors G = -eta delta (delta the loss gradient at W k) as the
  // forward applied them, V the values; the gradients of the per-head scale
  // and shift come out per chain.
  const void* V;             // [chains][T][d] in_dtype
  const float* gamma;        // [H][d]
  const float* beta;         // [H][d]
  float eps;
  float* dgamma;             // [chains][d]
  float* dbeta;              // [chains][d]
};
bool linear_bwd_mfma_supported(const BwdArgs& a);
hipError_t launch_linear_bwd_mfma(const BwdArgs& a, hipStream_t s);
bool linear_bwd_generic_supported(int d, int b);
const char* linear_bwd_generic_name(int d);
hipError_t launch_linear_bwd_generic(const BwdArgs& a, hipStream_t s);
// Backward of TTT-Linear with the layer norm: d = 64, b = 16, bf16 inputs; the
// matrix-core kernel and the fp32 one (the cross-check).
bool linear_ln_bwd_supported(const BwdArgs& a);
hipError_t launch_linear_ln_bwd(const BwdArgs& a, hipStream_t s);
hipError_t launch_linear_ln_bwd_mfma(const BwdArgs& a, hipStream_t s);

struct MlpArgs {
  int B, H, T, d, dh, b;
  int in_dtype, out_dtype;
  const void* Q;
  const void* K;
  const void* V;
  const float* W1;
  const float* W2;
  int64_t w_bstride;
  const float* eta;
  int64_t esb, esh, est;
  void* Z;
  float* W1f;
  float* W2f;
  // Layer norm and residual inside f (f(x) = x + LN(W2 GELU(W1 x))); gamma == nullptr: plain f.
  const float* gamma;   // [H][d]
  const float* beta;    // [H][d]
  float eps;
};

// Primal form (token by token): full forward and decode.
struct PrimalArgs {
  int B, H, T, d, b;
  int in_dtype, out_dtype;
  const void* Q;
  const void* K;
  const void* V;
  const float* W_in;   // state at position pos
  const float* Wb_in;  // mini-batch-start state at position pos
  int64_t w_in_bstride;
  const float* eta;
  int64_t esb, esh, est;
  void* Z;
  float* W_out;        // [B, H, d, d]
  float* Wb_out;       // [B, H, d, d] or nullptr
  int64_t pos;         // tokens already processed
  const float* gamma;  // [H, d] layer-norm scale, or nullptr for f(x) = W x
  const float* beta;   // [H, d] layer-norm shift (with gamma)
  float eps;
};
bool linear_primal_supported(int d);
const char* linear_primal_name(int d, bool ln = false);
hipError_t launch_linear_primal(const PrimalArgs& a, hipStream_t s);

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

// TTT-MLP primal form (token by token): full forward and decode, d = 64, dh = 256.
struct MlpPrimalArgs {
  int B, H, T, d, dh, b;
  int in_dtype, out_dtype;
  const void* Q;
  const void* K;
  const void* V;
  const float* W1_in;   // state at position pos: W1 [dh][d], W2 [d][dh]
  const float* W2_in;
  const float* W1b_in;  // mini-batch-start state at position pos
  const float* W2b_in;
  int64_t w_in_bstride; // elements between sequences' input states (0: shared over B)
  const float* eta;
  int64_t esb, esh, est;
  void* Z;
  float* W1_out;        // [B, H, dh, d]
  float* W2_out;        // [B, H, d, dh]
  float* W1b_out;       // [B, H, dh, d] or nullptr
  float* W2b_out;       // [B, H, d, dh] or nullptr
  int64_t pos;          // tokens already processed
  const float* gamma;   // [H, d] layer-norm scale, or nullptr for f(x) = W2 GELU(W1 x)
  const float* beta;    // [H, d] layer-norm shift (with gamma)
  float eps;
};
bool mlp_primal_supported(int d, int dh);
hipError_t launch_mlp_primal(const MlpPrimalArgs& a, hipStream_t s);

// TTT-MLP kernel: d = 64, dh = 256, b = 16, bf16 Q/K/V.
bool mlp_supported(const MlpArgs& a);
const char* mlp_name(const MlpArgs& a);
hipError_t launch_mlp(const MlpArgs& a, hipStream_t s);

// bf16 <-> fp32 on raw bits (the library stores bf16 as uint16_t).
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, h);
}

}  // namespace ttt
