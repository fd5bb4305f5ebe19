// Primal-form (token by token) launches: TTT-Linear and TTT-MLP, full forward and decode.
#pragma once
#include "ttt_common.h"

namespace ttt {

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

}  // namespace ttt
