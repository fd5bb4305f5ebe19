// TTT-MLP backward launches (primal form, token by token in reverse).
#pragma once
#include "ttt_common.h"

namespace ttt {

// Backward of TTT-MLP (f(x) = W2 GELU(W1 x)) from the inputs and the initial
// state; the mini-batch-start states are written to the workspace by a
// forward pass in the same launch and read back in reverse order.
struct MlpBwdArgs {
  int B, H, T, d, dh, b;
  int in_dtype;            // Q, K, V: 0 fp32, 1 bf16 (dZ and every output fp32)
  const void* Q;
  const void* K;
  const void* V;
  const float* W1_in;      // [H or B*H, dh, d]
  const float* W2_in;      // [H or B*H, d, dh]
  int64_t w_in_bstride;    // elements between sequences' initial states (0: shared over B)
  const float* eta;
  int64_t esb, esh, est;
  const float* dZ;         // [B, H, T, d]
  const float* dW1f;       // [B, H, dh, d] or nullptr (zero)
  const float* dW2f;       // [B, H, d, dh] or nullptr (zero)
  float* ws;               // [B*H][ceil(T/b)][2][dh*d]
  float* dQ;
  float* dK;
  float* dV;               // [B, H, T, d]
  float* deta;             // [B, H, T]
  float* dW1;              // [B, H, dh, d]
  float* dW2;              // [B, H, d, dh]
  // Layer norm and residual inside f (f(x) = x + LN(W2 GELU(W1 x))); gamma ==
  // nullptr: plain f.  Primal form only.
  const float* gamma;      // [H][d]
  const float* beta;       // [H][d]
  float eps;
  float* dgamma;           // [B, H, d]
  float* dbeta;            // [B, H, d]
};
// Primal form (token by token, fp32 vector units): d = 64, dh = 256, b <= 16,
// any T, fp32 or bf16 inputs; the workspace holds the mini-batch-start states.
// With a.gamma set, f carries the layer norm and residual.
bool mlp_bwd_supported(int d, int dh, int b);
hipError_t launch_mlp_bwd(const MlpBwdArgs& a, hipStream_t s);
// Dual form on the matrix cores: d = 64, dh = 256, b = 16, T % 16 == 0, bf16
// inputs.  The states come from the forward kernel in checkpoint mode, which
// the caller launches first with the same workspace.
bool mlp_bwd_mfma_supported(int d, int dh, int b, int in_dtype, int T);
hipError_t launch_mlp_bwd_mfma(const MlpBwdArgs& a, hipStream_t s);

}  // namespace ttt
