// TTT-MLP dual-form launches.
#pragma once
#include "ttt_common.h"

namespace ttt {

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
  // Checkpoint mode (the first pass of the backward): the state at every
  // mini-batch start is written to ckpt ([B*H][T/b][W1 dh x d, W2 d x dh],
  // row-major fp32) and nothing else is written (Z, W1f, W2f unused).
  float* ckpt;
};

// TTT-MLP kernel: d = 64, dh = 256, b = 16, bf16 Q/K/V.
bool mlp_supported(const MlpArgs& a);
const char* mlp_name(const MlpArgs& a);
hipError_t launch_mlp(const MlpArgs& a, hipStream_t s);
// The same kernel in checkpoint mode (plain f, a.ckpt set).
hipError_t launch_mlp_ckpt(const MlpArgs& a, hipStream_t s);

}  // namespace ttt
