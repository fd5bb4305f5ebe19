// TTT-Linear backward launches (plain f and f with the layer norm).
#pragma once
#include "ttt_common.h"

namespace ttt {

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

}  // namespace ttt
