// GELU for the TTT-MLP kernels: the exact erf definition GELU(x) = x Phi(x)
// ([TTT] news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，一夜推翻Transformer",
// part 03 §9: the MLP of TTT-MLP uses GELU) and its derivative.
#pragma once

#include <hip/hip_runtime.h>

namespace ttt {

// GELU(x) = x Phi(x) and GELU'(x) = Phi(x) + x phi(x), exact erf form, with one
// erff per pre-activation shared by both.
__device__ __forceinline__ float gelu(float x) { return 0.5f * x * (1.f + erff(x * 0.70710678118654752f)); }
__device__ __forceinline__ void gelu_and_prime(float x, float& g, float& gp) {
  const float cdf = 0.5f * (1.f + erff(x * 0.70710678118654752f));
  g = x * cdf;
  // phi(x) = exp(-x^2 / 2) / sqrt(2 pi), as 2^(-x^2 log2(e) / 2) on the hardware exponential
  gp = cdf + x * 0.39894228040143268f * __builtin_amdgcn_exp2f(x * x * -0.72134752044448170f);
}

// Phi(x) = 0.5 + x Q(x^2) for x^2 < 2, Q of degree 5: the standard normal CDF
// from a polynomial fit of erf(z) / z in z^2 on |z| <= 1 (z = x / sqrt 2; a
// least-squares fit reweighted toward equal relative error, coefficients
// then scaled for x).  Measured in fp32 against the exact CDF over x^2 < 2:
// absolute error <= 1e-7, GELU relative error <= 1e-6.
__device__ __forceinline__ float phi_poly(float x, float u) {
  float q = -0x1.a0c4c4p-18f;
  q = fmaf(q, u, 0x1.c78590p-14f);
  q = fmaf(q, u, -0x1.356de2p-10f);
  q = fmaf(q, u, 0x1.46b4d2p-7f);
  q = fmaf(q, u, -0x1.10579cp-4f);
  q = fmaf(q, u, 0x1.988452p-2f);
  return fmaf(x, q, 0.5f);
}

// GELU (and GELU') of 8 pre-activations of a lane.  While every |x| in the
// wave is below sqrt 2 (the usual case: the pre-activations are small) the
// CDF comes from phi_poly with no per-value branch; otherwise all 8 take the
// library erff.  The test is wave-uniform, so the branch never diverges.
template <bool PRIME>
__device__ __forceinline__ void gelu8(const float x[8], float g[8], float gp[8]) {
  bool big = false;
#pragma unroll
  for (int k = 0; k < 8; ++k) big |= !(x[k] * x[k] < 2.f);
  if (__builtin_amdgcn_ballot_w64(big) == 0) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float u = x[k] * x[k];
      const float cdf = phi_poly(x[k], u);
      g[k] = x[k] * cdf;
      if constexpr (PRIME) gp[k] = fmaf(x[k] * 0.39894228040143268f, __builtin_amdgcn_exp2f(u * -0.72134752044448170f), cdf);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if constexpr (PRIME) {
        gelu_and_prime(x[k], g[k], gp[k]);
      } else {
        g[k] = gelu(x[k]);
      }
    }
  }
}

}  // namespace ttt
