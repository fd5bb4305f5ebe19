// Issue priority of a wave (s_setprio) for the matrix-core kernels.
//
// Two waves share each SIMD in these kernels, and both walk the same sequence
// of phases, so they tend to reach their matrix-core runs and their vector
// runs (splits into bf16 hi + lo, activations, masks) at the same time.  A
// wave raises its priority for a run of matrix-core instructions and drops it
// afterwards: when both waves have an instruction ready, the one feeding the
// matrix cores issues first, and the other wave's vector instructions fill the
// cycles the matrix cores are busy.  Only the order of issue changes, never a
// result (the kernels are bit-identical with and without it).
#pragma once

#include <hip/hip_runtime.h>

namespace ttt {

__device__ __forceinline__ void prio_mfma() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void prio_valu() { __builtin_amdgcn_s_setprio(0); }

}  // namespace ttt
