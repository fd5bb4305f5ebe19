// Shared by every kernel of libttt.so: bf16 <-> fp32 on raw bits (the library
// stores bf16 as uint16_t).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, h);
}

}  // namespace ttt
