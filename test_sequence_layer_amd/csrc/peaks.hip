// Achievable-peak microbenchmarks (contracts in include/ttt_peaks.h): an HBM
// copy with 16-byte non-temporal accesses, a bf16 matrix-core issue loop of
// independent v_mfma_f32_16x16x32_bf16 chains, and an fp32 vector loop of
// independent v_fma_f32 chains (unpacked: the library is built without packed
// fp32 instructions, so this is the vector rate its fp32 kernels can reach).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ttt_peaks.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float float4v __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kThreads = 256;
constexpr int kChains = 8;  // independent accumulators per wave: enough to keep the matrix pipe busy
constexpr int64_t kFlopsPerMfma = 2 * 16 * 16 * 32;
constexpr int kValuChains = 16;  // independent fma chains per thread: covers the dependent-issue latency
constexpr int kValuMaxIters = 300000;  // keeps the sum of the chains below 2^24 (exact)

__global__ __launch_bounds__(kThreads) void peak_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                             int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(kThreads) void peak_mfma_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    a[s] = static_cast<__bf16>(static_cast<float>((lane + s) % 5 - 2));
    b[s] = static_cast<__bf16>(static_cast<float>((3 * lane + s) % 7 - 3));
  }
  // distinct starting values keep the chains from being merged into one
  float4v acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = float4v{float(j), float(j), float(j), float(j)};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float4v sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kChains; ++j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sum[r] += acc[j][r] - float(j);
  }
  *reinterpret_cast<float4v*>(out + (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * 4) = sum;
}

// acc_j <- acc_j * x + c with x = 1 at run time (so nothing folds): every
// value is an integer below 2^24, so the result is exact and checkable.
__global__ __launch_bounds__(kThreads) void peak_valu_kernel(float* __restrict__ out, float x, int iters) {
  const float c = static_cast<float>(threadIdx.x & 3);
  float acc[kValuChains];
#pragma unroll
  for (int j = 0; j < kValuChains; ++j) acc[j] = static_cast<float>(j);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kValuChains; ++j) acc[j] = fmaf(acc[j], x, c);
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < kValuChains; ++j) sum += acc[j];
  out[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = sum;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" ttt_status ttt_peak_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return TTT_ERR_SHAPE;
  if (bytes == 0) return TTT_OK;
  if (!src || !dst) return TTT_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return TTT_ERR_ALIGN;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 < d0 + static_cast<uintptr_t>(bytes) && d0 < s0 + static_cast<uintptr_t>(bytes)) return TTT_ERR_ALIAS;
  const int64_t n = bytes / 16;
  int64_t grid = (n + kThreads - 1) / kThreads;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(peak_copy_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
  return hipGetLastError() == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

extern "C" int64_t ttt_peak_mfma_bf16_flops(int32_t blocks, int32_t iters) {
  if (blocks < 1 || iters < 0) return -1;
  return static_cast<int64_t>(blocks) * (kThreads / 64) * iters * kChains * kFlopsPerMfma;
}

extern "C" ttt_status ttt_peak_mfma_bf16(float* out, int32_t blocks, int32_t iters, void* stream) {
  if (blocks < 1 || iters < 0) return TTT_ERR_SHAPE;
  if (!out) return TTT_ERR_NULL;
  if (!aligned16(out)) return TTT_ERR_ALIGN;
  hipLaunchKernelGGL(peak_mfma_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), out, static_cast<int>(iters));
  return hipGetLastError() == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

extern "C" int64_t ttt_peak_valu_f32_flops(int32_t blocks, int32_t iters) {
  if (blocks < 1 || iters < 0) return -1;
  return static_cast<int64_t>(blocks) * kThreads * iters * kValuChains * 2;
}

extern "C" ttt_status ttt_peak_valu_f32(float* out, int32_t blocks, int32_t iters, void* stream) {
  if (blocks < 1 || iters < 0 || iters > kValuMaxIters) return TTT_ERR_SHAPE;
  if (!out) return TTT_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(out) & 3) != 0) return TTT_ERR_ALIGN;
  hipLaunchKernelGGL(peak_valu_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), out, 1.0f, static_cast<int>(iters));
  return hipGetLastError() == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}
