/*
 * Achievable-peak measurements for gfx950 (MI355X), beside the published
 * peaks (HBM 8 TB/s; dense bf16 matrix 2.5 PFLOP/s; fp32 vector 157.3 TFLOP/s,
 * a rate that needs packed fp32 instructions -- one v_fma_f32 per lane per
 * clock gives half of it).  They let a roofline
 * fraction be stated against what the chip really sustains as well as against
 * its specification.  Both calls are asynchronous on `stream` (hipStream_t,
 * NULL = the default stream); the caller times them (e.g. with HIP events) and
 * owns every buffer.  Status codes are ttt_status (ttt.h); validation errors
 * return before any launch.
 */
#ifndef TTT_PEAKS_H
#define TTT_PEAKS_H

#include <stdint.h>

#include "ttt.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Copy `bytes` bytes from src to dst (device memory) with 16-byte
 * non-temporal loads and stores, grid-stride: the HBM streaming ceiling
 * (2 * bytes of traffic per call).  bytes must be a multiple of 16
 * (TTT_ERR_SHAPE), src and dst 16-byte aligned (TTT_ERR_ALIGN), non-NULL when
 * bytes > 0 (TTT_ERR_NULL) and non-overlapping (TTT_ERR_ALIAS).
 */
ttt_status ttt_peak_copy(const void* src, void* dst, int64_t bytes, void* stream);

/*
 * Matrix-core issue loop: `blocks` workgroups of 4 waves, each wave running 8
 * independent accumulator chains of `iters` v_mfma_f32_16x16x32_bf16 each
 * (ttt_peak_mfma_bf16_flops() flops in all).  The operands are small integers,
 * so the result is exact and checkable: lane l of the wave holds
 *   A[m = l%16][k = 8(l/16) + s] = ((l + s) mod 5) - 2,
 *   B[k = 8(l/16) + s][n = l%16] = ((3l + s) mod 7) - 3      (s = 0..7),
 * chain j starts from j, and thread t of block q writes the 4 floats
 *   out[4 (256 q + t) + r] = 8 * iters * (A B)[4((t%64)/16) + r][t%16]
 * (exact for iters <= 10000).  out: blocks * 1024 floats, 16-byte aligned.
 * blocks >= 1 and iters >= 0, else TTT_ERR_SHAPE.
 */
ttt_status ttt_peak_mfma_bf16(float* out, int32_t blocks, int32_t iters, void* stream);

/* Flops one ttt_peak_mfma_bf16(out, blocks, iters) call performs (-1 for bad arguments). */
int64_t ttt_peak_mfma_bf16_flops(int32_t blocks, int32_t iters);

/*
 * fp32 vector issue loop: `blocks` workgroups of 256 threads, each thread
 * running 16 independent chains of `iters` unpacked v_fma_f32
 * (acc_j <- acc_j * 1 + c, the 1 passed at run time), for
 * ttt_peak_valu_f32_flops() flops in all.  Chain j starts from j and
 * c = (t mod 4) for thread t, so thread t of block q writes the exact value
 *   out[256 q + t] = 120 + 16 * iters * (t mod 4).
 * out: blocks * 256 floats, 4-byte aligned.  blocks >= 1 and
 * 0 <= iters <= 300000 (the exactness bound), else TTT_ERR_SHAPE.
 */
ttt_status ttt_peak_valu_f32(float* out, int32_t blocks, int32_t iters, void* stream);

/* Flops one ttt_peak_valu_f32(out, blocks, iters) call performs (2 per fma; -1 for bad arguments). */
int64_t ttt_peak_valu_f32_flops(int32_t blocks, int32_t iters);

#ifdef __cplusplus
}
#endif

#endif /* TTT_PEAKS_H */
