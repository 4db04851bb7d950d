/*
 * kda_calib.h -- calibration kernels shipped with the KDA library.
 *
 * They compute nothing of the method.  A benchmark runs them in the same
 * process as the method's kernels to measure what this GPU actually reaches:
 * the HBM rate of a plain copy and the dense rate of two bf16 matrix-core
 * instructions.  Against those, the method's kernels are placed as a fraction
 * of the achievable, beside the fraction of the vendor's peak figures.
 *
 * Both calls are asynchronous on `stream` (a hipStream_t, NULL = the null
 * stream) and return 0 on success, 2 for invalid arguments (nothing launched)
 * or 5 when the launch fails.
 */
#ifndef KDA_CALIB_H
#define KDA_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Copy `bytes` bytes (a multiple of 16) from src to dst, both 16-byte aligned
 * DEVICE pointers that do not overlap, with 16-byte non-temporal loads and
 * stores; reads and writes each byte once.
 */
int kda_calib_copy(const void* src, void* dst, size_t bytes, void* stream);

/*
 * Dense matrix-core loop: `blocks` workgroups of four waves, each wave
 * issuing 4 * iters matrix instructions on four independent accumulators;
 * kind 0 = v_mfma_f32_16x16x32_bf16 (16384 flops each), kind 1 =
 * v_mfma_f32_32x32x16_bf16 (32768 flops each).  One float per thread is
 * written to out (blocks * 256 floats, DEVICE) so the loop is not dead code.
 */
int kda_calib_mfma(float* out, int blocks, int64_t iters, int kind, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_CALIB_H */
