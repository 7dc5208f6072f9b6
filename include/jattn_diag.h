/*
 * jattn_diag.h -- C ABI of libjattn.so, part 4: measurement support. Not part of the attention or
 * projection math.
 *
 * Hardware busy counters (the SQ block's MFMA-busy and VALU-issue cycles) have no documented
 * full-scale value per GPU, clock and counter-aggregation mode. The probe kernels here keep one pipe
 * of every SIMD saturated for a known number of instructions, so a counter run that includes them
 * reads the full-scale value of those counters on the same GPU in the same run, and any other
 * kernel's busy fraction is its reading divided by the probe's.
 *
 * Conventions as in jattn.h: device pointers, asynchronous on `stream`, no allocation, host-side
 * checks before any HIP call.
 */
#ifndef JATTN_DIAG_H
#define JATTN_DIAG_H

#include "jattn.h"

#ifdef __cplusplus
extern "C" {
#endif

#define JATTN_PROBE_MFMA 0 /* only v_mfma_f32_32x32x16_bf16, four independent accumulators per wave */
#define JATTN_PROBE_FMA 1  /* only fp32 FMAs, sixteen independent chains per lane                   */

/* Run probe `which` on `blocks` workgroups of 256 threads (4 waves), each wave looping `iters`
 * times over 64 MFMAs (MFMA probe) or 128 FMAs (FMA probe) on register data derived from `seed`.
 *   out   device fp32 [blocks * 256]: one value per thread (keeps the work live), overwritten.
 * Errors: INVALID_VALUE for an unknown probe, blocks < 1, iters < 1, blocks * 256 >= 2^31 or a
 * null or misaligned out; HIP if the launch fails. */
jattn_status jattn_probe_saturate(int which, int blocks, int iters, float seed, float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* JATTN_DIAG_H */
