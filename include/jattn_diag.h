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

/* The memory traffic a key-parallel backward would need to accumulate dQ across key blocks, without
 * any of the attention arithmetic: `pairs` (batch, head) pairs of L query rows and D columns (D a
 * multiple of 4, at most 128), `nkb` key blocks per pair, each block contributing one fp32 value per
 * (query row, column), in 64-row query tiles.
 *   JATTN_PROBE_DQ_ATOMIC   pairs * nkb workgroups add their values into acc[pairs][L][D] with
 *                           hardware fp32 atomic adds (acc must start at zero for a meaningful sum);
 *   JATTN_PROBE_DQ_PARTIAL  the same workgroups store their values to acc[nkb][pairs][L][D];
 *   JATTN_PROBE_DQ_REDUCE   sums acc[nkb][pairs][L][D] over the key blocks into
 *                           acc[nkb * pairs * L * D ...] (the pass that finishes the partial scheme).
 * Every value added or stored is 1.0, so after ATOMIC each element of acc equals nkb.
 *   acc, acc_bytes  device fp32 buffer and its size: at least pairs*L*D*4 bytes (ATOMIC),
 *                   nkb*pairs*L*D*4 (PARTIAL), (nkb + 1)*pairs*L*D*4 (REDUCE); 16-byte aligned.
 * Errors: INVALID_VALUE for an unknown mode, sizes < 1, D not a multiple of 4 or > 128, nkb > 64,
 * element counts >= 2^31, or a null, misaligned or too small acc; HIP if the launch fails. */
#define JATTN_PROBE_DQ_ATOMIC 0
#define JATTN_PROBE_DQ_PARTIAL 1
#define JATTN_PROBE_DQ_REDUCE 2
jattn_status jattn_probe_dq_accumulation(int mode, int pairs, int L, int D, int nkb, float* acc, size_t acc_bytes,
                                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* JATTN_DIAG_H */
