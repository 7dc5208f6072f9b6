/*
 * jattn_diag.h -- C ABI of libjattn.so, part 4: measurement support. Not part of the attention or
 * projection math.
 *
 * Busy-counter calibration, a dQ-accumulation traffic probe, and probes of the dk/dv tile's
 * dependency structure, of LDS read rates and of the MFMA / VALU issue rates (the tile probes time
 * themselves with the shader clock).
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

/* The dk/dv tile's dependency structure at D = 64, without global loads: per 32-query half, 8 score
 * MFMAs (two chains of 4 k-steps, seeded with the rows' statistics), 16 exp2, 16 multiplies and 16
 * bf16 conversions, then 8 gradient MFMAs fed by transposed fragments; one 64-query tile (two halves)
 * per iteration, `iters` iterations per wave. `mode` selects which operands are read from LDS tiles
 * laid out like the kernel's (the rest come from registers):
 *   JATTN_PROBE_TILE_REGS          none;
 *   JATTN_PROBE_TILE_LDS           row fragments, statistics and transposed fragments, as in the kernel;
 *   JATTN_PROBE_TILE_LDS_BARRIER   the same with a workgroup barrier per tile;
 *   JATTN_PROBE_TILE_ROWS_STATS    row fragments and statistics;
 *   JATTN_PROBE_TILE_TRANSPOSED    transposed fragments;
 *   JATTN_PROBE_TILE_STATS         statistics;
 *   JATTN_PROBE_TILE_ROWS          row fragments;
 *   JATTN_PROBE_TILE_PIPELINED     as LDS, with the next half's statistics and rows read under the current
 *                                  half's softmax and gradient products.
 * `blocks` workgroups of 256 threads (4 waves) run it; blocks = (compute units) x (waves per SIMD).
 *   out     device fp32 [blocks * 256]: one value per thread (keeps the work live), overwritten;
 *   cycles  device uint64 [blocks * 4]: each wave's shader-clock cycles (s_memtime) over its loop.
 * Each iteration holds 32 MFMAs of 32x32x16 per wave: the MFMA pipe's busy fraction is
 * 1024 * iters * (waves per SIMD) / cycles.
 * Errors: INVALID_VALUE for an unknown mode, blocks < 1, iters < 1, blocks * 256 >= 2^31, or a null or
 * misaligned out or cycles; HIP if the launch fails. */
#define JATTN_PROBE_TILE_REGS 0
#define JATTN_PROBE_TILE_LDS 1
#define JATTN_PROBE_TILE_LDS_BARRIER 2
#define JATTN_PROBE_TILE_ROWS_STATS 3
#define JATTN_PROBE_TILE_TRANSPOSED 4
#define JATTN_PROBE_TILE_STATS 5
#define JATTN_PROBE_TILE_ROWS 6
#define JATTN_PROBE_TILE_PIPELINED 7
jattn_status jattn_probe_tile(int mode, int blocks, int iters, float seed, float* out, uint64_t* cycles,
                              hipStream_t stream);

/* LDS read rate: `blocks` workgroups of 256 threads each issue, per wave and iteration, 8 independent
 * reads of one kind and consume them together (`iters` iterations):
 *   JATTN_PROBE_LDS_B128            ds_read_b128, lane l at byte 16 l of a 1 KiB row (no bank conflicts);
 *   JATTN_PROBE_LDS_B128_BROADCAST  ds_read_b128, all lanes of a half-wave at one address;
 *   JATTN_PROBE_LDS_B64_TRANSPOSED  ds_read_b64_tr_b16, lane l at byte 8 l of a 512-byte row.
 *   cycles  device uint64 [blocks * 4]: each wave's shader-clock cycles over its loop.
 * Bytes returned per compute unit and cycle = 8 * iters * 64 * (16, 16 or 8) * (waves per CU) / cycles.
 * Errors: INVALID_VALUE for an unknown mode, blocks < 1, iters < 1, blocks * 256 >= 2^31, or a null or
 * misaligned cycles; HIP if the launch fails. */
#define JATTN_PROBE_LDS_B128 0
#define JATTN_PROBE_LDS_B128_BROADCAST 1
#define JATTN_PROBE_LDS_B64_TRANSPOSED 2
jattn_status jattn_probe_lds_read(int mode, int blocks, int iters, uint64_t* cycles, hipStream_t stream);

/* Issue rates of the matrix pipe, fp32 FMAs and exp2 (v_exp_f32), alone and together. `blocks`
 * workgroups of 512 threads (8 waves, two per SIMD: waves w and w + 4 share SIMD w % 4 as the waves of a
 * workgroup are placed in order) loop `iters` times over 8 steps each. Per wave and step:
 *   JATTN_PROBE_ISSUE_MFMA       one v_mfma_f32_32x32x16_bf16 (four independent accumulators in turn);
 *   JATTN_PROBE_ISSUE_FMA        16 fp32 FMAs (eight independent chains);
 *   JATTN_PROBE_ISSUE_EXP        8 exp2 (eight independent chains);
 *   JATTN_PROBE_ISSUE_MIXED_FMA  the MFMA and the 16 FMAs in every wave;
 *   JATTN_PROBE_ISSUE_MIXED_EXP  the MFMA and the 8 exp2 in every wave;
 *   JATTN_PROBE_ISSUE_SPLIT_FMA  the MFMA in waves 0-3, the 16 FMAs in waves 4-7 (one of each per SIMD);
 *   JATTN_PROBE_ISSUE_SPLIT_EXP  the MFMA in waves 0-3, the 8 exp2 in waves 4-7.
 *   out     device fp32 [blocks * 512]: one value per thread (keeps the work live), overwritten;
 *   cycles  device uint64 [blocks * 8]: each wave's shader-clock cycles (s_memtime) over its loop.
 * With one workgroup per compute unit, the larger of the cycles of waves w and w + 4 over 8 * iters is
 * the SIMD's cycles per step of both its waves.
 * Errors: INVALID_VALUE for an unknown mode, blocks < 1, iters < 1, blocks * 512 >= 2^31, or a null or
 * misaligned out or cycles; HIP if the launch fails. */
#define JATTN_PROBE_ISSUE_MFMA 0
#define JATTN_PROBE_ISSUE_FMA 1
#define JATTN_PROBE_ISSUE_EXP 2
#define JATTN_PROBE_ISSUE_MIXED_FMA 3
#define JATTN_PROBE_ISSUE_MIXED_EXP 4
#define JATTN_PROBE_ISSUE_SPLIT_FMA 5
#define JATTN_PROBE_ISSUE_SPLIT_EXP 6
jattn_status jattn_probe_issue(int mode, int blocks, int iters, float seed, float* out, uint64_t* cycles,
                               hipStream_t stream);

/* The forward tile's structure at D = 64 without global loads, to compare schedules of the two waves
 * that share a SIMD. `blocks` workgroups of 512 threads (8 waves, two per SIMD) loop `iters` times over
 * one step: per wave two 32-query tiles, each with 4 score MFMAs, 16 exp2, 8 bf16 packs and 8 row-sum
 * steps, then 4 PV MFMAs (16 MFMAs of 32x32x16 per wave and step). K and V fragments come from a
 * 64 x 64 LDS tile pair (lds = 1: ds_read_b128 and ds_read_b64_tr_b16) or from registers (lds = 0).
 *   JATTN_PROBE_PINGPONG_FREE     every wave runs scores -> softmax -> PV, no barrier;
 *   JATTN_PROBE_PINGPONG_BARRIER  the same with a workgroup barrier per step;
 *   JATTN_PROBE_PINGPONG_PHASED   two phases per step between barriers, waves 4-7 one phase behind
 *                                 waves 0-3: the MFMAs (S(t), PV(t - 1)) of one wave of each SIMD run
 *                                 while the other wave runs its softmax.
 *   out     device fp32 [blocks * 512], overwritten; cycles device uint64 [blocks * 8]: each wave's
 *   shader-clock cycles over its loop. MFMA pipe busy = 1024 * iters / cycles (two waves per SIMD).
 * Errors: INVALID_VALUE for an unknown mode, lds not 0 or 1, blocks < 1, iters < 1,
 * blocks * 512 >= 2^31, or a null or misaligned out or cycles; HIP if the launch fails. */
#define JATTN_PROBE_PINGPONG_FREE 0
#define JATTN_PROBE_PINGPONG_BARRIER 1
#define JATTN_PROBE_PINGPONG_PHASED 2
jattn_status jattn_probe_pingpong(int mode, int lds, int blocks, int iters, float seed, float* out, uint64_t* cycles,
                                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* JATTN_DIAG_H */
