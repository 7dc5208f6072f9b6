/*
 * jattn_adaln.h -- C ABI of libjattn.so, part 2: the adaLN-modulated QKV projection of the two token
 * streams of an MM-DiT layer, forward and backward, on MI355X (gfx950) HIP kernels. Its outputs are
 * the per-stream q, k, v tensors that jattn_fwd_streams (jattn.h) reads, in the same layout.
 *
 * What is computed (re-diffusion README: the DiT-layer box of the architecture flowchart applies
 * adaLN with the conditioning vector to the image stream and to the text stream and computes Q, K
 * and V for each stream; the design-notes table gives adaLN as scale + shift, zero-initialised,
 * without gate). For stream s with rows x_i (C channels) of sample b:
 *
 *   mean_i = mean_c x_ic,   rstd_i = 1 / sqrt(mean_c (x_ic - mean_i)^2 + eps)
 *   h_i    = (x_i - mean_i) * rstd_i * (1 + scale_b) + shift_b        (shift_b = mod[b, 0, :],
 *                                                                      scale_b = mod[b, 1, :])
 *   y_i    = h_i W^T + bias,   q_i = y_i[0, C),  k_i = y_i[C, 2C),  v_i = y_i[2C, 3C)
 *
 * The LayerNorm has no affine parameters of its own (the modulation supplies them). (shift, scale)
 * is the output of the conditioning linear layer of the timestep embedding, computed by the caller.
 * The backward pass returns the gradients of sum(q dq + k dk + v dv) with respect to x, mod, W and
 * the bias.
 *
 * Rounding: h is rounded to bf16 once and is the MFMA operand (and is kept in the forward workspace
 * for the weight gradient); products accumulate in fp32; q, k, v and dx are rounded to bf16 once.
 *
 * Conventions (as in jattn.h): device pointers to contiguous row-major memory owned by the caller;
 * bf16 tensors and fp32 arrays 16-byte aligned, workspaces 256-byte aligned; inputs read only,
 * outputs fully overwritten; work enqueued on `stream`; no allocation, synchronisation or printing;
 * every argument checked on the host before any HIP call. Per-stream arguments are host arrays of 2
 * device pointers {image stream, text stream}. A stream with 0 tokens per sample has no token work:
 * its pointers may be NULL, and its parameter gradients dmod, dw and dbias, where not NULL, are set
 * to zero. Row r of a stream's [B, n_s, C] tensor belongs to sample r / n_s.
 *
 * Sizes: B >= 1; n_img, n_txt >= 0 with n_img + n_txt >= 1; C a multiple of 64 with 64 <= C <= 4096
 * (C = H * D: q, k, v are [B, n_s, H, D] for any head split); B * n_s * C < 2^31 per stream.
 * Otherwise INVALID_VALUE (bad values) or NOT_SUPPORTED (sizes too large).
 */
#ifndef JATTN_ADALN_H
#define JATTN_ADALN_H

#include "jattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the forward workspace: h (bf16 [B n_s, C]) and the row statistics (fp32 [B n_s, 2]) of
 * both streams, each rounded up to 256 bytes. The backward pass reads this workspace as written by the
 * forward call with the same inputs. Returns 0 for invalid or unsupported sizes. */
size_t jattn_adaln_qkv_fwd_workspace_bytes(int B, int n_img, int n_txt, int C);

/* Bytes of the backward workspace: W^T of both streams, the fp32 input-gradient of h, and the
 * partial sums of the modulation, weight and bias gradients. Returns 0 for invalid sizes. */
size_t jattn_adaln_qkv_bwd_workspace_bytes(int B, int n_img, int n_txt, int C);

/* Number of kernels each pass enqueues (for stage events): forward 0 = modulation (h and the row
 * statistics), 1 = projection GEMM; backward 0 = W transpose, 1 = dh GEMM, 2 = LayerNorm backward
 * (dx and the modulation partials), 3 = weight-gradient GEMM, 4 = the reductions. */
#define JATTN_ADALN_FWD_STAGES 2
#define JATTN_ADALN_BWD_STAGES 5

/* Forward pass.
 *   x[s]        bf16 [B, n_s, C]    input token rows of stream s (s = 0 image, 1 text)
 *   mod[s]      fp32 [B, 2, C]      per-sample shift (row 0) and scale (row 1)
 *   w[s]        bf16 [3C, C]        projection weight, torch Linear layout (y = h W^T)
 *   bias[s]     fp32 [3C] or NULL   projection bias
 *   eps         LayerNorm epsilon (>= 0, finite)
 *   q[s], k[s], v[s]   bf16 [B, n_s, C] outputs (= [B, n_s, H, D])
 *   workspace   jattn_adaln_qkv_fwd_workspace_bytes(...) bytes; keep it for the backward pass
 *   stage_events / n_stage_events: as jattn_fwd_ex (NULL, 0 for none; at most JATTN_ADALN_FWD_STAGES)
 * Errors: INVALID_VALUE for null or misaligned pointers of a non-empty stream, bad sizes or eps, an
 * output overlapping another output, an input or the workspace; WORKSPACE for a missing or small
 * workspace; HIP if a launch or an event record fails. */
jattn_status jattn_adaln_qkv_fwd(const void* const x[2], const float* const mod[2], const void* const w[2],
                                 const float* const bias[2], int B, int n_img, int n_txt, int C, float eps,
                                 void* const q[2], void* const k[2], void* const v[2],
                                 void* workspace, size_t workspace_bytes,
                                 const hipEvent_t* stage_events, int n_stage_events, hipStream_t stream);

/* Backward pass.
 *   x, mod, w   the forward's inputs (the bias and eps are not needed: the row statistics in the
 *               forward workspace already hold rstd)
 *   dq[s], dk[s], dv[s]   bf16 [B, n_s, C] gradients of q, k, v
 *   dx[s]       bf16 [B, n_s, C] output
 *   dmod[s]     fp32 [B, 2, C] output (shift row, scale row)
 *   dw[s]       fp32 [3C, C] output
 *   dbias[s]    fp32 [3C] output, or NULL to skip it
 *   fwd_workspace  the forward call's workspace (h and the row statistics), fwd_workspace_bytes its size
 *   workspace   jattn_adaln_qkv_bwd_workspace_bytes(...) bytes of scratch
 *   stage_events / n_stage_events: as jattn_bwd_ex (at most JATTN_ADALN_BWD_STAGES)
 * Errors as for the forward; fwd_workspace NULL or smaller than the forward size -> WORKSPACE. All
 * results are deterministic (fixed-order sums, no atomics). */
jattn_status jattn_adaln_qkv_bwd(const void* const x[2], const float* const mod[2], const void* const w[2],
                                 const void* const dq[2], const void* const dk[2], const void* const dv[2],
                                 int B, int n_img, int n_txt, int C,
                                 void* const dx[2], float* const dmod[2], float* const dw[2], float* const dbias[2],
                                 const void* fwd_workspace, size_t fwd_workspace_bytes,
                                 void* workspace, size_t workspace_bytes,
                                 const hipEvent_t* stage_events, int n_stage_events, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* JATTN_ADALN_H */
