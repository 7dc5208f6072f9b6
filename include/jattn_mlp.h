/*
 * jattn_mlp.h -- C ABI of libjattn.so, part 3: the per-stream MLP block after the joint attention of
 * an MM-DiT layer, forward and backward, on MI355X (gfx950) HIP kernels. Its input o is a stream's
 * attention output as jattn_fwd_streams (jattn.h) writes it.
 *
 * What is computed (re-diffusion README: the DiT-layer box of the architecture flowchart continues
 * each stream after the split with fc, adaLN and a SwiGLU MLP, and one residual per stream; the
 * design-notes table gives the MLP as SwiGLU and one ungated residual per block). For stream s with
 * rows o_i (attention output) and x_i (the stream's input to the layer) of sample b:
 *
 *   z_i   = o_i Wfc^T + bfc                                   (fc: Wfc [C, C])
 *   u_i   = LN(z_i) * (1 + scale_b) + shift_b                 (adaLN as in jattn_adaln.h, this block's own
 *                                                              mod[b] = (shift, scale))
 *   [a|g] = u_i W12^T + b12,  W12 = [W1; W3] [2F, C]          (a = columns [0, F), g = [F, 2F))
 *   hid_i = silu(a) * g,      silu(a) = a / (1 + e^-a)
 *   out_i = x_i + hid_i W2^T + b2                             (W2 [C, F]; the one residual)
 *
 * The backward pass returns the gradients of sum(out * dout) with respect to o, mod and every weight
 * and bias. The gradient with respect to x is dout itself (the residual) and is not written.
 *
 * Rounding: z, u, [a|g] and hid are rounded to bf16 once (they are the MFMA operands and are kept in
 * the forward workspace for the backward pass); products accumulate in fp32; silu and its
 * derivative in fp32.
 *
 * Conventions as in jattn_adaln.h: device pointers, 16-byte alignment (workspaces 256), per-stream
 * arguments are host arrays of 2 device pointers {image stream, text stream}, a stream with 0 tokens
 * per sample has no token work (its pointers may be NULL; its parameter gradients, where not NULL,
 * are set to zero), inputs read only, outputs fully overwritten, no allocation or synchronisation,
 * all checks on the host before any HIP call. Bias pointers may be NULL (no bias); bias-gradient
 * pointers may be NULL (not computed).
 *
 * Sizes: B >= 1; n_img, n_txt >= 0 with n_img + n_txt >= 1; C and F multiples of 64 with
 * 64 <= C <= 4096 and 64 <= F <= 16384; B * n_s * 2F < 2^31 per stream. Otherwise INVALID_VALUE or
 * NOT_SUPPORTED.
 */
#ifndef JATTN_MLP_H
#define JATTN_MLP_H

#include "jattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the forward workspace: z, u (bf16 [B n_s, C]), the row statistics (fp32 [B n_s, 2]),
 * [a|g] (bf16 [B n_s, 2F]) and hid (bf16 [B n_s, F]) of both streams, each rounded up to 256 bytes.
 * The backward pass reads it as the forward call with the same inputs wrote it. 0 for invalid sizes. */
size_t jattn_mlp_fwd_workspace_bytes(int B, int n_img, int n_txt, int C, int F);

/* Bytes of the backward workspace: the transposed weights, the gradients of [a|g], u (fp32) and z,
 * and the partial sums of the modulation, weight and bias gradients. 0 for invalid sizes. */
size_t jattn_mlp_bwd_workspace_bytes(int B, int n_img, int n_txt, int C, int F);

/* Kernels each pass enqueues (for stage events): forward 0 = fc GEMM, 1 = adaLN modulation,
 * 2 = gate/up GEMM with the SwiGLU epilogue, 3 = down GEMM with bias and residual; backward
 * 0 = weight transposes, 1 = d(hid) GEMM with the SwiGLU backward (d[a|g]), 2 = dW2 GEMM,
 * 3 = du GEMM, 4 = dW12 GEMM, 5 = LayerNorm backward (dz, modulation partials), 6 = do GEMM,
 * 7 = dWfc GEMM, 8 = reductions. */
#define JATTN_MLP_FWD_STAGES 4
#define JATTN_MLP_BWD_STAGES 9

/* Forward pass.
 *   o[s], x[s]     bf16 [B, n_s, C]   attention output and the stream's input to the layer
 *   mod[s]         fp32 [B, 2, C]     this block's shift (row 0) and scale (row 1)
 *   wfc[s], bfc[s] bf16 [C, C], fp32 [C] or NULL
 *   w12[s], b12[s] bf16 [2F, C] (rows [0, F) = W1, [F, 2F) = W3), fp32 [2F] or NULL
 *   w2[s], b2[s]   bf16 [C, F], fp32 [C] or NULL
 *   eps            LayerNorm epsilon (>= 0, finite)
 *   out[s]         bf16 [B, n_s, C] output
 *   workspace      jattn_mlp_fwd_workspace_bytes(...) bytes; keep it for the backward pass
 *   stage_events / n_stage_events: as jattn_fwd_ex (at most JATTN_MLP_FWD_STAGES)
 * Errors: INVALID_VALUE for null or misaligned pointers of a non-empty stream, bad sizes or eps, an
 * output overlapping another output, an input or the workspace; WORKSPACE for a missing or small
 * workspace; HIP if a launch or an event record fails. */
jattn_status jattn_mlp_fwd(const void* const o[2], const void* const x[2], const float* const mod[2],
                           const void* const wfc[2], const float* const bfc[2], const void* const w12[2],
                           const float* const b12[2], const void* const w2[2], const float* const b2[2], int B,
                           int n_img, int n_txt, int C, int F, float eps, void* const out[2], void* workspace,
                           size_t workspace_bytes, const hipEvent_t* stage_events, int n_stage_events,
                           hipStream_t stream);

/* Backward pass.
 *   o, mod, wfc, w12, w2   the forward's inputs (x, the biases and eps are not needed)
 *   dout[s]        bf16 [B, n_s, C]   gradient of out (and, unchanged, of x)
 *   d_o[s]         bf16 [B, n_s, C]   output: gradient of o
 *   dmod[s]        fp32 [B, 2, C]     output
 *   dwfc[s], dw12[s], dw2[s]   fp32 [C, C], [2F, C], [C, F] outputs
 *   dbfc[s], db12[s], db2[s]   fp32 [C], [2F], [C] outputs, each may be NULL
 *   fwd_workspace  the forward call's workspace, fwd_workspace_bytes its size
 *   workspace      jattn_mlp_bwd_workspace_bytes(...) bytes of scratch
 *   stage_events / n_stage_events: as jattn_bwd_ex (at most JATTN_MLP_BWD_STAGES)
 * Errors as for the forward; fwd_workspace NULL or small -> WORKSPACE. Deterministic (fixed-order
 * sums, no atomics). */
jattn_status jattn_mlp_bwd(const void* const o[2], const float* const mod[2], const void* const wfc[2],
                           const void* const w12[2], const void* const w2[2], const void* const dout[2], int B,
                           int n_img, int n_txt, int C, int F, void* const d_o[2], float* const dmod[2],
                           float* const dwfc[2], float* const dbfc[2], float* const dw12[2], float* const db12[2],
                           float* const dw2[2], float* const db2[2], const void* fwd_workspace,
                           size_t fwd_workspace_bytes, void* workspace, size_t workspace_bytes,
                           const hipEvent_t* stage_events, int n_stage_events, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* JATTN_MLP_H */
