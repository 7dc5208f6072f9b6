/*
 * jattn.h -- C ABI of libjattn.so: QK-RMSNorm joint image+text attention, forward and backward,
 * on MI355X (gfx950) HIP kernels.
 *
 * What is computed (re-diffusion README: the DiT-layer box of the architecture flowchart
 * concatenates the per-stream Q/K/V and runs one joint multi-head attention over the concatenated
 * sequence; the design-notes table, "QK norm" row, applies RMSNorm to Q and K; the profiling
 * section describes the same attention as an explicit score matrix with an fp32 softmax. The
 * diffusion-pipe summary's attention wrapper has a varlen path, the source of the key-padding
 * length below). For every batch b and head h, with rows x of q and k over the head dim D:
 *
 *   r(x)   = 1 / sqrt(mean_d x_d^2 + eps)
 *   Qn_i   = q_i * r(q_i) * gains[0, :]          Kn_j = k_j * r(k_j) * gains[1, :]
 *   S_ij   = softmax_scale * <Qn_i, Kn_j>        for keys j < n_b, where n_b = clamp(valid_len[b], 0, L)
 *   P_ij   = exp(S_ij - lse_i),  lse_i = log sum_{j < n_b} exp(S_ij)     (natural log)
 *   out_i  = sum_j P_ij v_j                      (non-causal: every query sees every valid key)
 *
 * Padded keys (j >= n_b) are excluded; padded query rows are still computed over the valid keys.
 * A row with no valid key gets out = 0 and lse = -inf. The backward pass returns the gradients of
 * sum(out * dout) with respect to q, k, v and both gain rows; no gradient flows into lse.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers to contiguous row-major memory owned by the caller.
 *    bf16 tensors ([B, L, H, D], 2 bytes per element, element (b, l, h, d) at ((b*L + l)*H + h)*D + d)
 *    must be 16-byte aligned; fp32 / int32 arrays 4-byte aligned; the workspace 256-byte aligned.
 *  - Inputs are read only. Outputs are fully overwritten (including zeros for dk and dv at padded
 *    keys); dgains is overwritten, not accumulated.
 *  - Work is enqueued asynchronously on `stream` (NULL = the null stream). The library never
 *    allocates, frees, synchronises or prints. Its only mutable global state is the device-resident
 *    scratch array of jattn_fwd_noalloc (one per GPU, with its address looked up once per device).
 *  - Arguments are validated on the host before any HIP call. Device-side data (valid_len values,
 *    tensor contents) is not validated: valid_len values are clamped to [0, L]; NaN inputs propagate.
 *  - Supported head dims: every multiple of 8 from 32 to 128. Sizes must satisfy L*H*D < 2^31 and
 *    B*H*L < 2^31.
 */
#ifndef JATTN_H
#define JATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    JATTN_SUCCESS = 0,
    JATTN_ERROR_INVALID_VALUE = 1, /* null pointer, size < 1, misalignment, non-finite scale,
                                      eps < 0 or non-finite, output aliasing another buffer  */
    JATTN_ERROR_NOT_SUPPORTED = 2, /* head dim outside the compiled set, or sizes too large    */
    JATTN_ERROR_WORKSPACE = 3,     /* workspace NULL or smaller than the *_workspace_bytes size */
    JATTN_ERROR_HIP = 4            /* a kernel launch failed (hipGetLastError)                 */
} jattn_status;

/* Relation to the boundary first specified for this library (jattn_fwd(q, k, v, gains, valid_len, B, L, H,
 * D, softmax_scale, eps, out, lse, stream) and jattn_bwd(..., workspace, workspace_bytes, stream)): the
 * forward takes a caller workspace, because its keys are RMS-normalised once into device memory
 * before the attention kernel streams them and the library never allocates; the backward takes the
 * forward's workspace as an optional extra argument, to reuse those normalised keys instead of
 * computing them again (NULL: the backward normalises them itself, as the first specification has
 * it). A caller written to that first forward prototype, and any caller that cannot provide device
 * memory, uses jattn_fwd_noalloc below, which has exactly that parameter list. */

/* Bytes of device workspace jattn_fwd needs for these sizes: the RMS-normalised K rows
 * (B*L*H*D bf16, rounded up to 256 bytes). Returns 0 for invalid or unsupported sizes. */
size_t jattn_fwd_workspace_bytes(int B, int L, int H, int D);

/* Forward pass.
 *   q, k, v    bf16 [B, L, H, D] inputs.
 *   gains      fp32 [2, D]: row 0 multiplies the normalised Q rows, row 1 the normalised K rows.
 *   valid_len  int32 [B] number of valid (unpadded) keys per sequence, or NULL for all L.
 *   softmax_scale  any finite value (the usual choice is 1/sqrt(D)); eps >= 0 (e.g. 1e-6).
 *   out        bf16 [B, L, H, D] output.
 *   lse        fp32 [B, H, L] row log-sum-exp of the scaled scores (natural log), used by jattn_bwd.
 *   workspace  device scratch of at least jattn_fwd_workspace_bytes(B, L, H, D) bytes, 256-byte
 *              aligned; its contents on entry do not matter and are clobbered.
 * out, lse and the workspace must not overlap any input or each other. */
jattn_status jattn_fwd(const void* q, const void* k, const void* v, const float* gains,
                       const int32_t* valid_len, int B, int L, int H, int D,
                       float softmax_scale, float eps, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* jattn_fwd for callers that cannot allocate or pass device memory (code under HIP graph capture,
 * serving loops, harnesses that forbid allocation): the same arguments and results as jattn_fwd
 * without the workspace. The normalised K rows go to a fixed device-resident scratch array of
 * jattn_fwd_noalloc_max_scratch_bytes() bytes (64 MiB) that the library holds on every GPU it runs
 * on until the process ends; the call allocates nothing. B*L*H*D*2 bytes (rounded up to 256) must
 * fit in it, else JATTN_ERROR_WORKSPACE (checked on the host before any HIP call). All calls on one
 * GPU share that GPU's array: two calls whose executions overlap on the same GPU (other streams,
 * other threads) race and give undefined results; calls ordered on one stream are fine. The
 * backward of such a call is jattn_bwd with fwd_workspace = NULL. Errors as jattn_fwd; a failure to
 * find the scratch array -> JATTN_ERROR_HIP. */
jattn_status jattn_fwd_noalloc(const void* q, const void* k, const void* v, const float* gains,
                               const int32_t* valid_len, int B, int L, int H, int D,
                               float softmax_scale, float eps, void* out, float* lse, hipStream_t stream);

/* Size in bytes of the scratch array of jattn_fwd_noalloc. */
size_t jattn_fwd_noalloc_max_scratch_bytes(void);

/* Number of kernels jattn_fwd enqueues, in order: 0 = K-row RMS normalisation (into the
 * workspace), 1 = the attention forward. */
#define JATTN_FWD_STAGES 2

/* jattn_fwd with per-stage timing hooks; identical results. stage_events / n_stage_events as for
 * jattn_bwd_ex below, with JATTN_FWD_STAGES stages. */
jattn_status jattn_fwd_ex(const void* q, const void* k, const void* v, const float* gains,
                          const int32_t* valid_len, int B, int L, int H, int D,
                          float softmax_scale, float eps, void* out, float* lse,
                          void* workspace, size_t workspace_bytes,
                          const hipEvent_t* stage_events, int n_stage_events, hipStream_t stream);

/* Bytes of device workspace jattn_bwd needs for these sizes: normalised K rows and pre-scaled
 * normalised Q rows (2 * B*L*H*D bf16), two fp32 row statistics per query row, and per-workgroup
 * partial sums of the gain gradients. Returns 0 for invalid or unsupported sizes. */
size_t jattn_bwd_workspace_bytes(int B, int L, int H, int D);

/* Backward pass. Takes the forward inputs, the forward outputs out and lse (from jattn_fwd with the
 * same arguments) and dout (bf16 [B, L, H, D], the gradient of the loss with respect to out).
 *   dq, dk, dv  bf16 [B, L, H, D] gradients with respect to q, k, v (overwritten).
 *   dgains      fp32 [2, D] gradient with respect to gains (overwritten; deterministic).
 *   workspace   device scratch of at least jattn_bwd_workspace_bytes(B, L, H, D) bytes, 256-byte
 *               aligned; its contents on entry do not matter and are clobbered.
 *   fwd_workspace  NULL, or the workspace of the jattn_fwd call that produced out and lse, unchanged
 *               since (it holds the normalised K rows; the backward then reuses them instead of
 *               normalising K again). Read only; 256-byte aligned.
 * Outputs and workspace must not overlap any input (fwd_workspace included) or each other. */
jattn_status jattn_bwd(const void* q, const void* k, const void* v, const float* gains,
                       const int32_t* valid_len, const void* out, const float* lse, const void* dout,
                       int B, int L, int H, int D, float softmax_scale, float eps,
                       void* dq, void* dk, void* dv, float* dgains,
                       void* workspace, size_t workspace_bytes, const void* fwd_workspace,
                       hipStream_t stream);

/* Number of kernels jattn_bwd enqueues, in order: 0 = K-row RMS normalisation (skipped, with its
 * event still recorded, when fwd_workspace is given), 1 = dq
 * (query-parallel; also writes the normalised Q rows and the row statistics), 2 = dk/dv
 * (key-parallel), 3 = gain-gradient reduction. */
#define JATTN_BWD_STAGES 4

/* jattn_bwd with per-stage timing hooks, for callers that attribute time to the individual kernels
 * (profilers, benchmarks). Identical results to jattn_bwd. If n_stage_events > 0, stage_events points
 * to n_stage_events (<= JATTN_BWD_STAGES) events created by the caller; event i is recorded on `stream`
 * right after stage i is enqueued, so hipEventElapsedTime between an event recorded before the call
 * and event 0, or between events i-1 and i, gives the duration of stage i. A NULL entry records
 * nothing after its stage (each recorded event is a timestamp on the stream, which costs the stream a
 * few microseconds, so a caller timing one stage records only the events around it).
 * n_stage_events < 0, or > 0 with a NULL array, or > JATTN_BWD_STAGES -> INVALID_VALUE. A failed
 * hipEventRecord -> HIP. */
jattn_status jattn_bwd_ex(const void* q, const void* k, const void* v, const float* gains,
                          const int32_t* valid_len, const void* out, const float* lse, const void* dout,
                          int B, int L, int H, int D, float softmax_scale, float eps,
                          void* dq, void* dk, void* dv, float* dgains,
                          void* workspace, size_t workspace_bytes, const void* fwd_workspace,
                          const hipEvent_t* stage_events, int n_stage_events, hipStream_t stream);

/* ------------------------------------------------------------------------------------------------
 * Local-window entry points. The diffusion-pipe summary's attention wrapper has a windowed variant
 * besides the full one; here it is a sliding window over the joint sequence: query i sees only the
 * keys j with  i - window_left <= j <= i + window_right  (and j < n_b as before). A negative bound is
 * no bound on that side, so (-1, 0) is causal attention and (-1, -1) the joint attention above. A
 * query whose window holds no valid key gets out = 0, lse = -inf and zero gradients. Everything else
 * (arguments, layouts, workspaces from jattn_fwd_workspace_bytes / jattn_bwd_workspace_bytes, stage
 * events, errors) is as for jattn_fwd_ex and jattn_bwd_ex; lse and out from jattn_fwd_window go with
 * jattn_bwd_window and the same window. Only the key tiles a block of queries can reach are read. */
jattn_status jattn_fwd_window(const void* q, const void* k, const void* v, const float* gains,
                              const int32_t* valid_len, int B, int L, int H, int D,
                              float softmax_scale, float eps, int window_left, int window_right,
                              void* out, float* lse, void* workspace, size_t workspace_bytes,
                              const hipEvent_t* stage_events, int n_stage_events, hipStream_t stream);

jattn_status jattn_bwd_window(const void* q, const void* k, const void* v, const float* gains,
                              const int32_t* valid_len, const void* out, const float* lse, const void* dout,
                              int B, int L, int H, int D, float softmax_scale, float eps,
                              int window_left, int window_right,
                              void* dq, void* dk, void* dv, float* dgains,
                              void* workspace, size_t workspace_bytes, const void* fwd_workspace,
                              const hipEvent_t* stage_events, int n_stage_events, hipStream_t stream);

/* ------------------------------------------------------------------------------------------------
 * Two-stream entry points (zero-copy image + text streams with a QK-norm gain pair per stream).
 *
 * The re-diffusion README's DiT-layer box computes Q, K and V separately for each stream ("QKV
 * each"), concatenates them, runs the joint attention and splits the result back per stream. These
 * entry points take each per-token tensor as its two stream parts and write the outputs back to
 * them, so no concatenation or split copy is needed around the attention, and let each stream keep
 * its own QK-RMSNorm gains. The result is the joint attention above on the concatenated sequence
 * [image rows; text rows] (L = n_img + n_txt, image first), with every row of stream s normalised
 * by that stream's gains:
 *   Qn_i = q_i * r(q_i) * gains[s(i)][0, :]        Kn_j = k_j * r(k_j) * gains[s(j)][1, :]
 *
 * Tensor arguments are HOST arrays of two DEVICE pointers, {image part, text part}:
 *   part 0  bf16 [B, n_img, H, D] (rows 0 .. n_img-1 of each joint sequence),
 *   part 1  bf16 [B, n_txt, H, D] (rows n_img .. L-1),
 * each contiguous and 16-byte aligned; the pointer of an empty stream (n = 0) is ignored and may be
 * NULL. The host arrays are read during the call only.
 *   gains   fp32 [2, 2, D]: gains[s][0] = Q gain, gains[s][1] = K gain of stream s (0 = image).
 *   valid_len, lse, softmax_scale, eps and the workspaces: as for the joint entry points, with L =
 *           n_img + n_txt (valid_len[b] counts keys of the joint sequence, image rows first; lse is
 *           [B, H, L] in joint row order). Workspace sizes: jattn_fwd_workspace_bytes(B, L, H, D)
 *           and jattn_bwd_workspace_bytes(B, L, H, D).
 * Errors as for the joint entry points; n_img < 0, n_txt < 0 or n_img + n_txt < 1, a NULL host
 * array, or a NULL / misaligned pointer of a non-empty stream -> INVALID_VALUE. Every output part
 * must be disjoint from every input part and from the other outputs. */

/* Forward pass over the two streams. Stages and events as jattn_fwd_ex (JATTN_FWD_STAGES; pass
 * NULL, 0 for none). out = {image output, text output}. */
jattn_status jattn_fwd_streams(const void* const q[2], const void* const k[2], const void* const v[2],
                               const float* gains, const int32_t* valid_len, int B, int n_img, int n_txt,
                               int H, int D, float softmax_scale, float eps, void* const out[2], float* lse,
                               void* workspace, size_t workspace_bytes,
                               const hipEvent_t* stage_events, int n_stage_events, hipStream_t stream);

/* Backward pass over the two streams: out and lse from jattn_fwd_streams with the same arguments,
 * dout the gradient with respect to out (two parts). Writes dq, dk, dv (two parts each) and
 * dgains fp32 [2, 2, D] (the gradient with respect to gains; overwritten, deterministic).
 * fwd_workspace: NULL or the workspace of that jattn_fwd_streams call, unchanged since. Stages and
 * events as jattn_bwd_ex (JATTN_BWD_STAGES; pass NULL, 0 for none). */
jattn_status jattn_bwd_streams(const void* const q[2], const void* const k[2], const void* const v[2],
                               const float* gains, const int32_t* valid_len, const void* const out[2],
                               const float* lse, const void* const dout[2], int B, int n_img, int n_txt,
                               int H, int D, float softmax_scale, float eps, void* const dq[2],
                               void* const dk[2], void* const dv[2], float* dgains,
                               void* workspace, size_t workspace_bytes, const void* fwd_workspace,
                               const hipEvent_t* stage_events, int n_stage_events, hipStream_t stream);

/* ------------------------------------------------------------------------------------------------
 * Packed variable-length entry points (no padding: sequences of different lengths back to back).
 *
 * The diffusion-pipe summary's attention wrapper has a variable-length path besides the padded one;
 * mixed caption lengths and multi-resolution buckets (the re-diffusion README's aspect buckets) give
 * such batches. Here B sequences are stored back to back: q, k, v, out, dout, dq, dk, dv are bf16
 * [total, H, D] with sequence b at token rows [cu_seqlens[b], cu_seqlens[b+1]). Each sequence attends
 * only to itself, with all of its keys valid, and gets exactly the joint attention above (one gain
 * pair gains fp32 [2, D], as jattn_fwd).
 *   cu_seqlens  int32 [B + 1] on the DEVICE, non-decreasing, cu_seqlens[0] = 0, cu_seqlens[B] <= total.
 *               Device data is not validated, but every access stays inside the tensors: sequence b
 *               is taken as rows [start, end) with start = clamp(cu[b], 0, total) and end =
 *               clamp(cu[b+1], start, min(total, start + max_seqlen)); rows not covered by any
 *               sequence are left unwritten, and overlapping sequences give undefined results.
 *   max_seqlen  the longest sequence (an upper bound on cu[b+1] - cu[b]); sizes the grids.
 *   total       token rows of the tensors (>= 1).
 *   lse         fp32, total * H elements: sequence b, head h, row l at cu[b] * H + h * L_b + l (one
 *               [H, L_b] block per sequence; a fixed-length batch gives exactly [B, H, L]).
 *   dgains      fp32 [2, D], summed over all sequences.
 * Workspace sizes: jattn_varlen_fwd_workspace_bytes and jattn_varlen_bwd_workspace_bytes; stages and
 * events as jattn_fwd_ex / jattn_bwd_ex (pass NULL, 0 for none). Errors as for the joint entry points;
 * NULL cu_seqlens or total < 1 -> INVALID_VALUE; B > 65535 -> NOT_SUPPORTED. */
size_t jattn_varlen_fwd_workspace_bytes(int B, int max_seqlen, int total, int H, int D);
size_t jattn_varlen_bwd_workspace_bytes(int B, int max_seqlen, int total, int H, int D);

jattn_status jattn_fwd_varlen(const void* q, const void* k, const void* v, const float* gains,
                              const int32_t* cu_seqlens, int B, int max_seqlen, int total, int H, int D,
                              float softmax_scale, float eps, void* out, float* lse,
                              void* workspace, size_t workspace_bytes,
                              const hipEvent_t* stage_events, int n_stage_events, hipStream_t stream);

jattn_status jattn_bwd_varlen(const void* q, const void* k, const void* v, const float* gains,
                              const int32_t* cu_seqlens, const void* out, const float* lse, const void* dout,
                              int B, int max_seqlen, int total, int H, int D, float softmax_scale, float eps,
                              void* dq, void* dk, void* dv, float* dgains,
                              void* workspace, size_t workspace_bytes, const void* fwd_workspace,
                              const hipEvent_t* stage_events, int n_stage_events, hipStream_t stream);

/* Static, human-readable name of a status code (never NULL). */
const char* jattn_status_string(jattn_status s);

/* Version of this ABI; bumped on any incompatible change. */
int jattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* JATTN_H */
