// Backward pass of QK-RMSNorm joint attention on gfx950.
//
// Gradients of L = sum(out * dout) (the analytic backward of the attention defined in the
// re-diffusion README's flowchart and design-notes table; P is recomputed from the saved row
// log-sum-exp, the score matrix is never stored):
//   P = exp(S - lse),  dP = dO V^T,  Delta_i = sum_d dO_id O_id,  dS = P * (dP - Delta)
//   dV = P^T dO,  dQn = scale dS Kn,  dKn = scale dS^T Qn,
//   RMSNorm backward: dx = r (g * dxn) - x (r^3 / D) <g * dxn, x>,   dg = sum_rows dxn * x * r.
//
// Gain gradients. The gains enter the scores only through their product w = g_q * g_k:
// S_ij = scale * sum_d Xq_i[d] w[d] Xk_j[d] with Xq = q r_q, Xk = k r_k. So dg_q = g_k * T and
// dg_k = g_q * T with T[d] = scale * sum_ij dS_ij Xq_i[d] Xk_j[d] = sum_j dKn_j[d] Xk_j[d] / g_q[d]: one
// column sum, taken in the key-parallel kernel.
//
// Four kernels, no atomics:
//  * prenorm (jattn_prenorm.hip): Kr = bf16(k * r_k), normalised keys without gain, into the
//    workspace as [B, H, L, D].
//  * dq kernel (query-parallel, like the forward): each wave owns 32 queries and streams Kr and V;
//    per 32-key step S^T, dP^T (both: lane = query), dS^T in registers, dQn^T += Kr^T dS^T with Kr^T
//    read by ds_read_b64_tr_b16. Epilogue: Q-side RMSNorm backward and dq, and for the key-parallel
//    kernel the pre-scaled normalised queries Qs = bf16(scale log2(e) q r_q) and the row statistics
//    -lse log2(e) and -Delta.
//  * dkdv kernel (key-parallel): each wave owns 32 keys (K rows normalised with both gains, and V
//    rows, in registers) and streams Qs, dO and the row statistics; per 32-query step S, dP
//    (lane = key), then dV^T += dO^T P and dKn^T += Qs^T dS with the transposed operands read by
//    ds_read_b64_tr_b16. Epilogue: K-side RMSNorm backward, dk, dv and per-workgroup partial sums of
//    T. Padded keys get exact zeros.
//  * a small kernel sums the partials in a fixed order and scales them by the other gain
//    (deterministic dgains).
//
// Two-stream variant (S): image and text tokens in their own tensors, addressed through a two-block
// row map, and a gain pair per stream. The gain product then depends on the (query, key) stream
// pair and no longer factors out, so every normalised row carries its own stream's gain (Kr and the
// register key rows the K gain, the query fragments and Qs the Q gain) and the gain gradients are
// summed directly, dg_q,s = sum over queries of stream s of dQn * q * r_q (dq kernel) and
// dg_k,s = sum over keys of stream s of dKn * k * r_k (dk/dv kernel), one partial-sum set each.
// The streamed tiles go straight from memory into LDS (buffer loads with the LDS bit), issued two
// tiles ahead into a ring of LDS buffers: no registers or VALU work are spent on staging.
// dQ is recomputed rather than accumulated across key blocks: fp32 atomics on this chip sustain a
// few hundred G/s, far below what a key-parallel dQ accumulation would need.
#include "jattn_bwd_kernels.h"

namespace jattn {

// Head dims up to 72 run two waves per SIMD with the MFMA accumulators in VGPRs (this file is
// compiled with -amdgpu-mfma-vgpr-form: the score tiles feed VALU work at once). The wider head dims
// are instantiated in jattn_bwd_wide.hip.
template <bool S, bool V, bool W>
static hipError_t launch_bwd_s(int D, const BwdArgs& a, bool prenorm, const hipEvent_t* events, int n_events,
                               hipStream_t stream) {
  switch (D) {
#define JATTN_CASE(DD) \
  case DD: return launch_bwd_d<DD, S, V, W>(a, prenorm, events, n_events, stream);
    JATTN_FOR_EACH_NARROW_HEAD_DIM(JATTN_CASE)
#undef JATTN_CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd(int D, Variant var, const BwdArgs& a, bool prenorm, const hipEvent_t* events,
                      int n_events, hipStream_t stream) {
  if (D > kNarrowMaxD) return launch_bwd_wide(D, var, a, prenorm, events, n_events, stream);
  switch (var) {
    case kStreams: return launch_bwd_s<true, false, false>(D, a, prenorm, events, n_events, stream);
    case kVarlen: return launch_bwd_s<false, true, false>(D, a, prenorm, events, n_events, stream);
    case kWindow: return launch_bwd_s<false, false, true>(D, a, prenorm, events, n_events, stream);
    default: return launch_bwd_s<false, false, false>(D, a, prenorm, events, n_events, stream);
  }
}

}  // namespace jattn
