// C ABI of libjattn.so (declared in include/jattn.h): host-side argument validation, workspace
// sizing and kernel dispatch. Every check runs before the first HIP call, so invalid calls never
// touch the device.
#include "jattn.h"

#include <cmath>
#include <cstdint>

#include "jattn_launch.h"

namespace {

using jattn::kBwdRowsPerBlock;

constexpr int kAbiVersion = 3;

bool supported_head_dim(int D) { return D == 32 || D == 64 || D == 72 || D == 128; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
  const void* p;
  size_t bytes;
};

bool overlap(const Range& x, const Range& y) {
  if (!x.p || !y.p || x.bytes == 0 || y.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(x.p), a1 = a0 + x.bytes;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(y.p), b1 = b0 + y.bytes;
  return a0 < b1 && b0 < a1;
}

// Each output must be disjoint from every other listed buffer (inputs and outputs).
bool outputs_disjoint(const Range* outs, int nout, const Range* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j])) return false;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return false;
  }
  return true;
}

jattn_status check_sizes(int B, int L, int H, int D) {
  if (B < 1 || L < 1 || H < 1 || D < 1) return JATTN_ERROR_INVALID_VALUE;
  if (!supported_head_dim(D)) return JATTN_ERROR_NOT_SUPPORTED;
  const int64_t lhd = (int64_t)L * H * D, bhl = (int64_t)B * H * L;
  const int64_t items = (int64_t)B * H * ((L + kBwdRowsPerBlock - 1) / kBwdRowsPerBlock);
  if ((int64_t)(L + 256) * H * D >= (int64_t(1) << 31) || bhl >= (int64_t(1) << 31) || items * D >= (int64_t(1) << 31) ||
      (int64_t)B * lhd >= (int64_t(1) << 40))
    return JATTN_ERROR_NOT_SUPPORTED;
  return JATTN_SUCCESS;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WorkspaceLayout {
  size_t kr, qs, nlse2, ndelta, part, total;
};

// Normalised key rows and pre-scaled normalised query rows (bf16, [B, H, L, D]), the two row
// statistics (fp32, [B, H, lp] with lp = L rounded up to whole row blocks) and the per-workgroup
// partial sums of the gain-gradient factor (fp32, [items, D]), each 256-byte aligned.
WorkspaceLayout workspace_layout(int B, int L, int H, int D) {
  const size_t nblk = (L + kBwdRowsPerBlock - 1) / kBwdRowsPerBlock;
  const size_t items = (size_t)B * H * nblk, lp = nblk * kBwdRowsPerBlock;
  const size_t rows = round_up((size_t)B * H * L * D * 2, 256), stats = round_up((size_t)B * H * lp * 4, 256),
               parts = round_up(items * D * sizeof(float), 256);
  WorkspaceLayout w;
  w.kr = 0;
  w.qs = w.kr + rows;
  w.nlse2 = w.qs + rows;
  w.ndelta = w.nlse2 + stats;
  w.part = w.ndelta + stats;
  w.total = w.part + parts;
  return w;
}

}  // namespace

extern "C" {

int jattn_abi_version(void) { return kAbiVersion; }

const char* jattn_status_string(jattn_status s) {
  switch (s) {
    case JATTN_SUCCESS: return "JATTN_SUCCESS";
    case JATTN_ERROR_INVALID_VALUE: return "JATTN_ERROR_INVALID_VALUE";
    case JATTN_ERROR_NOT_SUPPORTED: return "JATTN_ERROR_NOT_SUPPORTED";
    case JATTN_ERROR_WORKSPACE: return "JATTN_ERROR_WORKSPACE";
    case JATTN_ERROR_HIP: return "JATTN_ERROR_HIP";
  }
  return "JATTN_UNKNOWN_STATUS";
}

size_t jattn_fwd_workspace_bytes(int B, int L, int H, int D) {
  if (check_sizes(B, L, H, D) != JATTN_SUCCESS) return 0;
  return round_up((size_t)B * H * L * D * 2, 256);  // the normalised key rows
}

size_t jattn_bwd_workspace_bytes(int B, int L, int H, int D) {
  if (check_sizes(B, L, H, D) != JATTN_SUCCESS) return 0;
  return workspace_layout(B, L, H, D).total;
}

jattn_status jattn_fwd_ex(const void* q, const void* k, const void* v, const float* gains,
                          const int32_t* valid_len, int B, int L, int H, int D, float softmax_scale,
                          float eps, void* out, float* lse, void* workspace, size_t workspace_bytes,
                          const hipEvent_t* stage_events, int n_stage_events, hipStream_t stream) {
  if (n_stage_events < 0 || n_stage_events > JATTN_FWD_STAGES || (n_stage_events > 0 && !stage_events))
    return JATTN_ERROR_INVALID_VALUE;
  if (!q || !k || !v || !gains || !out || !lse) return JATTN_ERROR_INVALID_VALUE;
  const jattn_status st = check_sizes(B, L, H, D);
  if (st != JATTN_SUCCESS) return st;
  if (!std::isfinite(softmax_scale) || !std::isfinite(eps) || eps < 0.f) return JATTN_ERROR_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(gains, 4) ||
      !aligned(lse, 4) || !aligned(valid_len, 4))
    return JATTN_ERROR_INVALID_VALUE;
  const size_t wsb = jattn_fwd_workspace_bytes(B, L, H, D);
  if (!workspace || workspace_bytes < wsb) return JATTN_ERROR_WORKSPACE;
  if (!aligned(workspace, 256)) return JATTN_ERROR_INVALID_VALUE;
  const size_t tb = (size_t)B * L * H * D * 2, lb = (size_t)B * H * L * 4;
  const Range ins[] = {{q, tb}, {k, tb}, {v, tb}, {gains, (size_t)2 * D * 4}, {valid_len, (size_t)B * 4}};
  const Range outs[] = {{out, tb}, {lse, lb}, {workspace, wsb}};
  if (!outputs_disjoint(outs, 3, ins, 5)) return JATTN_ERROR_INVALID_VALUE;

  jattn::FwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.kr = static_cast<const uint16_t*>(workspace);
  a.gains = gains;
  a.valid_len = valid_len;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.B = B;
  a.L = L;
  a.H = H;
  a.c = softmax_scale * 1.4426950408889634f;
  a.eps = eps;
  a.nblk = (L + jattn::fwd_rows_per_block(D) - 1) / jattn::fwd_rows_per_block(D);
  a.items = B * H * a.nblk;
  return jattn::launch_fwd(D, a, stage_events, n_stage_events, stream) == hipSuccess ? JATTN_SUCCESS
                                                                                  : JATTN_ERROR_HIP;
}

jattn_status jattn_fwd(const void* q, const void* k, const void* v, const float* gains,
                       const int32_t* valid_len, int B, int L, int H, int D, float softmax_scale,
                       float eps, void* out, float* lse, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  return jattn_fwd_ex(q, k, v, gains, valid_len, B, L, H, D, softmax_scale, eps, out, lse, workspace,
                      workspace_bytes, nullptr, 0, stream);
}

jattn_status jattn_bwd(const void* q, const void* k, const void* v, const float* gains,
                       const int32_t* valid_len, const void* out, const float* lse, const void* dout,
                       int B, int L, int H, int D, float softmax_scale, float eps, void* dq, void* dk,
                       void* dv, float* dgains, void* workspace, size_t workspace_bytes,
                       const void* fwd_workspace, hipStream_t stream) {
  return jattn_bwd_ex(q, k, v, gains, valid_len, out, lse, dout, B, L, H, D, softmax_scale, eps, dq, dk, dv,
                      dgains, workspace, workspace_bytes, fwd_workspace, nullptr, 0, stream);
}

jattn_status jattn_bwd_ex(const void* q, const void* k, const void* v, const float* gains,
                          const int32_t* valid_len, const void* out, const float* lse, const void* dout,
                          int B, int L, int H, int D, float softmax_scale, float eps, void* dq, void* dk,
                          void* dv, float* dgains, void* workspace, size_t workspace_bytes,
                          const void* fwd_workspace, const hipEvent_t* stage_events, int n_stage_events,
                          hipStream_t stream) {
  if (n_stage_events < 0 || n_stage_events > JATTN_BWD_STAGES || (n_stage_events > 0 && !stage_events))
    return JATTN_ERROR_INVALID_VALUE;
  if (!q || !k || !v || !gains || !out || !lse || !dout || !dq || !dk || !dv || !dgains)
    return JATTN_ERROR_INVALID_VALUE;
  const jattn_status st = check_sizes(B, L, H, D);
  if (st != JATTN_SUCCESS) return st;
  if (!std::isfinite(softmax_scale) || !std::isfinite(eps) || eps < 0.f) return JATTN_ERROR_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(gains, 4) || !aligned(lse, 4) ||
      !aligned(dgains, 4) || !aligned(valid_len, 4))
    return JATTN_ERROR_INVALID_VALUE;
  const WorkspaceLayout wl = workspace_layout(B, L, H, D);
  if (!workspace || workspace_bytes < wl.total) return JATTN_ERROR_WORKSPACE;
  if (!aligned(workspace, 256) || !aligned(fwd_workspace, 256)) return JATTN_ERROR_INVALID_VALUE;
  const size_t tb = (size_t)B * L * H * D * 2, lb = (size_t)B * H * L * 4;
  const size_t fwb = fwd_workspace ? jattn_fwd_workspace_bytes(B, L, H, D) : 0;
  const Range ins[] = {{q, tb},   {k, tb},    {v, tb},
                       {gains, (size_t)2 * D * 4}, {valid_len, (size_t)B * 4}, {out, tb},
                       {lse, lb}, {dout, tb}, {fwd_workspace, fwb}};
  const Range outs[] = {{dq, tb}, {dk, tb}, {dv, tb}, {dgains, (size_t)2 * D * 4}, {workspace, wl.total}};
  if (!outputs_disjoint(outs, 5, ins, 9)) return JATTN_ERROR_INVALID_VALUE;

  char* ws = static_cast<char*>(workspace);
  jattn::BwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.gains = gains;
  a.valid_len = valid_len;
  a.out = static_cast<const uint16_t*>(out);
  a.lse = lse;
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.dgains = dgains;
  // normalised keys: the forward's own copy when the caller passes its workspace, else computed here
  a.kr = fwd_workspace ? static_cast<uint16_t*>(const_cast<void*>(fwd_workspace))
                       : reinterpret_cast<uint16_t*>(ws + wl.kr);
  a.qs = reinterpret_cast<uint16_t*>(ws + wl.qs);
  a.nlse2 = reinterpret_cast<float*>(ws + wl.nlse2);
  a.ndelta = reinterpret_cast<float*>(ws + wl.ndelta);
  a.part = reinterpret_cast<float*>(ws + wl.part);
  a.B = B;
  a.L = L;
  a.H = H;
  a.scale = softmax_scale;
  a.c = softmax_scale * 1.4426950408889634f;
  a.eps = eps;
  a.nblk = (L + kBwdRowsPerBlock - 1) / kBwdRowsPerBlock;
  a.items = B * H * a.nblk;
  a.lp = a.nblk * kBwdRowsPerBlock;
  return jattn::launch_bwd(D, a, fwd_workspace == nullptr, stage_events, n_stage_events, stream) == hipSuccess
             ? JATTN_SUCCESS
                                                                                    : JATTN_ERROR_HIP;
}

}  // extern "C"
