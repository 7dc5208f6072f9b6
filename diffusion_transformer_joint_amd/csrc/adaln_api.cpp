// C ABI of the adaLN-modulated QKV projection (declared in include/jattn_adaln.h): host-side
// validation, workspace layouts and kernel dispatch. Every check runs before the first HIP call.
#include "jattn_adaln.h"

#include <climits>
#include <cmath>
#include <cstdint>

#include "adaln_launch.h"
#include "api_common.h"

namespace {

using jattn::kBwdRowChunk;
using jattn::kGemmK;
using namespace jattn_api;

struct Sizes {
  int B, n[2], C;
  int64_t T[2];
};

jattn_status check_sizes(int B, int n_img, int n_txt, int C, Sizes* z) {
  if (B < 1 || n_img < 0 || n_txt < 0 || (int64_t)n_img + n_txt < 1 || C < 64 || C % 64 != 0)
    return JATTN_ERROR_INVALID_VALUE;
  if (C > 4096) return JATTN_ERROR_NOT_SUPPORTED;
  z->B = B;
  z->n[0] = n_img;
  z->n[1] = n_txt;
  z->C = C;
  for (int s = 0; s < 2; ++s) {
    z->T[s] = (int64_t)B * z->n[s];
    if (z->T[s] * 3 * C >= (int64_t(1) << 31)) return JATTN_ERROR_NOT_SUPPORTED;
  }
  if (z->T[0] + z->T[1] >= (int64_t(1) << 31) / 4) return JATTN_ERROR_NOT_SUPPORTED;
  return JATTN_SUCCESS;
}

struct FwdLayout {
  size_t h[2], stats[2], total;
};

FwdLayout fwd_layout(const Sizes& z) {
  FwdLayout l;
  size_t off = 0;
  for (int s = 0; s < 2; ++s) {
    l.h[s] = off;
    off += round_up((size_t)z.T[s] * z.C * 2, 256);
  }
  for (int s = 0; s < 2; ++s) {
    l.stats[s] = off;
    off += round_up((size_t)z.T[s] * 2 * 4, 256);
  }
  l.total = off;
  return l;
}

struct BwdLayout {
  size_t wt[2], dh[2], modpart[2], wpart[2], cpart[2], total;
  int chunks[2], splits[2], kchunk[2];
};

BwdLayout bwd_layout(const Sizes& z) {
  BwdLayout l;
  const size_t C = z.C;
  size_t off = 0;
  dw_splits(z.T, z.C, 3 * z.C, l.splits, l.kchunk);
  for (int s = 0; s < 2; ++s) {
    l.chunks[s] = (z.n[s] + kBwdRowChunk - 1) / kBwdRowChunk;
    const bool on = z.T[s] > 0;
    l.wt[s] = off;
    off += on ? round_up(3 * C * C * 2, 256) : 0;
    l.dh[s] = off;
    off += round_up((size_t)z.T[s] * C * 4, 256);
    l.modpart[s] = off;
    off += round_up((size_t)z.B * l.chunks[s] * 2 * C * 4, 256);
    const bool parts = on && l.splits[s] > 1;  // (one split writes the gradients directly)
    l.wpart[s] = off;
    off += parts ? round_up((size_t)l.splits[s] * 3 * C * C * 4, 256) : 0;
    l.cpart[s] = off;
    off += parts ? round_up((size_t)l.splits[s] * 3 * C * 4, 256) : 0;
  }
  l.total = off;
  return l;
}

}  // namespace

extern "C" {

size_t jattn_adaln_qkv_fwd_workspace_bytes(int B, int n_img, int n_txt, int C) {
  Sizes z;
  if (check_sizes(B, n_img, n_txt, C, &z) != JATTN_SUCCESS) return 0;
  return fwd_layout(z).total;
}

size_t jattn_adaln_qkv_bwd_workspace_bytes(int B, int n_img, int n_txt, int C) {
  Sizes z;
  if (check_sizes(B, n_img, n_txt, C, &z) != JATTN_SUCCESS) return 0;
  return bwd_layout(z).total;
}

jattn_status jattn_adaln_qkv_fwd(const void* const x[2], const float* const mod[2], const void* const w[2],
                                 const float* const bias[2], int B, int n_img, int n_txt, int C, float eps,
                                 void* const q[2], void* const k[2], void* const v[2], void* workspace,
                                 size_t workspace_bytes, const hipEvent_t* stage_events, int n_stage_events,
                                 hipStream_t stream) {
  if (!x || !mod || !w || !bias || !q || !k || !v) return JATTN_ERROR_INVALID_VALUE;
  Sizes z;
  jattn_status st = check_sizes(B, n_img, n_txt, C, &z);
  if (st != JATTN_SUCCESS) return st;
  if (!std::isfinite(eps) || eps < 0.f) return JATTN_ERROR_INVALID_VALUE;
  if ((st = check_events(stage_events, n_stage_events, JATTN_ADALN_FWD_STAGES)) != JATTN_SUCCESS) return st;
  const FwdLayout lay = fwd_layout(z);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < lay.total) return JATTN_ERROR_WORKSPACE;
  Range outs[7], ins[8];
  int no = 0, ni = 0;
  outs[no++] = {workspace, lay.total};
  for (int s = 0; s < 2; ++s) {
    if (z.T[s] == 0) continue;
    if (!ptr_ok(x[s]) || !ptr_ok(mod[s]) || !ptr_ok(w[s]) || !ptr_ok(q[s]) || !ptr_ok(k[s]) || !ptr_ok(v[s]) ||
        (bias[s] && !aligned(bias[s], 16)))
      return JATTN_ERROR_INVALID_VALUE;
    const size_t act = (size_t)z.T[s] * C * 2;
    outs[no++] = {q[s], act};
    outs[no++] = {k[s], act};
    outs[no++] = {v[s], act};
    ins[ni++] = {x[s], act};
    ins[ni++] = {mod[s], (size_t)B * 2 * C * 4};
    ins[ni++] = {w[s], (size_t)3 * C * C * 2};
    ins[ni++] = {bias[s], bias[s] ? (size_t)3 * C * 4 : 0};
  }
  if (!disjoint(outs, no, ins, ni)) return JATTN_ERROR_INVALID_VALUE;

  char* ws = static_cast<char*>(workspace);
  jattn::ModulateArgs ma{};
  jattn::GemmArgs g{};
  for (int s = 0; s < 2; ++s) {
    const bool on = z.T[s] > 0;
    ma.x[s] = static_cast<const uint16_t*>(on ? x[s] : nullptr);
    ma.mod[s] = on ? mod[s] : nullptr;
    ma.h[s] = reinterpret_cast<uint16_t*>(ws + lay.h[s]);
    ma.stats[s] = reinterpret_cast<float*>(ws + lay.stats[s]);
    ma.n[s] = z.n[s] > 0 ? z.n[s] : 1;
    ma.T[s] = (int)z.T[s];
    jattn::GemmProblem& p = g.pr[s];
    p.a = mat(on ? w[s] : workspace, nullptr, nullptr, C, C, 3 * (int64_t)C, C);
    p.b = mat(ws + lay.h[s], nullptr, nullptr, C, C, z.T[s], C);
    p.M = 3 * C;
    p.N = (int)z.T[s];
    p.K = C;
    p.splits = 1;
    p.kchunk = C;
    p.out[0] = on ? q[s] : nullptr;
    p.out[1] = on ? k[s] : nullptr;
    p.out[2] = on ? v[s] : nullptr;
    p.out_seg = C;
    p.bias = on ? bias[s] : nullptr;
    p.colsum = nullptr;
  }
  ma.C = C;
  ma.eps = eps;
  finish(g, jattn::kQkvMA, jattn::kQkvMB);

  jattn::launch_modulate(ma, stream);
  if (!stage_done(0, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  jattn::launch_qkv_gemm(g, stream);
  if (!stage_done(1, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  return JATTN_SUCCESS;
}

jattn_status jattn_adaln_qkv_bwd(const void* const x[2], const float* const mod[2], const void* const w[2],
                                 const void* const dq[2], const void* const dk[2], const void* const dv[2], int B,
                                 int n_img, int n_txt, int C, void* const dx[2], float* const dmod[2],
                                 float* const dw[2], float* const dbias[2], const void* fwd_workspace,
                                 size_t fwd_workspace_bytes, void* workspace, size_t workspace_bytes,
                                 const hipEvent_t* stage_events, int n_stage_events, hipStream_t stream) {
  if (!x || !mod || !w || !dq || !dk || !dv || !dx || !dmod || !dw || !dbias) return JATTN_ERROR_INVALID_VALUE;
  Sizes z;
  jattn_status st = check_sizes(B, n_img, n_txt, C, &z);
  if (st != JATTN_SUCCESS) return st;
  if ((st = check_events(stage_events, n_stage_events, JATTN_ADALN_BWD_STAGES)) != JATTN_SUCCESS) return st;
  const FwdLayout fl = fwd_layout(z);
  const BwdLayout bl = bwd_layout(z);
  if (!fwd_workspace || !aligned(fwd_workspace, 256) || fwd_workspace_bytes < fl.total) return JATTN_ERROR_WORKSPACE;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < bl.total) return JATTN_ERROR_WORKSPACE;
  Range outs[9], ins[14];
  int no = 0, ni = 0;
  outs[no++] = {workspace, bl.total};
  ins[ni++] = {fwd_workspace, fl.total};
  for (int s = 0; s < 2; ++s) {
    if (z.T[s] == 0) {  // an empty stream's parameter gradients, where given, are written as zeros
      if ((dmod[s] && !aligned(dmod[s], 16)) || (dw[s] && !aligned(dw[s], 16)) || (dbias[s] && !aligned(dbias[s], 16)))
        return JATTN_ERROR_INVALID_VALUE;
      outs[no++] = {dmod[s], dmod[s] ? (size_t)B * 2 * C * 4 : 0};
      outs[no++] = {dw[s], dw[s] ? (size_t)3 * C * C * 4 : 0};
      outs[no++] = {dbias[s], dbias[s] ? (size_t)3 * C * 4 : 0};
      continue;
    }
    if (!ptr_ok(x[s]) || !ptr_ok(mod[s]) || !ptr_ok(w[s]) || !ptr_ok(dq[s]) || !ptr_ok(dk[s]) || !ptr_ok(dv[s]) ||
        !ptr_ok(dx[s]) || !ptr_ok(dmod[s]) || !ptr_ok(dw[s]) || (dbias[s] && !aligned(dbias[s], 16)))
      return JATTN_ERROR_INVALID_VALUE;
    const size_t act = (size_t)z.T[s] * C * 2;
    outs[no++] = {dx[s], act};
    outs[no++] = {dmod[s], (size_t)B * 2 * C * 4};
    outs[no++] = {dw[s], (size_t)3 * C * C * 4};
    outs[no++] = {dbias[s], dbias[s] ? (size_t)3 * C * 4 : 0};
    ins[ni++] = {x[s], act};
    ins[ni++] = {mod[s], (size_t)B * 2 * C * 4};
    ins[ni++] = {w[s], (size_t)3 * C * C * 2};
    ins[ni++] = {dq[s], act};
    ins[ni++] = {dk[s], act};
    ins[ni++] = {dv[s], act};
  }
  if (!disjoint(outs, no, ins, ni)) return JATTN_ERROR_INVALID_VALUE;

  const char* fws = static_cast<const char*>(fwd_workspace);
  char* ws = static_cast<char*>(workspace);
  jattn::TransposeArgs ta{};
  jattn::GemmArgs gdh{}, gdw{};
  jattn::RowsBwdArgs ra{};
  jattn::ReduceArgs rm{}, rw{};
  ta.n = 0;
  ta.start[0] = 0;
  for (int s = 0; s < 2; ++s) {
    const bool on = z.T[s] > 0;
    const uint16_t* wt = reinterpret_cast<const uint16_t*>(ws + bl.wt[s]);
    if (on) {  // W [3C, C] -> W^T
      ta.src[ta.n] = static_cast<const uint16_t*>(w[s]);
      ta.dst[ta.n] = reinterpret_cast<uint16_t*>(ws + bl.wt[s]);
      ta.rows[ta.n] = 3 * C;
      ta.cols[ta.n] = C;
      ta.start[ta.n + 1] = ta.start[ta.n] + 3 * (C / 64) * (C / 64);
      ++ta.n;
    }
    const void* h = fws + fl.h[s];
    // dh = dY W: MFMA-A = W^T [C, 3C], MFMA-B = dY [T, 3C] over the three tensors
    jattn::GemmProblem& p = gdh.pr[s];
    p.a = mat(on ? (const void*)wt : workspace, nullptr, nullptr, 3 * C, 3 * C, C, 3 * C);
    p.b = mat(on ? dq[s] : workspace, on ? dk[s] : nullptr, on ? dv[s] : nullptr, C, C, z.T[s], 3 * C);
    p.M = C;
    p.N = (int)z.T[s];
    p.K = 3 * C;
    p.splits = 1;
    p.kchunk = 3 * C;
    p.out[0] = ws + bl.dh[s];
    p.out[1] = p.out[2] = nullptr;
    p.out_seg = C;
    p.bias = nullptr;
    p.colsum = nullptr;
    // dW = dY^T h: MFMA-A = h^T (channels), MFMA-B = dY^T (output columns), split over the tokens
    jattn::GemmProblem& r = gdw.pr[s];
    r.a = mat(on ? h : workspace, nullptr, nullptr, C, C, z.T[s], C);
    r.b = mat(on ? dq[s] : workspace, on ? dk[s] : nullptr, on ? dv[s] : nullptr, C, C, z.T[s], 3 * C);
    r.M = C;
    r.N = 3 * C;
    r.K = (int)z.T[s];
    r.splits = bl.splits[s];
    r.kchunk = bl.kchunk[s];
    const bool direct = bl.splits[s] == 1;  // one split: straight into dw and dbias
    r.out[0] = direct ? static_cast<void*>(on ? dw[s] : nullptr) : static_cast<void*>(ws + bl.wpart[s]);
    r.out[1] = r.out[2] = nullptr;
    r.out_seg = C;
    r.bias = nullptr;
    r.colsum = on && dbias[s] ? (direct ? dbias[s] : reinterpret_cast<float*>(ws + bl.cpart[s])) : nullptr;
    if (!on) r.M = 0;
    // LayerNorm backward
    ra.x[s] = static_cast<const uint16_t*>(on ? x[s] : nullptr);
    ra.mod[s] = on ? mod[s] : nullptr;
    ra.stats[s] = reinterpret_cast<const float*>(fws + fl.stats[s]);
    ra.dh[s] = reinterpret_cast<const float*>(ws + bl.dh[s]);
    ra.dx[s] = static_cast<uint16_t*>(on ? dx[s] : nullptr);
    ra.part[s] = reinterpret_cast<float*>(ws + bl.modpart[s]);
    ra.n[s] = z.n[s] > 0 ? z.n[s] : 1;
    ra.chunks[s] = on ? bl.chunks[s] : 0;
    // reductions
    rm.part[s] = ra.part[s];
    rm.cpart[s] = nullptr;
    rm.out[s] = dmod[s];
    rm.cout[s] = nullptr;
    rm.count[s] = on ? bl.chunks[s] : 0;  // (no partials: zeros)
    rm.len[s] = dmod[s] ? B * 2 * C : 0;
    rm.inner[s] = 2 * C;
    rm.clen[s] = 0;
    rw.part[s] = reinterpret_cast<const float*>(ws + bl.wpart[s]);
    // reduction of the split partials; a stream with one split has nothing to reduce, an empty
    // stream gets zeros (count 0)
    const bool reduce = !on || !direct;
    rw.out[s] = dw[s];
    rw.cpart[s] = on ? r.colsum : rw.part[s];
    rw.cout[s] = reduce ? (on ? (r.colsum ? dbias[s] : nullptr) : dbias[s]) : nullptr;
    rw.count[s] = on ? bl.splits[s] : 0;
    rw.len[s] = reduce && dw[s] ? 3 * C * C : 0;
    rw.inner[s] = 0;
    rw.clen[s] = 3 * C;
  }
  ra.B = B;
  ra.C = C;
  ra.blocks0 = B * ra.chunks[0];
  finish(gdh, jattn::kDhMA, jattn::kDhMB);
  finish(gdw, jattn::kDwMA, jattn::kDwMB);

  jattn::launch_transpose_w(ta, stream);
  if (!stage_done(0, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  jattn::launch_dh_gemm(gdh, stream);
  if (!stage_done(1, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  jattn::launch_rows_bwd(ra, stream);
  if (!stage_done(2, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  jattn::launch_dw_gemm(gdw, stream);
  if (!stage_done(3, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  jattn::launch_mod_reduce(rm, stream);
  if (!launched()) return JATTN_ERROR_HIP;
  jattn::launch_w_reduce(rw, stream);
  if (!stage_done(4, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  return JATTN_SUCCESS;
}

}  // extern "C"
