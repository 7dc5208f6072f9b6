// C ABI of the MLP block after the joint attention (declared in include/jattn_mlp.h): host-side
// validation, workspace layouts and kernel dispatch. Every check runs before the first HIP call.
// The block reuses the projection kernels of adaln_qkv.hip: the bf16-output GEMM (fc, the down
// projection with its residual, the input gradient), the modulation and LayerNorm-backward row
// kernels, the fp32-output GEMM (with the SwiGLU backward in its epilogue for d(hid)), the
// weight-gradient GEMM, the reductions, and the SwiGLU gate/up GEMM.
#include "jattn_mlp.h"

#include <cmath>
#include <cstdint>

#include "adaln_launch.h"
#include "api_common.h"

namespace {

using namespace jattn_api;
using jattn::kBwdRowChunk;

struct Sizes {
  int B, n[2], C, F;
  int64_t T[2];
};

jattn_status check_sizes(int B, int n_img, int n_txt, int C, int F, Sizes* z) {
  if (B < 1 || n_img < 0 || n_txt < 0 || (int64_t)n_img + n_txt < 1 || C < 64 || C % 64 != 0 || F < 64 || F % 64 != 0)
    return JATTN_ERROR_INVALID_VALUE;
  if (C > 4096 || F > 16384) return JATTN_ERROR_NOT_SUPPORTED;
  z->B = B;
  z->n[0] = n_img;
  z->n[1] = n_txt;
  z->C = C;
  z->F = F;
  for (int s = 0; s < 2; ++s) {
    z->T[s] = (int64_t)B * z->n[s];
    if (z->T[s] * 2 * F >= (int64_t(1) << 31) || z->T[s] * C >= (int64_t(1) << 31)) return JATTN_ERROR_NOT_SUPPORTED;
  }
  if (z->T[0] + z->T[1] >= (int64_t(1) << 31) / 4) return JATTN_ERROR_NOT_SUPPORTED;
  return JATTN_SUCCESS;
}

struct FwdLayout {
  size_t z[2], u[2], stats[2], ag[2], hid[2], total;
};

FwdLayout fwd_layout(const Sizes& d) {
  FwdLayout l;
  size_t off = 0;
  for (int s = 0; s < 2; ++s) {
    const size_t T = (size_t)d.T[s];
    l.z[s] = off;
    off += round_up(T * d.C * 2, 256);
    l.u[s] = off;
    off += round_up(T * d.C * 2, 256);
    l.stats[s] = off;
    off += round_up(T * 2 * 4, 256);
    l.ag[s] = off;
    off += round_up(T * 2 * d.F * 2, 256);
    l.hid[s] = off;
    off += round_up(T * d.F * 2, 256);
  }
  l.total = off;
  return l;
}

// One weight gradient (output [N, M] of the weight-gradient GEMM) of both streams: its token splits
// and, with more than one split, the offsets of its partials.
struct WGradLayout {
  int splits[2], kchunk[2];
  size_t part[2], cpart[2];
};

struct BwdLayout {
  size_t w2t[2], w12t[2], wfct[2], dag[2], du[2], dz[2], modpart[2], total;
  int chunks[2];
  WGradLayout g2, g12, gfc;
};

void wgrad_layout(const Sizes& d, int M, int N, WGradLayout* g, size_t* off, int s) {
  const bool parts = d.T[s] > 0 && g->splits[s] > 1;
  g->part[s] = *off;
  *off += parts ? round_up((size_t)g->splits[s] * N * M * 4, 256) : 0;
  g->cpart[s] = *off;
  *off += parts ? round_up((size_t)g->splits[s] * N * 4, 256) : 0;
}

BwdLayout bwd_layout(const Sizes& d) {
  BwdLayout l;
  const size_t C = d.C, F = d.F;
  dw_splits(d.T, d.F, d.C, l.g2.splits, l.g2.kchunk);       // dW2 [C, F]: M = F, N = C
  dw_splits(d.T, d.C, 2 * d.F, l.g12.splits, l.g12.kchunk);  // dW12 [2F, C]: M = C, N = 2F
  dw_splits(d.T, d.C, d.C, l.gfc.splits, l.gfc.kchunk);     // dWfc [C, C]
  size_t off = 0;
  for (int s = 0; s < 2; ++s) {
    const size_t T = (size_t)d.T[s];
    const bool on = T > 0;
    l.chunks[s] = (d.n[s] + kBwdRowChunk - 1) / kBwdRowChunk;
    l.w2t[s] = off;
    off += on ? round_up(F * C * 2, 256) : 0;
    l.w12t[s] = off;
    off += on ? round_up(2 * F * C * 2, 256) : 0;
    l.wfct[s] = off;
    off += on ? round_up(C * C * 2, 256) : 0;
    l.dag[s] = off;
    off += round_up(T * 2 * F * 2, 256);
    l.du[s] = off;
    off += round_up(T * C * 4, 256);
    l.dz[s] = off;
    off += round_up(T * C * 2, 256);
    l.modpart[s] = off;
    off += round_up((size_t)d.B * l.chunks[s] * 2 * C * 4, 256);
    wgrad_layout(d, d.F, d.C, &l.g2, &off, s);
    wgrad_layout(d, d.C, 2 * d.F, &l.g12, &off, s);
    wgrad_layout(d, d.C, d.C, &l.gfc, &off, s);
  }
  l.total = off;
  return l;
}

// Set up stream s of a weight-gradient GEMM (A = a^T, B = b^T over the tokens; output [N, M]) and its
// reduction: one split writes dw and db directly; more write partials that the reduction sums; an
// empty stream's dw and db (where given) are zeroed by a reduction over no partials.
void wgrad(jattn::GemmArgs& g, jattn::ReduceArgs& r, int s, const Sizes& d, const WGradLayout& wl, char* ws,
           const jattn::MatRef& a, const jattn::MatRef& b, int M, int N, float* dw, float* db) {
  const bool on = d.T[s] > 0, direct = wl.splits[s] == 1;
  jattn::GemmProblem& p = g.pr[s];
  p = problem(a, b, on ? M : 0, N, (int)d.T[s]);
  p.splits = wl.splits[s];
  p.kchunk = wl.kchunk[s];
  p.out[0] = direct ? static_cast<void*>(dw) : static_cast<void*>(ws + wl.part[s]);
  p.colsum = on && db ? (direct ? db : reinterpret_cast<float*>(ws + wl.cpart[s])) : nullptr;
  const bool reduce = !on || !direct;
  r.part[s] = reinterpret_cast<const float*>(ws + wl.part[s]);
  r.cpart[s] = on ? p.colsum : r.part[s];
  r.out[s] = dw;
  r.cout[s] = reduce ? (on ? (p.colsum ? db : nullptr) : db) : nullptr;
  r.count[s] = on ? wl.splits[s] : 0;
  r.len[s] = reduce && dw ? N * M : 0;
  r.inner[s] = 0;
  r.clen[s] = N;
}

}  // namespace

extern "C" {

size_t jattn_mlp_fwd_workspace_bytes(int B, int n_img, int n_txt, int C, int F) {
  Sizes z;
  if (check_sizes(B, n_img, n_txt, C, F, &z) != JATTN_SUCCESS) return 0;
  return fwd_layout(z).total;
}

size_t jattn_mlp_bwd_workspace_bytes(int B, int n_img, int n_txt, int C, int F) {
  Sizes z;
  if (check_sizes(B, n_img, n_txt, C, F, &z) != JATTN_SUCCESS) return 0;
  return bwd_layout(z).total;
}

jattn_status jattn_mlp_fwd(const void* const o[2], const void* const x[2], const float* const mod[2],
                           const void* const wfc[2], const float* const bfc[2], const void* const w12[2],
                           const float* const b12[2], const void* const w2[2], const float* const b2[2], int B,
                           int n_img, int n_txt, int C, int F, float eps, void* const out[2], void* workspace,
                           size_t workspace_bytes, const hipEvent_t* stage_events, int n_stage_events,
                           hipStream_t stream) {
  if (!o || !x || !mod || !wfc || !bfc || !w12 || !b12 || !w2 || !b2 || !out) return JATTN_ERROR_INVALID_VALUE;
  Sizes d;
  jattn_status st = check_sizes(B, n_img, n_txt, C, F, &d);
  if (st != JATTN_SUCCESS) return st;
  if (!std::isfinite(eps) || eps < 0.f) return JATTN_ERROR_INVALID_VALUE;
  if ((st = check_events(stage_events, n_stage_events, JATTN_MLP_FWD_STAGES)) != JATTN_SUCCESS) return st;
  const FwdLayout lay = fwd_layout(d);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < lay.total) return JATTN_ERROR_WORKSPACE;
  Range outs[3], ins[18];
  int no = 0, ni = 0;
  outs[no++] = {workspace, lay.total};
  for (int s = 0; s < 2; ++s) {
    if (d.T[s] == 0) continue;
    if (!ptr_ok(o[s]) || !ptr_ok(x[s]) || !ptr_ok(mod[s]) || !ptr_ok(wfc[s]) || !ptr_ok(w12[s]) || !ptr_ok(w2[s]) ||
        !ptr_ok(out[s]) || (bfc[s] && !aligned(bfc[s], 16)) || (b12[s] && !aligned(b12[s], 16)) ||
        (b2[s] && !aligned(b2[s], 16)))
      return JATTN_ERROR_INVALID_VALUE;
    const size_t act = (size_t)d.T[s] * C * 2;
    outs[no++] = {out[s], act};
    ins[ni++] = {o[s], act};
    ins[ni++] = {x[s], act};
    ins[ni++] = {mod[s], (size_t)B * 2 * C * 4};
    ins[ni++] = {wfc[s], (size_t)C * C * 2};
    ins[ni++] = {w12[s], (size_t)2 * F * C * 2};
    ins[ni++] = {w2[s], (size_t)C * F * 2};
    ins[ni++] = {bfc[s], bfc[s] ? (size_t)C * 4 : 0};
    ins[ni++] = {b12[s], b12[s] ? (size_t)2 * F * 4 : 0};
    ins[ni++] = {b2[s], b2[s] ? (size_t)C * 4 : 0};
  }
  if (!disjoint(outs, no, ins, ni)) return JATTN_ERROR_INVALID_VALUE;

  char* ws = static_cast<char*>(workspace);
  jattn::GemmArgs gfc{}, gsw{}, gdn{};
  jattn::ModulateArgs ma{};
  for (int s = 0; s < 2; ++s) {
    const bool on = d.T[s] > 0;
    const int64_t T = d.T[s];
    const void* dummy = workspace;  // (never read: an empty stream has no tiles)
    void* z = ws + lay.z[s];
    void* u = ws + lay.u[s];
    // fc: z = o Wfc^T + bfc
    gfc.pr[s] = problem(mat(on ? wfc[s] : dummy, nullptr, nullptr, C, C, C, C), mat(on ? o[s] : dummy, nullptr, nullptr, C, C, T, C),
                        C, (int)T, C);
    gfc.pr[s].out[0] = z;
    gfc.pr[s].out_seg = C;
    gfc.pr[s].bias = on ? bfc[s] : nullptr;
    // adaLN of z
    ma.x[s] = static_cast<const uint16_t*>(z);
    ma.mod[s] = on ? mod[s] : nullptr;
    ma.h[s] = static_cast<uint16_t*>(u);
    ma.stats[s] = reinterpret_cast<float*>(ws + lay.stats[s]);
    ma.n[s] = d.n[s] > 0 ? d.n[s] : 1;
    ma.T[s] = (int)T;
    // gate/up with SwiGLU: A = W12 rows j and F + j, B = u rows
    gsw.pr[s] = problem(mat(on ? w12[s] : dummy, nullptr, nullptr, C, C, 2 * (int64_t)F, C),
                        mat(u, nullptr, nullptr, C, C, T, C), 2 * F, (int)T, C);
    gsw.pr[s].out[0] = ws + lay.ag[s];
    gsw.pr[s].out[1] = ws + lay.hid[s];
    gsw.pr[s].bias = on ? b12[s] : nullptr;
    gsw.pr[s].pair_off = F;
    // down projection with bias and residual: out = x + hid W2^T + b2
    gdn.pr[s] = problem(mat(on ? w2[s] : dummy, nullptr, nullptr, F, F, C, F),
                        mat(ws + lay.hid[s], nullptr, nullptr, F, F, T, F), C, (int)T, F);
    gdn.pr[s].out[0] = on ? out[s] : nullptr;
    gdn.pr[s].out_seg = C;
    gdn.pr[s].bias = on ? b2[s] : nullptr;
    gdn.pr[s].aux = on ? static_cast<const uint16_t*>(x[s]) : nullptr;
  }
  ma.C = C;
  ma.eps = eps;
  finish(gfc, jattn::kQkvMA, jattn::kQkvMB);
  finish(gsw, jattn::kSwigluMA, jattn::kSwigluMB);
  finish(gdn, jattn::kQkvMA, jattn::kQkvMB);

  jattn::launch_qkv_gemm(gfc, stream);
  if (!stage_done(0, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  jattn::launch_modulate(ma, stream);
  if (!stage_done(1, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  jattn::launch_swiglu_gemm(gsw, stream);
  if (!stage_done(2, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  jattn::launch_qkv_gemm(gdn, stream);
  if (!stage_done(3, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  return JATTN_SUCCESS;
}

jattn_status jattn_mlp_bwd(const void* const o[2], const float* const mod[2], const void* const wfc[2],
                           const void* const w12[2], const void* const w2[2], const void* const dout[2], int B,
                           int n_img, int n_txt, int C, int F, void* const d_o[2], float* const dmod[2],
                           float* const dwfc[2], float* const dbfc[2], float* const dw12[2], float* const db12[2],
                           float* const dw2[2], float* const db2[2], const void* fwd_workspace,
                           size_t fwd_workspace_bytes, void* workspace, size_t workspace_bytes,
                           const hipEvent_t* stage_events, int n_stage_events, hipStream_t stream) {
  if (!o || !mod || !wfc || !w12 || !w2 || !dout || !d_o || !dmod || !dwfc || !dbfc || !dw12 || !db12 || !dw2 || !db2)
    return JATTN_ERROR_INVALID_VALUE;
  Sizes d;
  jattn_status st = check_sizes(B, n_img, n_txt, C, F, &d);
  if (st != JATTN_SUCCESS) return st;
  if ((st = check_events(stage_events, n_stage_events, JATTN_MLP_BWD_STAGES)) != JATTN_SUCCESS) return st;
  const FwdLayout fl = fwd_layout(d);
  const BwdLayout bl = bwd_layout(d);
  if (!fwd_workspace || !aligned(fwd_workspace, 256) || fwd_workspace_bytes < fl.total) return JATTN_ERROR_WORKSPACE;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < bl.total) return JATTN_ERROR_WORKSPACE;
  Range outs[17], ins[14];
  int no = 0, ni = 0;
  outs[no++] = {workspace, bl.total};
  ins[ni++] = {fwd_workspace, fl.total};
  for (int s = 0; s < 2; ++s) {
    float* const grads[6] = {dmod[s], dwfc[s], dbfc[s], dw12[s], db12[s], dw2[s]};
    const size_t gbytes[7] = {(size_t)B * 2 * C * 4, (size_t)C * C * 4, (size_t)C * 4, (size_t)2 * F * C * 4,
                              (size_t)2 * F * 4, (size_t)C * F * 4, (size_t)C * 4};
    for (int i = 0; i < 6; ++i)
      if (grads[i] && !aligned(grads[i], 16)) return JATTN_ERROR_INVALID_VALUE;
    if (db2[s] && !aligned(db2[s], 16)) return JATTN_ERROR_INVALID_VALUE;
    for (int i = 0; i < 6; ++i) outs[no++] = {grads[i], grads[i] ? gbytes[i] : 0};
    outs[no++] = {db2[s], db2[s] ? gbytes[6] : 0};
    if (d.T[s] == 0) continue;  // (an empty stream's parameter gradients, where given, are zeroed)
    if (!ptr_ok(o[s]) || !ptr_ok(mod[s]) || !ptr_ok(wfc[s]) || !ptr_ok(w12[s]) || !ptr_ok(w2[s]) || !ptr_ok(dout[s]) ||
        !ptr_ok(d_o[s]) || !dmod[s] || !dwfc[s] || !dw12[s] || !dw2[s])
      return JATTN_ERROR_INVALID_VALUE;
    const size_t act = (size_t)d.T[s] * C * 2;
    outs[no++] = {d_o[s], act};
    ins[ni++] = {o[s], act};
    ins[ni++] = {mod[s], (size_t)B * 2 * C * 4};
    ins[ni++] = {wfc[s], (size_t)C * C * 2};
    ins[ni++] = {w12[s], (size_t)2 * F * C * 2};
    ins[ni++] = {w2[s], (size_t)C * F * 2};
    ins[ni++] = {dout[s], act};
  }
  if (!disjoint(outs, no, ins, ni)) return JATTN_ERROR_INVALID_VALUE;

  const char* fws = static_cast<const char*>(fwd_workspace);
  char* ws = static_cast<char*>(workspace);
  jattn::TransposeArgs ta{};
  jattn::GemmArgs ghid{}, gw2{}, gdu{}, gw12{}, gdo{}, gwfc{};
  jattn::RowsBwdArgs ra{};
  jattn::ReduceArgs rm{}, r2{}, r12{}, rfc{};
  auto add_transpose = [&](const void* src, void* dst, int rows, int cols) {
    ta.src[ta.n] = static_cast<const uint16_t*>(src);
    ta.dst[ta.n] = static_cast<uint16_t*>(dst);
    ta.rows[ta.n] = rows;
    ta.cols[ta.n] = cols;
    ta.start[ta.n + 1] = ta.start[ta.n] + (rows / 64) * (cols / 64);
    ++ta.n;
  };
  for (int s = 0; s < 2; ++s) {
    const bool on = d.T[s] > 0;
    const int64_t T = d.T[s];
    const void* dummy = workspace;  // (never read: an empty stream has no tiles)
    void* w2t = ws + bl.w2t[s];
    void* w12t = ws + bl.w12t[s];
    void* wfct = ws + bl.wfct[s];
    void* dag = ws + bl.dag[s];
    void* dz = ws + bl.dz[s];
    const void* ag = fws + fl.ag[s];
    const void* hid = fws + fl.hid[s];
    const void* u = fws + fl.u[s];
    const void* dy = on ? dout[s] : dummy;
    if (on) {
      add_transpose(w2[s], w2t, C, F);         // W2 [C, F] -> [F, C]
      add_transpose(w12[s], w12t, 2 * F, C);   // W12 [2F, C] -> [C, 2F]
      add_transpose(wfc[s], wfct, C, C);       // Wfc -> Wfc^T
    }
    // d(hid) = dout W2, then the SwiGLU backward: d[a|g]
    ghid.pr[s] = problem(mat(on ? w2t : dummy, nullptr, nullptr, C, C, F, C), mat(dy, nullptr, nullptr, C, C, T, C), F,
                         (int)T, C);
    ghid.pr[s].out[0] = dag;
    ghid.pr[s].aux = static_cast<const uint16_t*>(ag);
    // dW2 = dout^T hid (and db2)
    wgrad(gw2, r2, s, d, bl.g2, ws, mat(hid, nullptr, nullptr, F, F, T, F), mat(dy, nullptr, nullptr, C, C, T, C), F, C,
          dw2[s], db2[s]);
    // du = d[a|g] W12
    gdu.pr[s] = problem(mat(on ? w12t : dummy, nullptr, nullptr, 2 * F, 2 * F, C, 2 * F),
                        mat(dag, nullptr, nullptr, 2 * F, 2 * F, T, 2 * F), C, (int)T, 2 * F);
    gdu.pr[s].out[0] = ws + bl.du[s];
    gdu.pr[s].out_seg = C;
    // dW12 = d[a|g]^T u (and db12)
    wgrad(gw12, r12, s, d, bl.g12, ws, mat(u, nullptr, nullptr, C, C, T, C),
          mat(dag, nullptr, nullptr, 2 * F, 2 * F, T, 2 * F), C, 2 * F, dw12[s], db12[s]);
    // LayerNorm backward: dz and the modulation partials
    ra.x[s] = static_cast<const uint16_t*>(static_cast<const void*>(fws + fl.z[s]));
    ra.mod[s] = on ? mod[s] : nullptr;
    ra.stats[s] = reinterpret_cast<const float*>(fws + fl.stats[s]);
    ra.dh[s] = reinterpret_cast<const float*>(ws + bl.du[s]);
    ra.dx[s] = static_cast<uint16_t*>(dz);
    ra.part[s] = reinterpret_cast<float*>(ws + bl.modpart[s]);
    ra.n[s] = d.n[s] > 0 ? d.n[s] : 1;
    ra.chunks[s] = on ? bl.chunks[s] : 0;
    rm.part[s] = ra.part[s];
    rm.out[s] = dmod[s];
    rm.count[s] = on ? bl.chunks[s] : 0;
    rm.len[s] = dmod[s] ? B * 2 * C : 0;
    rm.inner[s] = 2 * C;
    // do = dz Wfc
    gdo.pr[s] = problem(mat(on ? wfct : dummy, nullptr, nullptr, C, C, C, C), mat(dz, nullptr, nullptr, C, C, T, C), C,
                        (int)T, C);
    gdo.pr[s].out[0] = on ? d_o[s] : nullptr;
    gdo.pr[s].out_seg = C;
    // dWfc = dz^T o (and dbfc)
    wgrad(gwfc, rfc, s, d, bl.gfc, ws, mat(on ? o[s] : dummy, nullptr, nullptr, C, C, T, C),
          mat(dz, nullptr, nullptr, C, C, T, C), C, C, dwfc[s], dbfc[s]);
  }
  ra.B = B;
  ra.C = C;
  ra.blocks0 = B * ra.chunks[0];
  finish(ghid, jattn::kDhMA, jattn::kDhMB);
  finish(gw2, jattn::kDwMA, jattn::kDwMB);
  finish(gdu, jattn::kDhMA, jattn::kDhMB);
  finish(gw12, jattn::kDwMA, jattn::kDwMB);
  finish(gdo, jattn::kQkvMA, jattn::kQkvMB);
  finish(gwfc, jattn::kDwMA, jattn::kDwMB);

  jattn::launch_transpose_w(ta, stream);
  if (!stage_done(0, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  jattn::launch_dhid_gemm(ghid, stream);
  if (!stage_done(1, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  jattn::launch_dw_gemm(gw2, stream);
  if (!stage_done(2, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  jattn::launch_dh_gemm(gdu, stream);
  if (!stage_done(3, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  jattn::launch_dw_gemm(gw12, stream);
  if (!stage_done(4, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  jattn::launch_rows_bwd(ra, stream);
  if (!stage_done(5, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  jattn::launch_qkv_gemm(gdo, stream);
  if (!stage_done(6, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  jattn::launch_dw_gemm(gwfc, stream);
  if (!stage_done(7, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  jattn::launch_mod_reduce(rm, stream);
  if (!launched()) return JATTN_ERROR_HIP;
  jattn::launch_w_reduce(r2, stream);
  if (!launched()) return JATTN_ERROR_HIP;
  jattn::launch_w_reduce(r12, stream);
  if (!launched()) return JATTN_ERROR_HIP;
  jattn::launch_w_reduce(rfc, stream);
  if (!stage_done(8, stage_events, n_stage_events, stream)) return JATTN_ERROR_HIP;
  return JATTN_SUCCESS;
}

}  // extern "C"
