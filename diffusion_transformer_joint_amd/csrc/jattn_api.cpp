// C ABI of libjattn.so (declared in include/jattn.h): host-side argument validation, workspace
// sizing and kernel dispatch. Every check runs before the first HIP call, so invalid calls never
// touch the device.
#include "jattn.h"

#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "jattn_launch.h"

namespace {

using jattn::kBwdRowsPerBlock;

constexpr int kAbiVersion = 9;

bool supported_head_dim(int D) { return D % 8 == 0 && D >= 32 && D <= 128; }

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

// Normalised key rows and pre-scaled normalised query rows (bf16, one [L, D] block per (sequence,
// head): [B, H, L, D] for fixed-length batches, total * H rows for packed ones), the two row
// statistics (fp32, [B, H, lp] with lp = L rounded up to whole row blocks; packed batches
// (total + 128 B) * H rows, see SeqGeom) and the per-workgroup partial sums of the gain gradients
// (fp32, [kPartSets, D, items]), each 256-byte aligned. L is the longest sequence; total < 0 means
// a fixed-length batch (total = B L).
WorkspaceLayout workspace_layout(int B, int L, int H, int D, int64_t total = -1) {
  const size_t nblk = (L + kBwdRowsPerBlock - 1) / kBwdRowsPerBlock;
  const size_t items = (size_t)B * H * nblk, lp = nblk * kBwdRowsPerBlock;
  const size_t nrows = total < 0 ? (size_t)B * L : (size_t)total;
  const size_t rows = round_up(nrows * H * D * 2, 256),
               stats = round_up((total < 0 ? (size_t)B * H * lp : (nrows + 128 * (size_t)B) * H) * 4, 256),
               parts = round_up(jattn::kPartSets * items * D * sizeof(float), 256);
  WorkspaceLayout w;
  w.kr = 0;
  w.qs = w.kr + rows;
  w.nlse2 = w.qs + rows;
  w.ndelta = w.nlse2 + stats;
  w.part = w.ndelta + stats;
  w.total = w.part + parts;
  return w;
}

// Kernel arguments of a validated call. Tensors come as (block 0, block 1) pointer pairs: rows
// [0, n0) of each sequence in block 0, the rest in block 1 (the joint entry points pass n0 = L).
jattn_status run_fwd(jattn::Variant var, const void* const q[2], const void* const k[2], const void* const v[2],
                     const float* gains, const int32_t* valid_len, const int32_t* cu_seqlens, int total, int B,
                     int L, int n0, int H, int D,
                     float softmax_scale, float eps, void* const out[2], float* lse, void* workspace,
                     const hipEvent_t* stage_events, int n_stage_events, hipStream_t stream, int wl = 0, int wr = 0) {
  auto in = [](const void* p) { return static_cast<const uint16_t*>(p); };
  jattn::FwdArgs a;
  a.q = in(q[0]);
  a.k = in(k[0]);
  a.v = in(v[0]);
  a.q1 = in(q[1]);
  a.k1 = in(k[1]);
  a.v1 = in(v[1]);
  a.kr = static_cast<const uint16_t*>(workspace);
  a.gains = gains;
  a.valid_len = valid_len;
  a.cu_seqlens = cu_seqlens;
  a.out = static_cast<uint16_t*>(out[0]);
  a.out1 = static_cast<uint16_t*>(out[1]);
  a.lse = lse;
  a.B = B;
  a.L = L;
  a.H = H;
  a.n0 = n0;
  a.total = total;
  a.wl = wl;
  a.wr = wr;
  a.c = softmax_scale * 1.4426950408889634f;
  a.eps = eps;
  a.nblk = (L + jattn::fwd_rows_per_block(D) - 1) / jattn::fwd_rows_per_block(D);
  a.items = B * H * a.nblk;
  return jattn::launch_fwd(D, var, a, stage_events, n_stage_events, stream) == hipSuccess ? JATTN_SUCCESS
                                                                                       : JATTN_ERROR_HIP;
}

jattn_status run_bwd(jattn::Variant var, const void* const q[2], const void* const k[2], const void* const v[2],
                     const float* gains, const int32_t* valid_len, const int32_t* cu_seqlens, int total,
                     const void* const out[2], const float* lse, const void* const dout[2], int B, int L, int n0,
                     int H, int D, float softmax_scale, float eps,
                     void* const dq[2], void* const dk[2], void* const dv[2], float* dgains, void* workspace,
                     const void* fwd_workspace, const hipEvent_t* stage_events, int n_stage_events,
                     hipStream_t stream, int win_left = 0, int win_right = 0) {
  auto in = [](const void* p) { return static_cast<const uint16_t*>(p); };
  auto outp = [](void* p) { return static_cast<uint16_t*>(p); };
  const WorkspaceLayout wl = workspace_layout(B, L, H, D, var == jattn::kVarlen ? total : -1);
  char* ws = static_cast<char*>(workspace);
  jattn::BwdArgs a;
  a.q = in(q[0]);
  a.k = in(k[0]);
  a.v = in(v[0]);
  a.q1 = in(q[1]);
  a.k1 = in(k[1]);
  a.v1 = in(v[1]);
  a.gains = gains;
  a.valid_len = valid_len;
  a.cu_seqlens = cu_seqlens;
  a.out = in(out[0]);
  a.out1 = in(out[1]);
  a.lse = lse;
  a.dout = in(dout[0]);
  a.dout1 = in(dout[1]);
  a.dq = outp(dq[0]);
  a.dk = outp(dk[0]);
  a.dv = outp(dv[0]);
  a.dq1 = outp(dq[1]);
  a.dk1 = outp(dk[1]);
  a.dv1 = outp(dv[1]);
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
  a.n0 = n0;
  a.total = total;
  a.wl = win_left;
  a.wr = win_right;
  a.scale = softmax_scale;
  a.c = softmax_scale * 1.4426950408889634f;
  a.eps = eps;
  a.nblk = (L + kBwdRowsPerBlock - 1) / kBwdRowsPerBlock;
  a.items = B * H * a.nblk;
  a.lp = a.nblk * kBwdRowsPerBlock;
  return jattn::launch_bwd(D, var, a, fwd_workspace == nullptr, stage_events, n_stage_events, stream) ==
                 hipSuccess
             ? JATTN_SUCCESS
             : JATTN_ERROR_HIP;
}

// A window bound as the kernels take it: negative (no bound) or past the sequence -> L.
int window_bound(int w, int L) { return w < 0 || w > L ? L : w; }

// Sizes of a packed variable-length call: B sequences, the longest max_seqlen rows, total token rows.
jattn_status check_varlen_sizes(int B, int max_seqlen, int total, int H, int D) {
  if (total < 1) return JATTN_ERROR_INVALID_VALUE;
  const jattn_status st = check_sizes(B, max_seqlen, H, D);
  if (st != JATTN_SUCCESS) return st;
  if (B > 65535) return JATTN_ERROR_NOT_SUPPORTED;  // (the key normalisation puts the sequence in grid y)
  if ((int64_t)total * H * D >= (int64_t(1) << 39) || ((int64_t)total + 128 * (int64_t)B) * H >= (int64_t(1) << 31))
    return JATTN_ERROR_NOT_SUPPORTED;
  return JATTN_SUCCESS;
}

// Sizes of a two-stream call: N_img, N_txt >= 0 with at least one token.
jattn_status check_stream_sizes(int B, int n_img, int n_txt, int H, int D, int* L) {
  if (n_img < 0 || n_txt < 0) return JATTN_ERROR_INVALID_VALUE;
  const int64_t l = (int64_t)n_img + n_txt;
  if (l > INT_MAX) return JATTN_ERROR_NOT_SUPPORTED;
  *L = (int)l;
  return check_sizes(B, *L, H, D);
}

// A (image, text) pointer pair: the host array exists, and each pointer of a non-empty stream is
// non-null and 16-byte aligned (a pointer of an empty stream is ignored).
bool pair_ok(const void* const p[2], int n_img, int n_txt) {
  if (!p) return false;
  if (n_img > 0 && (!p[0] || !aligned(p[0], 16))) return false;
  if (n_txt > 0 && (!p[1] || !aligned(p[1], 16))) return false;
  return true;
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

// The joint forward, optionally with a local window (window_left / window_right < 0: unbounded).
static jattn_status joint_fwd(bool windowed, int window_left, int window_right, const void* q, const void* k,
                              const void* v, const float* gains, const int32_t* valid_len, int B, int L, int H, int D,
                              float softmax_scale, float eps, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, const hipEvent_t* stage_events, int n_stage_events,
                              hipStream_t stream) {
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

  const void* const qp[2] = {q, nullptr};
  const void* const kp[2] = {k, nullptr};
  const void* const vp[2] = {v, nullptr};
  void* const op[2] = {out, nullptr};
  return run_fwd(windowed ? jattn::kWindow : jattn::kJoint, qp, kp, vp, gains, valid_len, nullptr, B * L, B, L, L, H, D,
                 softmax_scale, eps, op, lse, workspace, stage_events, n_stage_events, stream,
                 window_bound(window_left, L), window_bound(window_right, L));
}

jattn_status jattn_fwd_ex(const void* q, const void* k, const void* v, const float* gains,
                          const int32_t* valid_len, int B, int L, int H, int D, float softmax_scale,
                          float eps, void* out, float* lse, void* workspace, size_t workspace_bytes,
                          const hipEvent_t* stage_events, int n_stage_events, hipStream_t stream) {
  return joint_fwd(false, -1, -1, q, k, v, gains, valid_len, B, L, H, D, softmax_scale, eps, out, lse, workspace,
                   workspace_bytes, stage_events, n_stage_events, stream);
}

jattn_status jattn_fwd_window(const void* q, const void* k, const void* v, const float* gains,
                              const int32_t* valid_len, int B, int L, int H, int D, float softmax_scale, float eps,
                              int window_left, int window_right, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, const hipEvent_t* stage_events, int n_stage_events,
                              hipStream_t stream) {
  return joint_fwd(true, window_left, window_right, q, k, v, gains, valid_len, B, L, H, D, softmax_scale, eps, out, lse,
                   workspace, workspace_bytes, stage_events, n_stage_events, stream);
}

jattn_status jattn_fwd(const void* q, const void* k, const void* v, const float* gains,
                       const int32_t* valid_len, int B, int L, int H, int D, float softmax_scale,
                       float eps, void* out, float* lse, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  return jattn_fwd_ex(q, k, v, gains, valid_len, B, L, H, D, softmax_scale, eps, out, lse, workspace,
                      workspace_bytes, nullptr, 0, stream);
}

}  // extern "C"

// Device-resident scratch of jattn_fwd_noalloc: the normalised key rows of the last call on each GPU.
// Each device holds its own copy for the life of the process; host code reaches it only through the
// per-device address that hipGetSymbolAddress returns (the array's name is a host-side stand-in).
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint16_t scratch[kNoallocScratchBytes / sizeof(uint16_t)];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The address of this device's scratch array, looked up once per device with that device current.
hipError_t scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return *ptr ? hipSuccess : hipErrorInvalidSymbol;
}
}  // namespace

extern "C" {

size_t jattn_fwd_noalloc_max_scratch_bytes(void) { return kNoallocScratchBytes; }

jattn_status jattn_fwd_noalloc(const void* q, const void* k, const void* v, const float* gains,
                               const int32_t* valid_len, int B, int L, int H, int D, float softmax_scale,
                               float eps, void* out, float* lse, hipStream_t stream) {
  // every check before the first HIP call, as for jattn_fwd
  if (!q || !k || !v || !gains || !out || !lse) return JATTN_ERROR_INVALID_VALUE;
  const jattn_status st = check_sizes(B, L, H, D);
  if (st != JATTN_SUCCESS) return st;
  if (!std::isfinite(softmax_scale) || !std::isfinite(eps) || eps < 0.f) return JATTN_ERROR_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(gains, 4) ||
      !aligned(lse, 4) || !aligned(valid_len, 4))
    return JATTN_ERROR_INVALID_VALUE;
  if (jattn_fwd_workspace_bytes(B, L, H, D) > kNoallocScratchBytes) return JATTN_ERROR_WORKSPACE;
  const size_t tb = (size_t)B * L * H * D * 2, lb = (size_t)B * H * L * 4;
  const Range ins[] = {{q, tb}, {k, tb}, {v, tb}, {gains, (size_t)2 * D * 4}, {valid_len, (size_t)B * 4}};
  const Range outs[] = {{out, tb}, {lse, lb}};
  if (!outputs_disjoint(outs, 2, ins, 5)) return JATTN_ERROR_INVALID_VALUE;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return JATTN_ERROR_HIP;
  const void* const qp[2] = {q, nullptr};
  const void* const kp[2] = {k, nullptr};
  const void* const vp[2] = {v, nullptr};
  void* const op[2] = {out, nullptr};
  return run_fwd(jattn::kJoint, qp, kp, vp, gains, valid_len, nullptr, B * L, B, L, L, H, D, softmax_scale, eps, op,
                 lse, ws, nullptr, 0, stream);
}

jattn_status jattn_bwd(const void* q, const void* k, const void* v, const float* gains,
                       const int32_t* valid_len, const void* out, const float* lse, const void* dout,
                       int B, int L, int H, int D, float softmax_scale, float eps, void* dq, void* dk,
                       void* dv, float* dgains, void* workspace, size_t workspace_bytes,
                       const void* fwd_workspace, hipStream_t stream) {
  return jattn_bwd_ex(q, k, v, gains, valid_len, out, lse, dout, B, L, H, D, softmax_scale, eps, dq, dk, dv,
                      dgains, workspace, workspace_bytes, fwd_workspace, nullptr, 0, stream);
}

// The joint backward, optionally with a local window.
static jattn_status joint_bwd(bool windowed, int window_left, int window_right, const void* q, const void* k,
                              const void* v, const float* gains, const int32_t* valid_len, const void* out,
                              const float* lse, const void* dout, int B, int L, int H, int D, float softmax_scale,
                              float eps, void* dq, void* dk, void* dv, float* dgains, void* workspace,
                              size_t workspace_bytes, const void* fwd_workspace, const hipEvent_t* stage_events,
                              int n_stage_events, hipStream_t stream) {
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

  const void* const qp[2] = {q, nullptr};
  const void* const kp[2] = {k, nullptr};
  const void* const vp[2] = {v, nullptr};
  const void* const op[2] = {out, nullptr};
  const void* const dop[2] = {dout, nullptr};
  void* const dqp[2] = {dq, nullptr};
  void* const dkp[2] = {dk, nullptr};
  void* const dvp[2] = {dv, nullptr};
  return run_bwd(windowed ? jattn::kWindow : jattn::kJoint, qp, kp, vp, gains, valid_len, nullptr, B * L, op, lse, dop,
                 B, L, L, H, D, softmax_scale, eps, dqp, dkp, dvp, dgains, workspace, fwd_workspace, stage_events,
                 n_stage_events, stream, window_bound(window_left, L), window_bound(window_right, L));
}

jattn_status jattn_bwd_ex(const void* q, const void* k, const void* v, const float* gains,
                          const int32_t* valid_len, const void* out, const float* lse, const void* dout,
                          int B, int L, int H, int D, float softmax_scale, float eps, void* dq, void* dk,
                          void* dv, float* dgains, void* workspace, size_t workspace_bytes,
                          const void* fwd_workspace, const hipEvent_t* stage_events, int n_stage_events,
                          hipStream_t stream) {
  return joint_bwd(false, -1, -1, q, k, v, gains, valid_len, out, lse, dout, B, L, H, D, softmax_scale, eps, dq, dk, dv,
                   dgains, workspace, workspace_bytes, fwd_workspace, stage_events, n_stage_events, stream);
}

jattn_status jattn_bwd_window(const void* q, const void* k, const void* v, const float* gains,
                              const int32_t* valid_len, const void* out, const float* lse, const void* dout, int B,
                              int L, int H, int D, float softmax_scale, float eps, int window_left, int window_right,
                              void* dq, void* dk, void* dv, float* dgains, void* workspace, size_t workspace_bytes,
                              const void* fwd_workspace, const hipEvent_t* stage_events, int n_stage_events,
                              hipStream_t stream) {
  return joint_bwd(true, window_left, window_right, q, k, v, gains, valid_len, out, lse, dout, B, L, H, D,
                   softmax_scale, eps, dq, dk, dv, dgains, workspace, workspace_bytes, fwd_workspace, stage_events,
                   n_stage_events, stream);
}

jattn_status jattn_fwd_streams(const void* const q[2], const void* const k[2], const void* const v[2],
                               const float* gains, const int32_t* valid_len, int B, int n_img, int n_txt, int H,
                               int D, float softmax_scale, float eps, void* const out[2], float* lse,
                               void* workspace, size_t workspace_bytes, const hipEvent_t* stage_events,
                               int n_stage_events, hipStream_t stream) {
  if (n_stage_events < 0 || n_stage_events > JATTN_FWD_STAGES || (n_stage_events > 0 && !stage_events))
    return JATTN_ERROR_INVALID_VALUE;
  if (!q || !k || !v || !out || !gains || !lse) return JATTN_ERROR_INVALID_VALUE;
  int L = 0;
  const jattn_status st = check_stream_sizes(B, n_img, n_txt, H, D, &L);
  if (st != JATTN_SUCCESS) return st;
  if (!pair_ok(q, n_img, n_txt) || !pair_ok(k, n_img, n_txt) || !pair_ok(v, n_img, n_txt) ||
      !pair_ok(out, n_img, n_txt))
    return JATTN_ERROR_INVALID_VALUE;
  if (!std::isfinite(softmax_scale) || !std::isfinite(eps) || eps < 0.f) return JATTN_ERROR_INVALID_VALUE;
  if (!aligned(gains, 4) || !aligned(lse, 4) || !aligned(valid_len, 4)) return JATTN_ERROR_INVALID_VALUE;
  const size_t wsb = jattn_fwd_workspace_bytes(B, L, H, D);
  if (!workspace || workspace_bytes < wsb) return JATTN_ERROR_WORKSPACE;
  if (!aligned(workspace, 256)) return JATTN_ERROR_INVALID_VALUE;
  const size_t ti = (size_t)B * n_img * H * D * 2, tt = (size_t)B * n_txt * H * D * 2, lb = (size_t)B * H * L * 4;
  const Range ins[] = {{q[0], ti}, {q[1], tt}, {k[0], ti}, {k[1], tt}, {v[0], ti}, {v[1], tt},
                       {gains, (size_t)4 * D * 4}, {valid_len, (size_t)B * 4}};
  const Range outs[] = {{out[0], ti}, {out[1], tt}, {lse, lb}, {workspace, wsb}};
  if (!outputs_disjoint(outs, 4, ins, 8)) return JATTN_ERROR_INVALID_VALUE;
  // (pointers of an empty stream are never dereferenced; pass them on as null)
  auto pick = [&](const void* const p[2], int s) -> const void* { return (s == 0 ? n_img : n_txt) > 0 ? p[s] : nullptr; };
  const void* const qp[2] = {pick(q, 0), pick(q, 1)};
  const void* const kp[2] = {pick(k, 0), pick(k, 1)};
  const void* const vp[2] = {pick(v, 0), pick(v, 1)};
  void* const op[2] = {n_img > 0 ? out[0] : nullptr, n_txt > 0 ? out[1] : nullptr};
  return run_fwd(jattn::kStreams, qp, kp, vp, gains, valid_len, nullptr, B * L, B, L, n_img, H, D, softmax_scale,
                 eps, op, lse, workspace, stage_events, n_stage_events, stream);
}

jattn_status jattn_bwd_streams(const void* const q[2], const void* const k[2], const void* const v[2],
                               const float* gains, const int32_t* valid_len, const void* const out[2],
                               const float* lse, const void* const dout[2], int B, int n_img, int n_txt, int H,
                               int D, float softmax_scale, float eps, void* const dq[2], void* const dk[2],
                               void* const dv[2], float* dgains, void* workspace, size_t workspace_bytes,
                               const void* fwd_workspace, const hipEvent_t* stage_events, int n_stage_events,
                               hipStream_t stream) {
  if (n_stage_events < 0 || n_stage_events > JATTN_BWD_STAGES || (n_stage_events > 0 && !stage_events))
    return JATTN_ERROR_INVALID_VALUE;
  if (!q || !k || !v || !out || !dout || !dq || !dk || !dv || !gains || !lse || !dgains)
    return JATTN_ERROR_INVALID_VALUE;
  int L = 0;
  const jattn_status st = check_stream_sizes(B, n_img, n_txt, H, D, &L);
  if (st != JATTN_SUCCESS) return st;
  if (!pair_ok(q, n_img, n_txt) || !pair_ok(k, n_img, n_txt) || !pair_ok(v, n_img, n_txt) ||
      !pair_ok(out, n_img, n_txt) || !pair_ok(dout, n_img, n_txt) || !pair_ok(dq, n_img, n_txt) ||
      !pair_ok(dk, n_img, n_txt) || !pair_ok(dv, n_img, n_txt))
    return JATTN_ERROR_INVALID_VALUE;
  if (!std::isfinite(softmax_scale) || !std::isfinite(eps) || eps < 0.f) return JATTN_ERROR_INVALID_VALUE;
  if (!aligned(gains, 4) || !aligned(lse, 4) || !aligned(dgains, 4) || !aligned(valid_len, 4))
    return JATTN_ERROR_INVALID_VALUE;
  const WorkspaceLayout wl = workspace_layout(B, L, H, D);
  if (!workspace || workspace_bytes < wl.total) return JATTN_ERROR_WORKSPACE;
  if (!aligned(workspace, 256) || !aligned(fwd_workspace, 256)) return JATTN_ERROR_INVALID_VALUE;
  const size_t ti = (size_t)B * n_img * H * D * 2, tt = (size_t)B * n_txt * H * D * 2, lb = (size_t)B * H * L * 4;
  const size_t fwb = fwd_workspace ? jattn_fwd_workspace_bytes(B, L, H, D) : 0, gb = (size_t)4 * D * 4;
  const Range ins[] = {{q[0], ti},   {q[1], tt},   {k[0], ti},    {k[1], tt},        {v[0], ti},
                       {v[1], tt},   {out[0], ti}, {out[1], tt},  {dout[0], ti},     {dout[1], tt},
                       {gains, gb},  {lse, lb},    {valid_len, (size_t)B * 4},      {fwd_workspace, fwb}};
  const Range outs[] = {{dq[0], ti}, {dq[1], tt}, {dk[0], ti}, {dk[1], tt}, {dv[0], ti}, {dv[1], tt},
                        {dgains, gb}, {workspace, wl.total}};
  if (!outputs_disjoint(outs, 8, ins, 14)) return JATTN_ERROR_INVALID_VALUE;
  auto pick = [&](const void* const p[2], int s) -> const void* { return (s == 0 ? n_img : n_txt) > 0 ? p[s] : nullptr; };
  auto pickw = [&](void* const p[2], int s) -> void* { return (s == 0 ? n_img : n_txt) > 0 ? p[s] : nullptr; };
  const void* const qp[2] = {pick(q, 0), pick(q, 1)};
  const void* const kp[2] = {pick(k, 0), pick(k, 1)};
  const void* const vp[2] = {pick(v, 0), pick(v, 1)};
  const void* const op[2] = {pick(out, 0), pick(out, 1)};
  const void* const dop[2] = {pick(dout, 0), pick(dout, 1)};
  void* const dqp[2] = {pickw(dq, 0), pickw(dq, 1)};
  void* const dkp[2] = {pickw(dk, 0), pickw(dk, 1)};
  void* const dvp[2] = {pickw(dv, 0), pickw(dv, 1)};
  return run_bwd(jattn::kStreams, qp, kp, vp, gains, valid_len, nullptr, B * L, op, lse, dop, B, L, n_img, H, D,
                 softmax_scale, eps, dqp, dkp, dvp, dgains, workspace, fwd_workspace, stage_events, n_stage_events,
                 stream);
}

size_t jattn_varlen_fwd_workspace_bytes(int B, int max_seqlen, int total, int H, int D) {
  if (check_varlen_sizes(B, max_seqlen, total, H, D) != JATTN_SUCCESS) return 0;
  return round_up((size_t)total * H * D * 2, 256);  // the normalised key rows
}

size_t jattn_varlen_bwd_workspace_bytes(int B, int max_seqlen, int total, int H, int D) {
  if (check_varlen_sizes(B, max_seqlen, total, H, D) != JATTN_SUCCESS) return 0;
  return workspace_layout(B, max_seqlen, H, D, total).total;
}

jattn_status jattn_fwd_varlen(const void* q, const void* k, const void* v, const float* gains,
                              const int32_t* cu_seqlens, int B, int max_seqlen, int total, int H, int D,
                              float softmax_scale, float eps, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, const hipEvent_t* stage_events, int n_stage_events,
                              hipStream_t stream) {
  if (n_stage_events < 0 || n_stage_events > JATTN_FWD_STAGES || (n_stage_events > 0 && !stage_events))
    return JATTN_ERROR_INVALID_VALUE;
  if (!q || !k || !v || !gains || !cu_seqlens || !out || !lse) return JATTN_ERROR_INVALID_VALUE;
  const jattn_status st = check_varlen_sizes(B, max_seqlen, total, H, D);
  if (st != JATTN_SUCCESS) return st;
  if (!std::isfinite(softmax_scale) || !std::isfinite(eps) || eps < 0.f) return JATTN_ERROR_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(gains, 4) ||
      !aligned(lse, 4) || !aligned(cu_seqlens, 4))
    return JATTN_ERROR_INVALID_VALUE;
  const size_t wsb = jattn_varlen_fwd_workspace_bytes(B, max_seqlen, total, H, D);
  if (!workspace || workspace_bytes < wsb) return JATTN_ERROR_WORKSPACE;
  if (!aligned(workspace, 256)) return JATTN_ERROR_INVALID_VALUE;
  const size_t tb = (size_t)total * H * D * 2, lb = (size_t)total * H * 4;
  const Range ins[] = {{q, tb}, {k, tb}, {v, tb}, {gains, (size_t)2 * D * 4}, {cu_seqlens, (size_t)(B + 1) * 4}};
  const Range outs[] = {{out, tb}, {lse, lb}, {workspace, wsb}};
  if (!outputs_disjoint(outs, 3, ins, 5)) return JATTN_ERROR_INVALID_VALUE;
  const void* const qp[2] = {q, nullptr};
  const void* const kp[2] = {k, nullptr};
  const void* const vp[2] = {v, nullptr};
  void* const op[2] = {out, nullptr};
  return run_fwd(jattn::kVarlen, qp, kp, vp, gains, nullptr, cu_seqlens, total, B, max_seqlen, max_seqlen, H, D,
                 softmax_scale, eps, op, lse, workspace, stage_events, n_stage_events, stream);
}

jattn_status jattn_bwd_varlen(const void* q, const void* k, const void* v, const float* gains,
                              const int32_t* cu_seqlens, const void* out, const float* lse, const void* dout, int B,
                              int max_seqlen, int total, int H, int D, float softmax_scale, float eps, void* dq,
                              void* dk, void* dv, float* dgains, void* workspace, size_t workspace_bytes,
                              const void* fwd_workspace, const hipEvent_t* stage_events, int n_stage_events,
                              hipStream_t stream) {
  if (n_stage_events < 0 || n_stage_events > JATTN_BWD_STAGES || (n_stage_events > 0 && !stage_events))
    return JATTN_ERROR_INVALID_VALUE;
  if (!q || !k || !v || !gains || !cu_seqlens || !out || !lse || !dout || !dq || !dk || !dv || !dgains)
    return JATTN_ERROR_INVALID_VALUE;
  const jattn_status st = check_varlen_sizes(B, max_seqlen, total, H, D);
  if (st != JATTN_SUCCESS) return st;
  if (!std::isfinite(softmax_scale) || !std::isfinite(eps) || eps < 0.f) return JATTN_ERROR_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(gains, 4) || !aligned(lse, 4) ||
      !aligned(dgains, 4) || !aligned(cu_seqlens, 4))
    return JATTN_ERROR_INVALID_VALUE;
  const size_t wsb = jattn_varlen_bwd_workspace_bytes(B, max_seqlen, total, H, D);
  if (!workspace || workspace_bytes < wsb) return JATTN_ERROR_WORKSPACE;
  if (!aligned(workspace, 256) || !aligned(fwd_workspace, 256)) return JATTN_ERROR_INVALID_VALUE;
  const size_t tb = (size_t)total * H * D * 2, lb = (size_t)total * H * 4;
  const size_t fwb = fwd_workspace ? jattn_varlen_fwd_workspace_bytes(B, max_seqlen, total, H, D) : 0;
  const Range ins[] = {{q, tb},   {k, tb},    {v, tb},   {gains, (size_t)2 * D * 4}, {cu_seqlens, (size_t)(B + 1) * 4},
                       {out, tb}, {lse, lb}, {dout, tb}, {fwd_workspace, fwb}};
  const Range outs[] = {{dq, tb}, {dk, tb}, {dv, tb}, {dgains, (size_t)2 * D * 4}, {workspace, wsb}};
  if (!outputs_disjoint(outs, 5, ins, 9)) return JATTN_ERROR_INVALID_VALUE;
  const void* const qp[2] = {q, nullptr};
  const void* const kp[2] = {k, nullptr};
  const void* const vp[2] = {v, nullptr};
  const void* const op[2] = {out, nullptr};
  const void* const dop[2] = {dout, nullptr};
  void* const dqp[2] = {dq, nullptr};
  void* const dkp[2] = {dk, nullptr};
  void* const dvp[2] = {dv, nullptr};
  return run_bwd(jattn::kVarlen, qp, kp, vp, gains, nullptr, cu_seqlens, total, op, lse, dop, B, max_seqlen,
                 max_seqlen, H, D, softmax_scale, eps, dqp, dkp, dvp, dgains, workspace, fwd_workspace, stage_events,
                 n_stage_events, stream);
}

}  // extern "C"
