// Host-side helpers shared by the C ABIs of the adaLN projection and of the MLP block: argument
// checks, buffer-overlap tests, stage events, GEMM problem set-up and the token splits of the
// weight-gradient GEMMs. Internal to the library.
#pragma once

#include <cstddef>
#include <cstdint>

#include "adaln_launch.h"
#include "jattn.h"

namespace jattn_api {

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline bool ptr_ok(const void* p) { return p != nullptr && aligned(p, 16); }

struct Range {
  const void* p;
  size_t bytes;
};

inline bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Each output disjoint from every input and from every other output.
inline bool disjoint(const Range* outs, int nout, const Range* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j])) return false;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return false;
  }
  return true;
}

inline jattn_status check_events(const hipEvent_t* ev, int n, int max) {
  if (n < 0 || n > max || (n > 0 && ev == nullptr)) return JATTN_ERROR_INVALID_VALUE;
  return JATTN_SUCCESS;
}

// After a launch that is not the last of its stage: was it enqueued? (Checked per launch, so that a
// failed launch cannot be hidden by a later one.)
inline bool launched() { return hipGetLastError() == hipSuccess; }

// After enqueueing stage i: check the launch and record its event.
inline bool stage_done(int i, const hipEvent_t* ev, int n, hipStream_t stream) {
  if (hipGetLastError() != hipSuccess) return false;
  if (i < n && ev[i] && hipEventRecord(ev[i], stream) != hipSuccess) return false;
  return true;
}

inline jattn::MatRef mat(const void* p0, const void* p1, const void* p2, int seg, int rs, int64_t rows, int width) {
  jattn::MatRef m;
  m.p[0] = static_cast<const uint16_t*>(p0);
  m.p[1] = static_cast<const uint16_t*>(p1 ? p1 : p0);
  m.p[2] = static_cast<const uint16_t*>(p2 ? p2 : p0);
  m.seg = seg;
  m.rs = rs;
  m.rows = (int)rows;
  m.width = width;
  return m;
}

// A problem with no epilogue extras: callers set what their kernel uses.
inline jattn::GemmProblem problem(const jattn::MatRef& a, const jattn::MatRef& b, int M, int N, int K) {
  jattn::GemmProblem p;
  p.a = a;
  p.b = b;
  p.M = M;
  p.N = N;
  p.K = K;
  p.splits = 1;
  p.kchunk = K;
  p.out[0] = p.out[1] = p.out[2] = nullptr;
  p.out_seg = 0;
  p.bias = nullptr;
  p.colsum = nullptr;
  p.aux = nullptr;
  p.pair_off = 0;
  return p;
}

// Tile counts of both problems for output tiles of ma x mb.
inline void finish(jattn::GemmArgs& g, int ma, int mb) {
  for (int s = 0; s < 2; ++s) {
    jattn::GemmProblem& p = g.pr[s];
    if (p.N <= 0 || p.M <= 0) {
      p.tiles_m = p.tiles_n = p.splits = 1;
      p.ntiles = 0;
      continue;
    }
    p.tiles_m = (p.M + ma - 1) / ma;
    p.tiles_n = (p.N + mb - 1) / mb;
    p.ntiles = p.tiles_m * p.tiles_n * p.splits;
  }
  g.ntiles = g.pr[0].ntiles + g.pr[1].ntiles;
}

// Splits of a weight-gradient GEMM (output M x N for both streams, contraction over each stream's T
// tokens). Its output has few tiles when the widths are small, so the tokens are split: each stream
// gets floor(steps_s / target) splits (at least one), where target is the contraction steps per
// workgroup that spread the whole launch over 256 workgroups. With one split the GEMM writes the
// gradients directly; with more, fp32 partials that a reduction sums in order.
inline void dw_splits(const int64_t T[2], int M, int N, int splits[2], int kchunk[2]) {
  const int64_t tiles = (int64_t)((M + jattn::kDwMA - 1) / jattn::kDwMA) * ((N + jattn::kDwMB - 1) / jattn::kDwMB);
  int64_t steps[2], total = 0;
  for (int s = 0; s < 2; ++s) {
    steps[s] = (T[s] + jattn::kGemmK - 1) / jattn::kGemmK;
    total += steps[s] * tiles;
  }
  const int64_t target = total > 0 ? (total + 255) / 256 : 1;
  for (int s = 0; s < 2; ++s) {
    int64_t sp = steps[s] / target;
    sp = sp < 1 ? 1 : sp > 64 ? 64 : sp;
    const int64_t per = steps[s] > 0 ? (steps[s] + sp - 1) / sp : 1;  // steps per split
    kchunk[s] = (int)(per * jattn::kGemmK);
    splits[s] = steps[s] > 0 ? (int)((steps[s] + per - 1) / per) : 1;
  }
}

}  // namespace jattn_api
