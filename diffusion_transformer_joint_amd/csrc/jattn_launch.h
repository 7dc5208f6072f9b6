// Internal interface between the C ABI (jattn_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace jattn {

// Token rows. Every per-token tensor is [B, L, H, D] bf16 with the rows of each sequence stored in
// two blocks: rows [0, n0) in the tensor's first pointer ([B, n0, H, D]) and rows [n0, L) in its
// second pointer (the `*1` fields, [B, L - n0, H, D]). The joint layout is the case n0 = L (second
// pointers unused). The two-stream entry points pass the image stream as block 0 (n0 = N_img) and
// the text stream as block 1; their kernels also select the QK-norm gains per row by block.
//
// Gains: joint entry points [2, D] (Q row, K row); two-stream entry points [2, 2, D]
// (gains[s][0] = Q gain and gains[s][1] = K gain of block s).
//
// Sequences. Fixed-length batches: B sequences of L rows, sequence b at token rows [b L, b L + L).
// Packed variable-length batches (the `varlen` kernels): `cu_seqlens` [B + 1] on the device gives the
// token row range of each sequence in [total, H, D] tensors (see SeqGeom), L is then the longest
// sequence (max_seqlen) and sizes the grids, and valid_len is not used.
//
// Local window (the `window` kernels): query i sees only keys i - wl <= j <= i + wr, besides j < n.
// The host passes wl, wr in [0, L] (L for an unbounded side).

struct PrenormArgs {
  const uint16_t* k;
  const uint16_t* k1;
  const float* gains;        // two-stream only: K rows are multiplied by their block's K gain
  const int32_t* valid_len;  // [B] or nullptr
  const int32_t* cu_seqlens; // varlen only
  uint16_t* kr;              // [B, H, L, D]: bf16(k * r_k) (times the K gain, two-stream), valid keys only
  int B, L, H, n0, total;
  float eps;
};

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* q1;
  const uint16_t* k1;
  const uint16_t* v1;
  const uint16_t* kr;      // workspace [B, H, L, D]: normalised keys, written by the prenorm kernel
  const float* gains;
  const int32_t* valid_len;  // [B] or nullptr
  const int32_t* cu_seqlens; // varlen only
  uint16_t* out;
  uint16_t* out1;
  float* lse;              // [B, H, L] natural log (varlen: per sequence [H, L_b], see SeqGeom)
  int B, L, H, n0, total;
  int wl, wr;              // window bounds (window kernels only)
  float c;                 // softmax_scale * log2(e)
  float eps;
  int nblk;                // query blocks per (batch, head)
  int items;               // B * H * nblk
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* q1;
  const uint16_t* k1;
  const uint16_t* v1;
  const float* gains;
  const int32_t* valid_len;
  const int32_t* cu_seqlens;  // varlen only
  const uint16_t* out;
  const uint16_t* out1;
  const float* lse;
  const uint16_t* dout;
  const uint16_t* dout1;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  uint16_t* dq1;
  uint16_t* dk1;
  uint16_t* dv1;
  float* dgains;           // [2, D] (joint) or [2, 2, D] (two-stream)
  uint16_t* kr;            // workspace [B, H, L, D]: normalised keys, valid keys only
  uint16_t* qs;            // workspace [B, H, L, D]: bf16(scale * log2(e) * q * r_q) (times the Q gain, two-stream)
  float* nlse2;            // workspace [B, H, lp]: -lse * log2(e) (-inf past L)
  float* ndelta;           // workspace [B, H, lp]: -rowsum(dout * out) (0 past L)
  float* part;             // workspace [kPartSets, D, items]: per row block partial sums of the gain gradients
  int B, L, H, n0, total;
  int wl, wr;              // window bounds (window kernels only)
  float scale;
  float c;                 // scale * log2(e)
  float eps;
  int nblk;                // row blocks (queries or keys) per (batch, head)
  int items;               // B * H * nblk
  int lp;                  // nblk * kBwdRowsPerBlock: statistics rows per (batch, head)
};

// Rows per workgroup, shared by the host-side grid and workspace sizing and the kernels.
// Forward: 4 waves of 32 queries. (Two 32-query tiles per wave, 256 rows per workgroup at two waves
// per SIMD, measured 3 % slower at D = 64 than one tile per wave at three: the smaller blocks also
// split the 1101-row sequences more evenly and shorten the reach of a local window.)
// The compiled head dims: every multiple of 8 from 32 to 128. X(D) is expanded once per head dim
// (used for the switch statements that pick a kernel instantiation).
#define JATTN_FOR_EACH_HEAD_DIM(X) JATTN_FOR_EACH_NARROW_HEAD_DIM(X) JATTN_FOR_EACH_WIDE_HEAD_DIM(X)
// The backward splits them at kNarrowMaxD: two waves per SIMD up to it (jattn_bwd.hip), one above
// (jattn_bwd_wide.hip, compiled with MFMA accumulators in AGPRs).
#define JATTN_FOR_EACH_NARROW_HEAD_DIM(X) X(32) X(40) X(48) X(56) X(64) X(72)
#define JATTN_FOR_EACH_WIDE_HEAD_DIM(X) X(80) X(88) X(96) X(104) X(112) X(120) X(128)
constexpr int kNarrowMaxD = 72;

constexpr int fwd_rows_per_block(int D) { return 128; }
// Waves per SIMD the forward kernel's register allocation targets: three for D = 32 and 64, whose
// key/value ring of three buffers leaves room for three workgroups per CU, else two. The windowed
// (W) instantiations keep two: their mask and tile-range state spills to scratch at three (D = 64).
constexpr int fwd_waves_per_eu(int D, bool W = false) { return (D == 32 || D == 64) && !W ? 3 : 2; }
// Backward: both kernels use workgroups of kBwdWaves waves of 32 rows.
constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBwdRowsPerBlock = 32 * kBwdWaves;
// Partial-sum sets of the gain gradients in the backward workspace: the joint pass uses set 0 (the
// shared factor T); the two-stream pass uses set 2 s (Q gain of block s, from the dq kernel) and
// set 2 s + 1 (K gain of block s, from the dk/dv kernel).
constexpr int kPartSets = 4;

// Grid size of a persistent kernel (`threads` per workgroup, no dynamic LDS) over `items` work items:
// as many workgroups as the current device keeps resident at once, a multiple of 8 and no more than
// the items need (rounded up to 8).
hipError_t persistent_grid(const void* kernel, int items, int threads, int* grid);

// Kernel variants: the joint kernels, the two-stream kernels (two row blocks, gains per block) and
// the packed variable-length kernels.
enum Variant { kJoint = 0, kStreams = 1, kVarlen = 2, kWindow = 3 };
hipError_t launch_prenorm(int D, Variant var, const PrenormArgs& a, hipStream_t stream);
// Enqueues the key normalisation (into a.kr) and the forward kernel; if n_events > 0, records
// events[i] after stage i (i < n_events; a NULL entry records nothing).
hipError_t launch_fwd(int D, Variant var, const FwdArgs& a, const hipEvent_t* events, int n_events,
                      hipStream_t stream);
// Enqueues the backward kernels (the key normalisation only if `prenorm`; a.kr then already holds
// it); if n_events > 0, records events[i] after stage i (i < n_events; a NULL entry records nothing).
hipError_t launch_bwd(int D, Variant var, const BwdArgs& a, bool prenorm, const hipEvent_t* events,
                      int n_events, hipStream_t stream);
// launch_bwd for D > kNarrowMaxD (defined in jattn_bwd_wide.hip).
hipError_t launch_bwd_wide(int D, Variant var, const BwdArgs& a, bool prenorm, const hipEvent_t* events,
                           int n_events, hipStream_t stream);

}  // namespace jattn
