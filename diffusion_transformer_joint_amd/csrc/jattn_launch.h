// Internal interface between the C ABI (jattn_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace jattn {

struct PrenormArgs {
  const uint16_t* k;
  const int32_t* valid_len;  // [B] or nullptr
  uint16_t* kr;              // [B, H, L, D]: bf16(k * r_k), valid keys only
  int B, L, H;
  float eps;
};

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* kr;      // workspace [B, H, L, D]: bf16(k * r_k), written by the prenorm kernel
  const float* gains;      // [2, D]
  const int32_t* valid_len;  // [B] or nullptr
  uint16_t* out;
  float* lse;              // [B, H, L] natural log
  int B, L, H;
  float c;                 // softmax_scale * log2(e)
  float eps;
  int nblk;                // query blocks per (batch, head)
  int items;               // B * H * nblk
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* gains;
  const int32_t* valid_len;
  const uint16_t* out;
  const float* lse;
  const uint16_t* dout;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dgains;           // [2, D]
  uint16_t* kr;            // workspace [B, H, L, D]: bf16(k * r_k), valid keys only
  uint16_t* qs;            // workspace [B, H, L, D]: bf16(scale * log2(e) * q * r_q)
  float* nlse2;            // workspace [B, H, lp]: -lse * log2(e) (-inf past L)
  float* ndelta;           // workspace [B, H, lp]: -rowsum(dout * out) (0 past L)
  float* part;             // workspace [items, D]: per key block partial sums of T (see jattn_bwd.hip)
  int B, L, H;
  float scale;
  float c;                 // scale * log2(e)
  float eps;
  int nblk;                // row blocks (queries or keys) per (batch, head)
  int items;               // B * H * nblk
  int lp;                  // nblk * kBwdRowsPerBlock: statistics rows per (batch, head)
};

// Rows per workgroup, shared by the host-side grid and workspace sizing and the kernels.
// Forward: 4 waves of 64 queries (two independent 32-query tiles per wave) for D <= 64, where the
// register budget allows it; 4 waves of 32 queries otherwise.
constexpr int fwd_rows_per_block(int D) { return D <= 64 ? 256 : 128; }
// Backward: both kernels use workgroups of kBwdWaves waves of 32 rows.
constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBwdRowsPerBlock = 32 * kBwdWaves;

// Grid size of a persistent kernel (`threads` per workgroup, no dynamic LDS) over `items` work items:
// as many workgroups as the current device keeps resident at once, a multiple of 8 and no more than
// the items need (rounded up to 8).
hipError_t persistent_grid(const void* kernel, int items, int threads, int* grid);

hipError_t launch_prenorm(int D, const PrenormArgs& a, hipStream_t stream);
// Enqueues the key normalisation (into a.kr) and the forward kernel; if n_events > 0, records
// events[i] after stage i (i < n_events).
hipError_t launch_fwd(int D, const FwdArgs& a, const hipEvent_t* events, int n_events, hipStream_t stream);
// Enqueues the backward kernels (the key normalisation only if `prenorm`; a.kr then already holds
// it); if n_events > 0, records events[i] after stage i (i < n_events).
hipError_t launch_bwd(int D, const BwdArgs& a, bool prenorm, const hipEvent_t* events, int n_events,
                      hipStream_t stream);

}  // namespace jattn
