// Saturating probe kernels for reading the full-scale values of the SQ busy counters (measurement
// support; see jattn_diag.h). Register data only; each thread writes one float.
#include "jattn_diag.h"
#include "jattn_device.h"

namespace jattn {

constexpr int kProbeThreads = 256;

// Four independent 32x32x16 bf16 MFMA chains per wave, 64 MFMAs per iteration: the matrix pipe of
// the SIMD stays busy (a dependent MFMA waits for its predecessor, four chains cover that latency).
__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(int iters, float seed, float* __restrict__ out) {
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(threadIdx.x + i));
    b[i] = (__bf16)(seed * (float)i);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = mfma(a, b, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

// Sixteen independent fp32 FMA chains per lane, 128 FMAs per iteration.
__global__ __launch_bounds__(kProbeThreads) void probe_fma_kernel(int iters, float seed, float* __restrict__ out) {
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = seed * (float)(threadIdx.x + i) * 1e-6f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = x[i] * 0.999f - 0.5f;
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += x[i];
  out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

// dQ accumulation patterns (see jattn_diag.h). Workgroup w handles pair w / nkb, key block w % nkb;
// element e of a 64-row tile is (row e / D, column e % D), so each wave instruction covers whole rows.
__global__ __launch_bounds__(kProbeThreads) void probe_dq_tiles_kernel(int mode, int L, int D, int nkb, int pairs,
                                                                       float* __restrict__ acc) {
  const int pair = blockIdx.x / nkb, kb = blockIdx.x - pair * nkb;
  const int ntiles = (L + 63) / 64, per_tile = 64 * D;
  float* base = mode == 0 ? acc + (size_t)pair * L * D : acc + ((size_t)kb * pairs + pair) * L * D;
  for (int tt = 0; tt < ntiles; ++tt) {
    const int t = (tt + 2 * kb) % ntiles;  // the key blocks of a pair start at different query tiles
    for (int e = threadIdx.x; e < per_tile; e += kProbeThreads) {
      const int r = t * 64 + e / D;
      if (r < L) {
        float* p = base + (size_t)r * D + e % D;
        if (mode == 0) unsafeAtomicAdd(p, 1.0f);
        else *p = 1.0f;
      }
    }
  }
}

__global__ __launch_bounds__(kProbeThreads) void probe_dq_reduce_kernel(size_t n, int nkb, float* __restrict__ acc) {
  for (size_t i = ((size_t)blockIdx.x * kProbeThreads + threadIdx.x) * 4; i < n; i += (size_t)gridDim.x * kProbeThreads * 4) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < nkb; ++kb) s += *reinterpret_cast<const f32x4*>(acc + (size_t)kb * n + i);
    *reinterpret_cast<f32x4*>(acc + (size_t)nkb * n + i) = s;
  }
}

}  // namespace jattn

extern "C" jattn_status jattn_probe_dq_accumulation(int mode, int pairs, int L, int D, int nkb, float* acc,
                                                    size_t acc_bytes, hipStream_t stream) {
  if (mode < JATTN_PROBE_DQ_ATOMIC || mode > JATTN_PROBE_DQ_REDUCE || pairs < 1 || L < 1 || D < 4 || D > 128 ||
      D % 4 != 0 || nkb < 1 || nkb > 64 || acc == nullptr || (reinterpret_cast<uintptr_t>(acc) & 15u) != 0)
    return JATTN_ERROR_INVALID_VALUE;
  const int64_t n = (int64_t)pairs * L * D;
  if (n * (nkb + 1) >= ((int64_t)1 << 31) || (int64_t)pairs * nkb >= ((int64_t)1 << 31))
    return JATTN_ERROR_INVALID_VALUE;
  const int64_t need = (mode == JATTN_PROBE_DQ_ATOMIC ? n : mode == JATTN_PROBE_DQ_PARTIAL ? nkb * n : (nkb + 1) * n) * 4;
  if ((int64_t)acc_bytes < need) return JATTN_ERROR_INVALID_VALUE;
  if (mode == JATTN_PROBE_DQ_REDUCE)
    hipLaunchKernelGGL(jattn::probe_dq_reduce_kernel, dim3(2048), dim3(jattn::kProbeThreads), 0, stream, (size_t)n, nkb,
                       acc);
  else
    hipLaunchKernelGGL(jattn::probe_dq_tiles_kernel, dim3(pairs * nkb), dim3(jattn::kProbeThreads), 0, stream, mode, L,
                       D, nkb, pairs, acc);
  return hipGetLastError() == hipSuccess ? JATTN_SUCCESS : JATTN_ERROR_HIP;
}

extern "C" jattn_status jattn_probe_saturate(int which, int blocks, int iters, float seed, float* out,
                                             hipStream_t stream) {
  if ((which != JATTN_PROBE_MFMA && which != JATTN_PROBE_FMA) || blocks < 1 || iters < 1 ||
      (int64_t)blocks * jattn::kProbeThreads >= ((int64_t)1 << 31) || out == nullptr ||
      (reinterpret_cast<uintptr_t>(out) & 3u) != 0)
    return JATTN_ERROR_INVALID_VALUE;
  if (which == JATTN_PROBE_MFMA)
    hipLaunchKernelGGL(jattn::probe_mfma_kernel, dim3(blocks), dim3(jattn::kProbeThreads), 0, stream, iters, seed,
                       out);
  else
    hipLaunchKernelGGL(jattn::probe_fma_kernel, dim3(blocks), dim3(jattn::kProbeThreads), 0, stream, iters, seed,
                       out);
  return hipGetLastError() == hipSuccess ? JATTN_SUCCESS : JATTN_ERROR_HIP;
}
