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

}  // namespace jattn

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
