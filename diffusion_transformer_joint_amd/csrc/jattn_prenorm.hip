// RMS normalisation of the key rows, shared by the forward and the backward pass.
//
// The normalised keys Kr = k * r_k with r_k = (mean_d k^2 + eps)^(-1/2) (the RMSNorm of the QK-norm
// row in the re-diffusion README's design-notes table, without its gain) are written once per call
// as bf16 in a [B, H, L, D] layout. With one gain pair for all tokens both gains are folded into the
// query side by the attention kernels; with a gain pair per stream (the two-stream entry points) the
// K gain of each key's stream is applied here. The attention kernels then stream Kr tiles straight
// into LDS with no arithmetic on the way.
#include "jattn_device.h"
#include "jattn_launch.h"

namespace jattn {

// Kr[b, h, l, :] = bf16(k[b, l, h, :] * r_k) for the valid keys (l < valid length; later rows are
// never read). Thread t covers chunks t%TPR + j*TPR of row t/TPR of each pass; rows are taken in
// the joint (b, l, h) order. Two-stream variant (S): the key rows come from two blocks (rows
// l < n0 from a.k, the rest from a.k1) and each is also multiplied by its block's K gain, since the
// query side can no longer carry one K gain for every key. Varlen variant (V): blockIdx.y is the
// sequence and the rows are those of its (token, head) pairs, into the per-sequence workspace rows.
constexpr int kPrenormPasses = 4;

template <int D, bool S, bool V>
__global__ __launch_bounds__(kThreads) void prenorm_kernel(PrenormArgs a) {
  using Dm = Dims<D>;
  const int tid = threadIdx.x, rr = tid / Dm::TPR, cc = tid % Dm::TPR;
  const int H = a.H;
  const SeqGeom<V> seq(a.cu_seqlens, blockIdx.y, a.L, a.total, a.L);
  const int L = seq.L;
  // rows of this launch: all B * L * H rows (fixed length) or the L * H rows of sequence blockIdx.y
  const int total = V ? L * H : a.B * L * H;
  u32x4 x[kPrenormPasses][Dm::CPT];
  int row[kPrenormPasses];
#pragma unroll
  for (int p = 0; p < kPrenormPasses; ++p) {
    row[p] = (blockIdx.x * kPrenormPasses + p) * Dm::RPP + rr;  // (b * L + l) * H + h, or l * H + h (V)
    const uint16_t* src = a.k + ((size_t)seq.start * H + row[p]) * D;
    if constexpr (S) {
      const int R = row[p] < total ? row[p] : 0;
      const int bl = R / H, h = R - bl * H, b = bl / L, l = bl - b * L;
      src = RowMap<true>((size_t)b * a.n0, (size_t)b * (L - a.n0), h, H, D, a.n0).row(a.k, a.k1, l);
    }
#pragma unroll
    for (int j = 0; j < Dm::CPT; ++j) {
      const int c = cc + j * Dm::TPR;
      x[p][j] = row[p] < total && c < Dm::NCH ? *reinterpret_cast<const u32x4*>(src + c * 8)
                                              : (u32x4){0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int p = 0; p < kPrenormPasses; ++p) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < Dm::CPT; ++j) ss = sumsq8(x[p][j], ss);
    ss = group_sum<Dm::TPR>(ss);
    const float r = rsqrtf(ss * (1.0f / D) + a.eps);
    const int R = row[p];
    if (R >= total) continue;
    const int bl = R / H, h = R - bl * H, b = V ? (int)blockIdx.y : bl / L, l = V ? bl : bl - b * L;
    const int n = !V && a.valid_len ? min(max(a.valid_len[b], 0), L) : L;
    if (l >= n) continue;
    uint16_t* dst = a.kr + (V ? seq.row0(h, H) + l : ((size_t)b * H + h) * L + l) * D;
    const float* gk = a.gains + (l < a.n0 ? 0 : 2 * D) + D;  // (two-stream only)
#pragma unroll
    for (int j = 0; j < Dm::CPT; ++j) {
      const int c = cc + j * Dm::TPR;
      if (c < Dm::NCH) {
        float f[8];
        unpack8(x[p][j], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] *= S ? r * gk[c * 8 + e] : r;
        *reinterpret_cast<bf16x8*>(dst + c * 8) = to_bf16x8(f);
      }
    }
  }
}

hipError_t persistent_grid(const void* kernel, int items, int threads, int* grid) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
  if (e != hipSuccess) return e;
  const int resident = ((cus * (per_cu > 0 ? per_cu : 1)) >> 3) << 3;
  const int need = grid_for_items(items);
  *grid = resident >= 8 && resident < need ? resident : need;
  return hipSuccess;
}

template <int D, bool S, bool V>
static hipError_t launch_prenorm_d(const PrenormArgs& a, hipStream_t stream) {
  const int rows = Dims<D>::RPP * kPrenormPasses;
  // (varlen: one row of blocks per sequence, each sized for the longest sequence a.L)
  const int64_t per = V ? (int64_t)a.L * a.H : (int64_t)a.B * a.L * a.H;
  const int blocks = (int)((per + rows - 1) / rows);
  hipLaunchKernelGGL((prenorm_kernel<D, S, V>), dim3(blocks, V ? a.B : 1), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <bool S, bool V>
static hipError_t launch_prenorm_s(int D, const PrenormArgs& a, hipStream_t stream) {
  switch (D) {
#define JATTN_CASE(DD) \
  case DD: return launch_prenorm_d<DD, S, V>(a, stream);
    JATTN_FOR_EACH_HEAD_DIM(JATTN_CASE)
#undef JATTN_CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prenorm(int D, Variant var, const PrenormArgs& a, hipStream_t stream) {
  switch (var) {
    case kStreams: return launch_prenorm_s<true, false>(D, a, stream);
    case kVarlen: return launch_prenorm_s<false, true>(D, a, stream);
    default: return launch_prenorm_s<false, false>(D, a, stream);
  }
}

}  // namespace jattn
