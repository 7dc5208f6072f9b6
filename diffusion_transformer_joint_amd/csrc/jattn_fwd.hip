// Forward pass of QK-RMSNorm joint attention on gfx950.
//
// Definition (re-diffusion README: architecture flowchart, DiT-layer box -- one multi-head attention
// over the concatenated image and text tokens; design-notes table, "QK norm" row -- RMSNorm on Q and
// K; profiling section -- the attention as an explicit fp32 softmax over the score matrix, which
// this kernel never materialises):
//   out_i = sum_j softmax_j(scale * <Qn_i, Kn_j>) v_j over valid keys j < n_b,  lse_i = log sum_j exp(.)
//
// One workgroup = 4 waves = 128 consecutive queries of one (batch, head) pair; each wave owns 32
// queries and streams all valid keys in tiles of 64 through LDS (double buffered, one barrier per
// tile). Per 32-key step a wave computes S^T = Kn Q'^T (4..8 MFMA over d, result: lane = query),
// turns it into P in registers, and accumulates O^T += V^T P^T with V^T read by ds_read_b64_tr_b16
// straight from the row-major V tile. Q' = bf16(q * r_q * g_q * scale * log2(e)) lives in registers
// for the whole loop, so scores come out in log2 units.
//
// Softmax shift. QK-RMSNorm bounds every score: ||Kn_j|| <= sqrt(D) * max|g_k| for any key, so
// |S'_ij| <= B_i = ||Q'_i|| * sqrt(D) * max|g_k| (plus a margin for bf16 rounding). When every row of
// the workgroup has B_i <= 48 (log2 units), the kernel uses the fixed shift B_i instead of a running
// maximum: the MFMA accumulator starts at -B_i, exp2 of the result lies in [2^-96, 1], and no row
// maximum, rescale or cross-lane exchange is needed inside the loop. Otherwise (large scale or gains)
// it runs the usual online softmax with a running maximum. Both give the same softmax up to rounding.
#include "jattn_device.h"
#include "jattn_launch.h"

namespace jattn {

constexpr float kBoundLimit = 48.f;
static_assert(kBlockRows == kRowsPerBlock, "host and device block sizes differ");

template <int D>
struct FwdSmem {
  static constexpr int STAGE = 2 * 2 * Dims<D>::TILE_ELEMS * 2;  // K and V, double buffered, bytes
  static constexpr int BYTES = STAGE + 16;
};

template <int D, bool BOUNDED>
__device__ __forceinline__ void fwd_loop(const FwdArgs& a, __bf16* sk, __bf16* sv,
                                         const uint16_t* __restrict__ kb, const uint16_t* __restrict__ vb,
                                         int rs, int n, const bf16x8 (&qf)[Dims<D>::KS], float shift,
                                         const float (&gk)[Dims<D>::CPT][8], f32x16 (&oacc)[Dims<D>::MT],
                                         float& lsum, float& mrow, int tid) {
  using Dm = Dims<D>;
  const int lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int ntiles = (n + kTile - 1) / kTile;
  TileRegs<D> tk, tv;
  if (ntiles > 0) {
    tile_load<D>(tk, kb, rs, 0, n, tid);
    tile_load<D>(tv, vb, rs, 0, n, tid);
  }
  f32x16 cinit;
#pragma unroll
  for (int i = 0; i < 16; ++i) cinit[i] = BOUNDED ? -shift : 0.f;

  for (int t = 0; t < ntiles; ++t) {
    __bf16* kt = sk + (t & 1) * Dm::TILE_ELEMS;
    __bf16* vt = sv + (t & 1) * Dm::TILE_ELEMS;
    tile_store_rmsnorm<D>(tk, kt, gk, a.eps, t * kTile, n, tid);
    tile_store_raw<D>(tv, vt, tid);
    __syncthreads();
    if (t + 1 < ntiles) {
      tile_load<D>(tk, kb, rs, (t + 1) * kTile, n, tid);
      tile_load<D>(tv, vb, rs, (t + 1) * kTile, n, tid);
    }
#pragma unroll
    for (int sb = 0; sb < kTile / 32; ++sb) {
      const int key0 = t * kTile + sb * 32;
      if (key0 >= n) break;
      // S'^T (keys x queries) = Kn Q'^T, accumulator seeded with the shift
      f32x16 s = cinit;
      const __bf16* kr = kt + (sb * 32 + l32) * Dm::PITCH + g * 8;
#pragma unroll
      for (int ks = 0; ks < Dm::KS; ++ks) s = mfma(lds_row_frag(kr + ks * 16), qf[ks], s);

      float p[16];
      const bool tail = key0 + 32 > n;
      if constexpr (BOUNDED) {
#pragma unroll
        for (int i = 0; i < 16; ++i) p[i] = fast_exp2(s[i]);
        if (tail) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (key0 + (i >> 2) * 8 + g * 4 + (i & 3) >= n) p[i] = 0.f;
        }
      } else {
        if (tail) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (key0 + (i >> 2) * 8 + g * 4 + (i & 3) >= n) s[i] = -INFINITY;
        }
        float mx = s[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(mrow, mx);
        const float mu = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = fast_exp2(mrow - mu);
#pragma unroll
        for (int i = 0; i < 16; ++i) p[i] = fast_exp2(s[i] - mu);
        lsum *= alpha;
#pragma unroll
        for (int mt = 0; mt < Dm::MT; ++mt) oacc[mt] *= alpha;
        mrow = mnew;
      }
      bf16x8 pf0, pf1;
      pack_probs(p, pf0, pf1, lsum);
      // O^T (d x queries) += V^T P^T
#pragma unroll
      for (int mt = 0; mt < Dm::MT; ++mt) {
        oacc[mt] = mfma(lds_tr_frag(vt, Dm::PITCH, sb * 32, mt * 32, lane), pf0, oacc[mt]);
        oacc[mt] = mfma(lds_tr_frag(vt, Dm::PITCH, sb * 32 + 16, mt * 32, lane), pf1, oacc[mt]);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_kernel(FwdArgs a) {
  using Dm = Dims<D>;
  __shared__ __attribute__((aligned(16))) char smem[FwdSmem<D>::BYTES];
  __bf16* sk = reinterpret_cast<__bf16*>(smem);
  __bf16* sv = sk + 2 * Dm::TILE_ELEMS;
  float* sbound = reinterpret_cast<float*>(smem + FwdSmem<D>::STAGE);

  int bh, blk, item;
  if (!map_item(a.items, a.nblk, bh, blk, item)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int L = a.L, H = a.H;
  const int b = bh / H;
  const int n = a.valid_len ? min(max(a.valid_len[b], 0), L) : L;
  const int rs = H * D;
  const size_t base = ((size_t)b * L * H + (bh - b * H)) * D;
  const uint16_t* qb = a.q + base;
  const uint16_t* kb = a.k + base;
  const uint16_t* vb = a.v + base;

  zero_pad_columns<D>(sk, 4, tid);

  float gk[Dm::CPT][8];
  stage_gains<D>(gk, a.gains + D, 1.f, tid);

  // This wave's 32 query rows, normalised and pre-scaled, as B-operand fragments.
  const int qrow = blk * kBlockRows + wave * kWaveRows + l32;
  const bool qvalid = qrow < L;
  bf16x8 qf[Dm::KS];
  float qq = 0.f;
  {
    float x[Dm::KS][8];
    load_row_chunks<D>(x, qb + (size_t)qrow * rs, qvalid, g);
    rmsnorm_row_frags<D>(qf, x, a.gains, a.c, a.eps, qvalid, g);
#pragma unroll
    for (int ks = 0; ks < Dm::KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = (float)qf[ks][e];
        qq += y * y;
      }
    qq += __shfl_xor(qq, 32);
  }
  // max |g_k| over d, then the per-row score bound in log2 units
  float gkmax = 0.f;
  for (int d = lane; d < D; d += 64) gkmax = fmaxf(gkmax, fabsf(a.gains[D + d]));
  gkmax = wave_max(gkmax);
  const float shift = sqrtf(qq) * sqrtf((float)D) * gkmax * (1.f + 1.f / 64.f);
  const float wmax = wave_max(shift);
  if (lane == 0) sbound[wave] = wmax;
  __syncthreads();
  const float bmax = fmaxf(fmaxf(sbound[0], sbound[1]), fmaxf(sbound[2], sbound[3]));

  f32x16 oacc[Dm::MT];
#pragma unroll
  for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[mt][i] = 0.f;
  float lsum = 0.f, mrow;
  if (bmax <= kBoundLimit) {  // uniform over the workgroup
    mrow = shift;
    fwd_loop<D, true>(a, sk, sv, kb, vb, rs, n, qf, shift, gk, oacc, lsum, mrow, tid);
  } else {
    mrow = -INFINITY;
    fwd_loop<D, false>(a, sk, sv, kb, vb, rs, n, qf, shift, gk, oacc, lsum, mrow, tid);
  }

  lsum += __shfl_xor(lsum, 32);
  if (!qvalid) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  if (g == 0) a.lse[(size_t)bh * L + qrow] = lsum > 0.f ? (mrow + __log2f(lsum)) * kLn2 : -INFINITY;
  uint16_t* orow = a.out + base + (size_t)qrow * rs;
#pragma unroll
  for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = mt * 32 + j4 * 8 + g * 4;
      if (d0 < D) {
        const u32x2 u = {pack2(oacc[mt][j4 * 4 + 0] * inv, oacc[mt][j4 * 4 + 1] * inv),
                         pack2(oacc[mt][j4 * 4 + 2] * inv, oacc[mt][j4 * 4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d0) = u;
      }
    }
}

template <int D>
static hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(fwd_kernel<D>, dim3(grid_for_items(a.items)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd(int D, const FwdArgs& a, hipStream_t stream) {
  switch (D) {
    case 32: return launch_fwd_d<32>(a, stream);
    case 64: return launch_fwd_d<64>(a, stream);
    case 72: return launch_fwd_d<72>(a, stream);
    case 128: return launch_fwd_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace jattn
