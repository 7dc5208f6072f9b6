// Backward pass of QK-RMSNorm joint attention on gfx950.
//
// Gradients of L = sum(out * dout) (the analytic backward of the attention defined in the
// re-diffusion README's flowchart and design-notes table; P is recomputed from the saved row
// log-sum-exp, the score matrix is never stored):
//   P = exp(S - lse),  dP = dO V^T,  Delta_i = sum_d dO_id O_id,  dS = P * (dP - Delta)
//   dV = P^T dO,  dQn = scale dS Kn,  dKn = scale dS^T Qn,
//   RMSNorm backward: dx = r (g * dxn) - x (r^3 / D) <g * dxn, x>,   dg = sum_rows dxn * x * r.
//
// Two kernels, no atomics:
//  * dq kernel  (query-parallel, like the forward): each wave owns 32 queries and streams Kn and V;
//    per 32-key step S^T, dP^T (both: lane = query), dS^T in registers, dQn^T += Kn^T dS^T with Kn^T
//    read by ds_read_b64_tr_b16. It also computes Delta for its rows (stored for the other kernel),
//    runs the Q-side RMSNorm backward in its epilogue and writes per-workgroup dg_q partials.
//  * dkdv kernel (key-parallel): each wave owns 32 keys (Kn and V rows in registers) and streams Q'
//    and dO; per 32-query step S, dP (lane = key), then dV^T += dO^T P and dKn^T += Q'^T dS with the
//    transposed operands read by ds_read_b64_tr_b16. Epilogue: K-side RMSNorm backward, dk, dv and
//    dg_k partials. Padded keys get exact zeros.
//  * a small kernel sums the gain partials in a fixed order (deterministic dgains).
// dQ is recomputed rather than accumulated across key blocks: fp32 atomics on this chip sustain a
// few hundred G/s, far below what a key-parallel dQ accumulation would need.
#include "jattn_device.h"
#include "jattn_launch.h"

namespace jattn {

template <int D>
struct BwdSmem {
  static constexpr int STAGE = 2 * 2 * Dims<D>::TILE_ELEMS * 2;  // two operands, double buffered
  static constexpr int STATS = 2 * 2 * kTile * 4;                 // -lse2 and -delta per staged row
  static constexpr int SCRATCH = (kBlockRows + 8) * Dims<D>::DM * 4;
  static constexpr int BYTES = (STAGE + STATS > SCRATCH ? STAGE + STATS : SCRATCH);
};

// RMSNorm backward for one wave row held in the C/D layout (lane = row; register i of tile mt
// holds d = 32*mt + 8*(i/4) + 4*g + i%4; the other half of the row is in lane l^32). If `exists`,
// writes the bf16 gradient row (zeros when not `valid`, i.e. a padded key). On return dxn holds the
// dg contributions dxn * x * r (zeros for rows that are not valid).
template <int D>
__device__ __forceinline__ void rmsnorm_backward_row(f32x16 (&dxn)[Dims<D>::MT], const uint16_t* __restrict__ xrow,
                                                     const float* __restrict__ gain, float r, bool valid,
                                                     bool exists, uint16_t* __restrict__ dxrow, int g) {
  using Dm = Dims<D>;
  float x[Dm::MT][16];
  float gv[Dm::MT][16];
  float t = 0.f;
#pragma unroll
  for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = mt * 32 + j4 * 8 + g * 4;
      float xv[4] = {0.f, 0.f, 0.f, 0.f};
      if (valid && d0 < D) unpack4(*reinterpret_cast<const u32x2*>(xrow + d0), xv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[mt][j4 * 4 + e] = xv[e];
        gv[mt][j4 * 4 + e] = d0 < D ? gain[d0 + e] : 0.f;
        t += gv[mt][j4 * 4 + e] * dxn[mt][j4 * 4 + e] * xv[e];
      }
    }
  t += __shfl_xor(t, 32);
  const float c3 = r * r * r * (1.0f / D) * t;
#pragma unroll
  for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = mt * 32 + j4 * 8 + g * 4;
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = j4 * 4 + e;
        y[e] = valid ? r * gv[mt][i] * dxn[mt][i] - x[mt][i] * c3 : 0.f;
      }
      if (exists && d0 < D)
        *reinterpret_cast<u32x2*>(dxrow + d0) = (u32x2){pack2(y[0], y[1]), pack2(y[2], y[3])};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = j4 * 4 + e;
        dxn[mt][i] = valid ? dxn[mt][i] * x[mt][i] * r : 0.f;  // reuse as the dg contribution
      }
    }
}

// ------------------------------------------------------------------------------------------------
// dq kernel: query-parallel
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(BwdArgs a) {
  using Dm = Dims<D>;
  __shared__ __attribute__((aligned(16))) char smem[BwdSmem<D>::BYTES];
  __bf16* sk = reinterpret_cast<__bf16*>(smem);
  __bf16* sv = sk + 2 * Dm::TILE_ELEMS;

  int bh, blk, item;
  if (!map_item(a.items, a.nblk, bh, blk, item)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int L = a.L, H = a.H;
  const int b = bh / H;
  const int n = a.valid_len ? min(max(a.valid_len[b], 0), L) : L;
  const int rs = H * D;
  const size_t base = ((size_t)b * L * H + (bh - b * H)) * D;

  zero_pad_columns<D>(sk, 4, tid);
  float gk[Dm::CPT][8];
  stage_gains<D>(gk, a.gains + D, 1.f, tid);

  const int qrow = blk * kBlockRows + wave * kWaveRows + l32;
  const bool qvalid = qrow < L;
  const size_t roff = base + (size_t)qrow * rs;
  bf16x8 qf[Dm::KS], dof[Dm::KS];
  float rq;
  {
    float x[Dm::KS][8];
    load_row_chunks<D>(x, a.q + roff, qvalid, g);
    rq = rmsnorm_row_frags<D>(qf, x, a.gains, a.c, a.eps, qvalid, g);
  }
  load_row_frags_raw<D>(dof, a.dout + roff, qvalid, g);
  float delta = 0.f;
  {
    float o[Dm::KS][8];
    load_row_chunks<D>(o, a.out + roff, qvalid, g);
#pragma unroll
    for (int ks = 0; ks < Dm::KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) delta += (float)dof[ks][e] * o[ks][e];
    delta += __shfl_xor(delta, 32);
  }
  const float lse2 = qvalid ? a.lse[(size_t)bh * L + qrow] * kLog2e : 0.f;
  if (qvalid && g == 0) a.delta[(size_t)bh * L + qrow] = delta;
  f32x16 cs, cp;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    cs[i] = -lse2;
    cp[i] = -delta;
  }
  f32x16 acc[Dm::MT];
#pragma unroll
  for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;

  const uint16_t* kb = a.k + base;
  const uint16_t* vb = a.v + base;
  const int ntiles = (n + kTile - 1) / kTile;
  TileRegs<D> tk, tv;
  if (ntiles > 0) {
    tile_load<D>(tk, kb, rs, 0, n, tid);
    tile_load<D>(tv, vb, rs, 0, n, tid);
  }
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
      f32x16 s = cs, dp = cp;
      const __bf16* kr = kt + (sb * 32 + l32) * Dm::PITCH + g * 8;
      const __bf16* vr = vt + (sb * 32 + l32) * Dm::PITCH + g * 8;
#pragma unroll
      for (int ks = 0; ks < Dm::KS; ++ks) s = mfma(lds_row_frag(kr + ks * 16), qf[ks], s);
#pragma unroll
      for (int ks = 0; ks < Dm::KS; ++ks) dp = mfma(lds_row_frag(vr + ks * 16), dof[ks], dp);
      float ds[16];
      const bool tail = key0 + 32 > n;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(s[i]);
        if (tail && key0 + (i >> 2) * 8 + g * 4 + (i & 3) >= n) p = 0.f;
        ds[i] = p * dp[i];
      }
      const bf16x8 f0 = to_bf16x8(ds), f1 = to_bf16x8(ds + 8);
#pragma unroll
      for (int mt = 0; mt < Dm::MT; ++mt) {
        acc[mt] = mfma(lds_tr_frag(kt, Dm::PITCH, sb * 32, mt * 32, lane), f0, acc[mt]);
        acc[mt] = mfma(lds_tr_frag(kt, Dm::PITCH, sb * 32 + 16, mt * 32, lane), f1, acc[mt]);
      }
    }
  }

#pragma unroll
  for (int mt = 0; mt < Dm::MT; ++mt) acc[mt] *= a.scale;  // dQn
  rmsnorm_backward_row<D>(acc, a.q + roff, a.gains, rq, qvalid, qvalid, a.dq + roff, g);
  __syncthreads();  // all waves are done with the staged tiles before the scratch reuse
  block_column_sums<D>(acc, reinterpret_cast<float*>(smem), a.part_q + (size_t)item * D, tid);
}

// ------------------------------------------------------------------------------------------------
// dkdv kernel: key-parallel
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_kernel(BwdArgs a) {
  using Dm = Dims<D>;
  __shared__ __attribute__((aligned(16))) char smem[BwdSmem<D>::BYTES];
  __bf16* sq = reinterpret_cast<__bf16*>(smem);
  __bf16* sdo = sq + 2 * Dm::TILE_ELEMS;
  float* slse = reinterpret_cast<float*>(smem + BwdSmem<D>::STAGE);  // [2][kTile]: -lse2
  float* sdel = slse + 2 * kTile;                                      // [2][kTile]: -delta

  int bh, blk, item;
  if (!map_item(a.items, a.nblk, bh, blk, item)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int L = a.L, H = a.H;
  const int b = bh / H;
  const int n = a.valid_len ? min(max(a.valid_len[b], 0), L) : L;
  const int rs = H * D;
  const size_t base = ((size_t)b * L * H + (bh - b * H)) * D;

  const int key = blk * kBlockRows + wave * kWaveRows + l32;
  const bool kin = key < L;      // row exists
  const bool kvalid = key < n;   // row is an unpadded key
  const size_t roff = base + (size_t)key * rs;

  if (blk * kBlockRows >= n) {
    // every key of this workgroup is padding: exact zeros, no dg contribution
    if (kin) {
#pragma unroll
      for (int c = g; c < Dm::NCH; c += 2) {
        *reinterpret_cast<u32x4*>(a.dk + roff + c * 8) = (u32x4){0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(a.dv + roff + c * 8) = (u32x4){0u, 0u, 0u, 0u};
      }
    }
    for (int d = tid; d < D; d += kThreads) a.part_k[(size_t)item * D + d] = 0.f;
    return;
  }

  zero_pad_columns<D>(sq, 4, tid);
  float gq[Dm::CPT][8];
  stage_gains<D>(gq, a.gains, a.c, tid);

  bf16x8 kf[Dm::KS], vf[Dm::KS];
  float rk;
  {
    float x[Dm::KS][8];
    load_row_chunks<D>(x, a.k + roff, kvalid, g);
    rk = rmsnorm_row_frags<D>(kf, x, a.gains + D, 1.f, a.eps, kvalid, g);
  }
  load_row_frags_raw<D>(vf, a.v + roff, kvalid, g);
  const bool wave_live = blk * kBlockRows + wave * kWaveRows < n;

  f32x16 dva[Dm::MT], dka[Dm::MT];
#pragma unroll
  for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dva[mt][i] = 0.f;
      dka[mt][i] = 0.f;
    }

  const uint16_t* qb = a.q + base;
  const uint16_t* ob = a.dout + base;
  const float* lse_bh = a.lse + (size_t)bh * L;
  const float* del_bh = a.delta + (size_t)bh * L;
  const int ntiles = (L + kTile - 1) / kTile;
  TileRegs<D> tq, to;
  float st_lse = 0.f, st_del = 0.f;
  auto load_stats = [&](int t) {
    if (tid < kTile) {
      const int qi = t * kTile + tid;
      st_lse = qi < L ? -lse_bh[qi] * kLog2e : -INFINITY;
      st_del = qi < L ? -del_bh[qi] : 0.f;
    }
  };
  tile_load<D>(tq, qb, rs, 0, L, tid);
  tile_load<D>(to, ob, rs, 0, L, tid);
  load_stats(0);
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    __bf16* qt = sq + buf * Dm::TILE_ELEMS;
    __bf16* ot = sdo + buf * Dm::TILE_ELEMS;
    tile_store_rmsnorm<D>(tq, qt, gq, a.eps, t * kTile, L, tid);
    tile_store_raw<D>(to, ot, tid);
    if (tid < kTile) {
      slse[buf * kTile + tid] = st_lse;
      sdel[buf * kTile + tid] = st_del;
    }
    __syncthreads();
    if (t + 1 < ntiles) {
      tile_load<D>(tq, qb, rs, (t + 1) * kTile, L, tid);
      tile_load<D>(to, ob, rs, (t + 1) * kTile, L, tid);
      load_stats(t + 1);
    }
    if (!wave_live) continue;
#pragma unroll
    for (int sb = 0; sb < kTile / 32; ++sb) {
      const int q0 = t * kTile + sb * 32;
      if (q0 >= L) break;
      f32x16 s, dp;
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(slse + buf * kTile + sb * 32 + j4 * 8 + g * 4);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(sdel + buf * kTile + sb * 32 + j4 * 8 + g * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[j4 * 4 + e] = l4[e];
          dp[j4 * 4 + e] = d4[e];
        }
      }
      const __bf16* qr = qt + (sb * 32 + l32) * Dm::PITCH + g * 8;
      const __bf16* orr = ot + (sb * 32 + l32) * Dm::PITCH + g * 8;
#pragma unroll
      for (int ks = 0; ks < Dm::KS; ++ks) s = mfma(lds_row_frag(qr + ks * 16), kf[ks], s);
#pragma unroll
      for (int ks = 0; ks < Dm::KS; ++ks) dp = mfma(lds_row_frag(orr + ks * 16), vf[ks], dp);
      float p[16], ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = kvalid ? fast_exp2(s[i]) : 0.f;
        ds[i] = p[i] * dp[i];
      }
      const bf16x8 pf0 = to_bf16x8(p), pf1 = to_bf16x8(p + 8);
      const bf16x8 df0 = to_bf16x8(ds), df1 = to_bf16x8(ds + 8);
#pragma unroll
      for (int mt = 0; mt < Dm::MT; ++mt) {
        dva[mt] = mfma(lds_tr_frag(ot, Dm::PITCH, sb * 32, mt * 32, lane), pf0, dva[mt]);
        dva[mt] = mfma(lds_tr_frag(ot, Dm::PITCH, sb * 32 + 16, mt * 32, lane), pf1, dva[mt]);
        dka[mt] = mfma(lds_tr_frag(qt, Dm::PITCH, sb * 32, mt * 32, lane), df0, dka[mt]);
        dka[mt] = mfma(lds_tr_frag(qt, Dm::PITCH, sb * 32 + 16, mt * 32, lane), df1, dka[mt]);
      }
    }
  }

  // dv (zeros at padded keys)
  if (kin) {
#pragma unroll
    for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int d0 = mt * 32 + j4 * 8 + g * 4;
        if (d0 < D) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = kvalid ? dva[mt][j4 * 4 + e] : 0.f;
          *reinterpret_cast<u32x2*>(a.dv + roff + d0) = (u32x2){pack2(y[0], y[1]), pack2(y[2], y[3])};
        }
      }
  }
  // dKn = scale * dS^T Qn = ln(2) * dS^T Q'   (Q' carries scale * log2(e))
#pragma unroll
  for (int mt = 0; mt < Dm::MT; ++mt) dka[mt] *= kLn2;
  if (kin) {
    rmsnorm_backward_row<D>(dka, a.k + roff, a.gains + D, rk, kvalid, true, a.dk + roff, g);
  } else {
#pragma unroll
    for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) dka[mt][i] = 0.f;
  }
  __syncthreads();
  block_column_sums<D>(dka, reinterpret_cast<float*>(smem), a.part_k + (size_t)item * D, tid);
}

// ------------------------------------------------------------------------------------------------
// dgains[side][d] = sum over workgroups of the partials, in a fixed order. Block (side, d); lane j
// sums items j, j + 64, ... with the loads issued in batches of 8, then a fixed butterfly.
__global__ __launch_bounds__(64) void dg_reduce_kernel(const float* __restrict__ part_q,
                                                       const float* __restrict__ part_k, int items,
                                                       int D, float* __restrict__ dgains) {
  const int side = blockIdx.x / D, d = blockIdx.x - side * D;
  const float* p = (side ? part_k : part_q) + d;
  float s = 0.f;
  int i = threadIdx.x;
  for (; i + 7 * 64 < items; i += 8 * 64) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(size_t)(i + u * 64) * D];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; i < items; i += 64) s += p[(size_t)i * D];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  if (threadIdx.x == 0) dgains[side * D + d] = s;
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a, const hipEvent_t* events, int n_events,
                               hipStream_t stream) {
  const dim3 grid(grid_for_items(a.items));
  hipLaunchKernelGGL(bwd_dq_kernel<D>, grid, dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && n_events > 0) e = hipEventRecord(events[0], stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkdv_kernel<D>, grid, dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e == hipSuccess && n_events > 1) e = hipEventRecord(events[1], stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dg_reduce_kernel, dim3(2 * D), dim3(64), 0, stream, a.part_q, a.part_k, a.items, D,
                     a.dgains);
  e = hipGetLastError();
  if (e == hipSuccess && n_events > 2) e = hipEventRecord(events[2], stream);
  return e;
}

hipError_t launch_bwd(int D, const BwdArgs& a, const hipEvent_t* events, int n_events, hipStream_t stream) {
  switch (D) {
    case 32: return launch_bwd_d<32>(a, events, n_events, stream);
    case 64: return launch_bwd_d<64>(a, events, n_events, stream);
    case 72: return launch_bwd_d<72>(a, events, n_events, stream);
    case 128: return launch_bwd_d<128>(a, events, n_events, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace jattn
