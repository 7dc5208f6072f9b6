// Measurement support (see jattn_diag.h): saturating probe kernels for reading the full-scale values
// of the SQ busy counters, the dQ-accumulation traffic probe, and probes of the dk/dv tile's
// dependency structure, of LDS read rates and of the MFMA / VALU issue rates.
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


// ------------------------------------------------------------------------------------------------
// The dk/dv tile's dependency structure at D = 64, without global loads: per 32-query half 8 score
// MFMAs (S and dP, 4 k-steps each, seeded with the row statistics), then 16 exp2, 16 multiplies and
// 16 bf16 conversions, then 8 gradient MFMAs fed by transposed fragments; one 64-query tile per
// iteration. Each operand comes from registers or from an LDS tile laid out like the kernel's (128-byte
// rows, 16-byte chunks XOR-swizzled by row), as the mode selects. The tiles hold small values, so the
// arithmetic stays finite; its results only feed the per-thread output.
constexpr int kTileBytes = 64 * 64 * 2;  // one 64 x 64 bf16 tile
constexpr int kTileStage = 2 * kTileBytes + 512;  // Qs and dO tiles, then -lse2 and -Delta of 64 rows

template <int MODE>
__global__ __launch_bounds__(kProbeThreads) void probe_tile_kernel(int iters, float seed, float* __restrict__ out,
                                                                   uint64_t* __restrict__ cycles) {
  constexpr bool ROWS = MODE == JATTN_PROBE_TILE_LDS || MODE == JATTN_PROBE_TILE_LDS_BARRIER ||
                        MODE == JATTN_PROBE_TILE_ROWS_STATS || MODE == JATTN_PROBE_TILE_ROWS ||
                        MODE == JATTN_PROBE_TILE_PIPELINED;
  constexpr bool STATS = MODE == JATTN_PROBE_TILE_LDS || MODE == JATTN_PROBE_TILE_LDS_BARRIER ||
                         MODE == JATTN_PROBE_TILE_ROWS_STATS || MODE == JATTN_PROBE_TILE_STATS ||
                         MODE == JATTN_PROBE_TILE_PIPELINED;
  constexpr bool TRANS = MODE == JATTN_PROBE_TILE_LDS || MODE == JATTN_PROBE_TILE_LDS_BARRIER ||
                         MODE == JATTN_PROBE_TILE_TRANSPOSED || MODE == JATTN_PROBE_TILE_PIPELINED;
  __shared__ __attribute__((aligned(16))) char smem[2 * kTileStage];
  const int tid = (int)threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  // (the tiles as small bf16 values, the statistics as small fp32 values: the fragments are read as bf16,
  // so fp32 patterns there would put arbitrary bit patterns, NaN among them, into the arithmetic)
  for (int i = tid; i < kTileStage; i += kProbeThreads) {  // 16-bit elements of both stages
    if ((i * 2) % kTileStage < 2 * kTileBytes) reinterpret_cast<__bf16*>(smem)[i] = (__bf16)(seed * (float)(i & 127));
  }
  for (int i = tid; i < 2 * 128; i += kProbeThreads)
    reinterpret_cast<float*>(smem + (i >> 7) * kTileStage + 2 * kTileBytes)[i & 127] = -seed * (float)(i & 63);
  __syncthreads();
  bf16x8 kf[4], vf[4], treg[2][2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kf[j][e] = (__bf16)(seed * (float)(lane + e + j));
      vf[j][e] = (__bf16)(seed * (float)(e - j));
    }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      treg[m][0][e] = (__bf16)(seed * (float)(e + m));
      treg[m][1][e] = (__bf16)(seed * (float)(e - m));
    }
  f32x16 sreg, dreg, acc[4];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    sreg[i] = -seed * (float)i;
    dreg[i] = 0.5f * seed * (float)i;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
  auto stage = [&](int u) { return smem + ((u >> 1) & 1) * kTileStage; };  // unit u = half u % 2 of tile u / 2
  auto row_off = [&](int h, int ks) {  // byte offset of this lane's row fragment (row h*32 + l32, k-step ks)
    const int row = h * 32 + l32;
    return row * 128 + (((ks * 2 + g) ^ (row & 7)) << 4);
  };
  auto tr_frag = [&](const char* tile, int row0, int mt) {  // transposed fragment: rows row0 .. row0 + 15
    const int r = row0 + 4 * (lane >> 5) + ((lane & 15) >> 2);
    const int c = mt * 32 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
    const int o0 = r * 128 + ((((c >> 3) ^ (r & 7)) << 4) | ((c & 7) * 2));
    const int o1 = (r + 8) * 128 + ((((c >> 3) ^ ((r + 8) & 7)) << 4) | ((c & 7) * 2));
    const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((JATTN_LDS i16x4*)(tile + o0));
    const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((JATTN_LDS i16x4*)(tile + o1));
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4, x), __builtin_bit_cast(bf16x4, y), 0, 1, 2, 3, 4, 5, 6, 7);
  };
  f32x16 s[2], dp[2];
  bf16x8 qr[2][4], orr[2][4];
  // statistics (seeds) and row fragments of unit u into set b
  auto read_unit = [&](int u, int b) {
    const char* base = stage(u);
    const int h = u & 1;
    if constexpr (STATS) {
      const float* st = reinterpret_cast<const float*>(base + 2 * kTileBytes);
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(st + h * 32 + j4 * 8 + g * 4);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(st + 64 + h * 32 + j4 * 8 + g * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[b][j4 * 4 + e] = l4[e];
          dp[b][j4 * 4 + e] = d4[e];
        }
      }
    } else {
      asm volatile("" : "+v"(sreg));  // (a fresh seed each unit, as the kernel's statistics are)
      s[b] = sreg;
      dp[b] = dreg;
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if constexpr (ROWS) {
        qr[b][ks] = *reinterpret_cast<const bf16x8*>(base + row_off(h, ks));
        orr[b][ks] = *reinterpret_cast<const bf16x8*>(base + kTileBytes + row_off(h, ks));
      } else {
        qr[b][ks] = kf[(ks + h + 1) & 3];
        orr[b][ks] = vf[(ks + h + 2) & 3];
      }
    }
  };
  auto unit = [&](int u, int b) {  // the products and softmax of unit u from set b
    const char* base = stage(u);
    const int h = u & 1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      s[b] = mfma(qr[b][ks], kf[ks], s[b]);
      dp[b] = mfma(orr[b][ks], vf[ks], dp[b]);
    }
    bf16x8 tq[2][2], to[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if constexpr (TRANS) {
          to[mt][r] = tr_frag(base + kTileBytes, h * 32 + r * 16, mt);
          tq[mt][r] = tr_frag(base, h * 32 + r * 16, mt);
        } else {
          to[mt][r] = treg[mt][r];
          tq[mt][r] = treg[mt][r ^ 1];
        }
      }
    if constexpr (MODE == JATTN_PROBE_TILE_PIPELINED) {
      read_unit(u + 1, b ^ 1);  // the next unit's reads go out under this unit's softmax and products
      __builtin_amdgcn_sched_barrier(0);
    }
    float p[16], ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = fast_exp2(s[b][i]);
      ds[i] = p[i] * dp[b][i];
    }
    const bf16x8 pf[2] = {to_bf16x8(p), to_bf16x8(p + 8)}, df[2] = {to_bf16x8(ds), to_bf16x8(ds + 8)};
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      acc[mt] = mfma(to[mt][0], pf[0], acc[mt]);
      acc[mt] = mfma(to[mt][1], pf[1], acc[mt]);
      acc[2 + mt] = mfma(tq[mt][0], df[0], acc[2 + mt]);
      acc[2 + mt] = mfma(tq[mt][1], df[1], acc[2 + mt]);
    }
  };
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  if constexpr (MODE == JATTN_PROBE_TILE_PIPELINED) {
    read_unit(0, 0);
    for (int it = 0; it < iters; ++it) {
      unit(2 * it, 0);
      __builtin_amdgcn_sched_barrier(0);
      unit(2 * it + 1, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        read_unit(2 * it + h, 0);
        unit(2 * it + h, 0);
      }
      if constexpr (MODE == JATTN_PROBE_TILE_LDS_BARRIER) __syncthreads();
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += acc[j][i];
  out[(size_t)blockIdx.x * kProbeThreads + tid] = sum;
  if (lane == 0) cycles[(size_t)blockIdx.x * (kProbeThreads / 64) + (tid >> 6)] = t1 - t0;
}

// LDS read rate: every wave issues 8 independent reads per iteration and consumes them together.
template <int MODE>
__global__ __launch_bounds__(kProbeThreads) void probe_lds_read_kernel(int iters, uint64_t* __restrict__ cycles) {
  __shared__ __attribute__((aligned(16))) float smem[16384];  // 64 KiB
  const int tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < 16384; i += kProbeThreads) smem[i] = (float)(i & 255);
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    const int base = ((it * 7 + w) & 7) * 2048;  // an 8 KiB window (floats)
    if constexpr (MODE == JATTN_PROBE_LDS_B128 || MODE == JATTN_PROBE_LDS_B128_BROADCAST) {
      f32x4 v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r)
        v[r] = MODE == JATTN_PROBE_LDS_B128 ? *reinterpret_cast<const f32x4*>(smem + base + r * 256 + lane * 4)
                                            : *reinterpret_cast<const f32x4*>(smem + base + r * 8 + (lane >> 5) * 4);
      asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
    } else {
      i16x4 v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r)
        v[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (JATTN_LDS i16x4*)(reinterpret_cast<char*>(smem) + (base + r * 128) * 4 + lane * 8));
      asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (lane == 0) cycles[(size_t)blockIdx.x * (kProbeThreads / 64) + w] = t1 - t0;
}


// Issue rates of the matrix pipe, fp32 FMAs and exp2 (v_exp_f32), alone and together: workgroups of
// 8 waves, two per SIMD (waves w and w + 4 share SIMD w % 4), each looping `iters` times over 8 steps.
// A step is one MFMA (four independent accumulators in turn), 16 FMAs (eight independent chains) or
// 8 exp2 (eight independent chains), or one MFMA plus the FMAs or exps in the same wave (MIXED), or
// the MFMA in waves 0-3 and the FMAs or exps in waves 4-7 (SPLIT).
constexpr int kIssueThreads = 512;

template <int MODE>
__global__ __launch_bounds__(kIssueThreads) void probe_issue_kernel(int iters, float seed, float* __restrict__ out,
                                                                    uint64_t* __restrict__ cycles) {
  const int tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool first = w < 4;  // (wave-uniform)
  constexpr bool ANY_MFMA = MODE != JATTN_PROBE_ISSUE_FMA && MODE != JATTN_PROBE_ISSUE_EXP;
  constexpr bool ANY_FMA = MODE == JATTN_PROBE_ISSUE_FMA || MODE == JATTN_PROBE_ISSUE_MIXED_FMA ||
                           MODE == JATTN_PROBE_ISSUE_SPLIT_FMA;
  constexpr bool ANY_EXP = MODE == JATTN_PROBE_ISSUE_EXP || MODE == JATTN_PROBE_ISSUE_MIXED_EXP ||
                           MODE == JATTN_PROBE_ISSUE_SPLIT_EXP;
  constexpr bool SPLIT = MODE == JATTN_PROBE_ISSUE_SPLIT_FMA || MODE == JATTN_PROBE_ISSUE_SPLIT_EXP;
  const bool do_mfma = ANY_MFMA && (!SPLIT || first);
  const bool do_valu = (ANY_FMA || ANY_EXP) && (!SPLIT || !first);
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
  bf16x8 a, b;
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(tid + i));
    b[i] = (__bf16)(seed * (float)i);
    x[i] = seed * (float)(tid + i) * 1e-3f;
  }
  auto valu = [&]() {
    if constexpr (ANY_FMA) {
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = x[i] * 0.999f + 1e-3f;
    } else if constexpr (ANY_EXP) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = fast_exp2(-x[i]);  // stays in [0.5, 1]
    }
  };
  // (one straight-line loop per wave kind: no branch inside the steps)
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  if (do_mfma && do_valu) {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        acc[r & 3] = mfma(a, b, acc[r & 3]);
        valu();
      }
  } else if (do_mfma) {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[r & 3] = mfma(a, b, acc[r & 3]);
  } else {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int r = 0; r < 8; ++r) valu();
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) sum += x[i];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += acc[j][i];
  out[(size_t)blockIdx.x * kIssueThreads + tid] = sum;
  if (lane == 0) cycles[(size_t)blockIdx.x * (kIssueThreads / 64) + w] = t1 - t0;
}


// The forward tile's structure at D = 64 without global loads: per wave and step two 32-query tiles,
// each with 4 score MFMAs (seeded accumulator), 16 exp2, 8 bf16 packs and 8 dot2 row-sum steps, and
// 4 PV MFMAs on the packed probabilities. Workgroups of 8 waves (two per SIMD). K fragments
// (ds_read_b128) and V fragments (ds_read_b64_tr_b16) come from a 64 x 64 LDS tile pair or registers.
template <int MODE, bool LDS>
__global__ __launch_bounds__(kIssueThreads) void probe_pingpong_kernel(int iters, float seed, float* __restrict__ out,
                                                                       uint64_t* __restrict__ cycles) {
  __shared__ __attribute__((aligned(16))) __bf16 tile[2][64 * 64];  // K rows, V rows
  const int tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  for (int i = tid; i < 2 * 64 * 64; i += kIssueThreads) (&tile[0][0])[i] = (__bf16)(seed * (float)(i & 63));
  __syncthreads();
  bf16x8 qf[2][4], kr[4], vr[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qf[0][ks][e] = (__bf16)(seed * (float)(tid + ks + e));
      qf[1][ks][e] = (__bf16)(seed * (float)(tid - ks + e));
      kr[ks][e] = (__bf16)(seed * (float)(lane + ks * e));
      vr[ks][e] = (__bf16)(seed * (float)(lane - ks * e));
    }
  f32x16 o[2][2], sc[2];
  bf16x8 pf[2][2];
  float lsum[2] = {0.f, 0.f};
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) o[qt][0][i] = o[qt][1][i] = sc[qt][i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[qt][0][e] = pf[qt][1][e] = (__bf16)0.f;
  }
  // (the fragments' tile offsets change every step, so the reads stay inside the loop: K rows koff ..
  // koff + 31 of 64, V columns up to voff + 47 of 64)
  int koff = 0, voff = 0;
  auto scores = [&]() {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      f32x16 c;
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = -4.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        c = mfma(LDS ? *reinterpret_cast<const bf16x8*>(&tile[0][(l32 + koff) * 64 + ks * 16 + g * 8]) : kr[ks],
                 qf[qt][ks], c);
      sc[qt] = c;
    }
  };
  auto pv = [&]() {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8 vf = vr[mt * 2 + h];
          if constexpr (LDS) {
            // lane j of each 16-lane group addresses row (j / 4) of its group's 4 rows, column 4 (j % 4)
            const int row = h * 16 + (lane >> 4) * 4 + ((lane & 15) >> 2), col = mt * 32 + 4 * (lane & 3) + voff;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (JATTN_LDS i16x4*)(reinterpret_cast<char*>(&tile[1][0]) + (row * 64 + col) * 2));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (JATTN_LDS i16x4*)(reinterpret_cast<char*>(&tile[1][0]) + ((row + 8) * 64 + col) * 2));
            vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
          o[qt][mt] = mfma(vf, pf[qt][h], o[qt][mt]);
        }
  };
  auto softmax = [&]() {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = fast_exp2(sc[qt][i]);
      pack_probs(p, pf[qt][0], pf[qt][1], lsum[qt]);
    }
  };
  const bool second = w >= 4;  // (wave-uniform)
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  if (MODE == JATTN_PROBE_PINGPONG_PHASED && second) __syncthreads();  // waves 4-7 start one phase later
  for (int it = 0; it < iters; ++it) {
    koff = (it & 1) * 32;
    voff = (it & 1) * 16;
    if constexpr (MODE == JATTN_PROBE_PINGPONG_PHASED) {
      scores();  // MFMA phase: S(t) and PV(t - 1)
      pv();
      __syncthreads();
      softmax();  // softmax phase, while the other wave of the SIMD runs its MFMA phase
      __syncthreads();
    } else {
      scores();
      softmax();
      pv();
      if constexpr (MODE == JATTN_PROBE_PINGPONG_BARRIER) __syncthreads();
    }
  }
  if (MODE == JATTN_PROBE_PINGPONG_PHASED && !second) __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  float sum = lsum[0] + lsum[1];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += o[qt][0][i] + o[qt][1][i];
  out[(size_t)blockIdx.x * kIssueThreads + tid] = sum;
  if (lane == 0) cycles[(size_t)blockIdx.x * (kIssueThreads / 64) + w] = t1 - t0;
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

extern "C" jattn_status jattn_probe_tile(int mode, int blocks, int iters, float seed, float* out, uint64_t* cycles,
                                         hipStream_t stream) {
  if (mode < JATTN_PROBE_TILE_REGS || mode > JATTN_PROBE_TILE_PIPELINED || blocks < 1 || iters < 1 ||
      (int64_t)blocks * jattn::kProbeThreads >= ((int64_t)1 << 31) || out == nullptr || cycles == nullptr ||
      (reinterpret_cast<uintptr_t>(out) & 3u) != 0 || (reinterpret_cast<uintptr_t>(cycles) & 7u) != 0)
    return JATTN_ERROR_INVALID_VALUE;
  switch (mode) {
#define JATTN_TILE_CASE(M) \
  case M: hipLaunchKernelGGL(jattn::probe_tile_kernel<M>, dim3(blocks), dim3(jattn::kProbeThreads), 0, stream, iters, \
                             seed, out, cycles); break;
    JATTN_TILE_CASE(JATTN_PROBE_TILE_REGS)
    JATTN_TILE_CASE(JATTN_PROBE_TILE_LDS)
    JATTN_TILE_CASE(JATTN_PROBE_TILE_LDS_BARRIER)
    JATTN_TILE_CASE(JATTN_PROBE_TILE_ROWS_STATS)
    JATTN_TILE_CASE(JATTN_PROBE_TILE_TRANSPOSED)
    JATTN_TILE_CASE(JATTN_PROBE_TILE_STATS)
    JATTN_TILE_CASE(JATTN_PROBE_TILE_ROWS)
    JATTN_TILE_CASE(JATTN_PROBE_TILE_PIPELINED)
#undef JATTN_TILE_CASE
  }
  return hipGetLastError() == hipSuccess ? JATTN_SUCCESS : JATTN_ERROR_HIP;
}

extern "C" jattn_status jattn_probe_lds_read(int mode, int blocks, int iters, uint64_t* cycles, hipStream_t stream) {
  if (mode < JATTN_PROBE_LDS_B128 || mode > JATTN_PROBE_LDS_B64_TRANSPOSED || blocks < 1 || iters < 1 ||
      (int64_t)blocks * jattn::kProbeThreads >= ((int64_t)1 << 31) || cycles == nullptr ||
      (reinterpret_cast<uintptr_t>(cycles) & 7u) != 0)
    return JATTN_ERROR_INVALID_VALUE;
  if (mode == JATTN_PROBE_LDS_B128)
    hipLaunchKernelGGL(jattn::probe_lds_read_kernel<JATTN_PROBE_LDS_B128>, dim3(blocks), dim3(jattn::kProbeThreads), 0,
                       stream, iters, cycles);
  else if (mode == JATTN_PROBE_LDS_B128_BROADCAST)
    hipLaunchKernelGGL(jattn::probe_lds_read_kernel<JATTN_PROBE_LDS_B128_BROADCAST>, dim3(blocks),
                       dim3(jattn::kProbeThreads), 0, stream, iters, cycles);
  else
    hipLaunchKernelGGL(jattn::probe_lds_read_kernel<JATTN_PROBE_LDS_B64_TRANSPOSED>, dim3(blocks),
                       dim3(jattn::kProbeThreads), 0, stream, iters, cycles);
  return hipGetLastError() == hipSuccess ? JATTN_SUCCESS : JATTN_ERROR_HIP;
}

extern "C" jattn_status jattn_probe_issue(int mode, int blocks, int iters, float seed, float* out, uint64_t* cycles,
                                          hipStream_t stream) {
  if (mode < JATTN_PROBE_ISSUE_MFMA || mode > JATTN_PROBE_ISSUE_SPLIT_EXP || blocks < 1 || iters < 1 ||
      (int64_t)blocks * jattn::kIssueThreads >= ((int64_t)1 << 31) || out == nullptr || cycles == nullptr ||
      (reinterpret_cast<uintptr_t>(out) & 3u) != 0 || (reinterpret_cast<uintptr_t>(cycles) & 7u) != 0)
    return JATTN_ERROR_INVALID_VALUE;
  const dim3 grid(blocks), block(jattn::kIssueThreads);
  switch (mode) {
#define JATTN_ISSUE_CASE(M) \
  case M: hipLaunchKernelGGL(jattn::probe_issue_kernel<M>, grid, block, 0, stream, iters, seed, out, cycles); break;
    JATTN_ISSUE_CASE(JATTN_PROBE_ISSUE_MFMA)
    JATTN_ISSUE_CASE(JATTN_PROBE_ISSUE_FMA)
    JATTN_ISSUE_CASE(JATTN_PROBE_ISSUE_EXP)
    JATTN_ISSUE_CASE(JATTN_PROBE_ISSUE_MIXED_FMA)
    JATTN_ISSUE_CASE(JATTN_PROBE_ISSUE_MIXED_EXP)
    JATTN_ISSUE_CASE(JATTN_PROBE_ISSUE_SPLIT_FMA)
    JATTN_ISSUE_CASE(JATTN_PROBE_ISSUE_SPLIT_EXP)
#undef JATTN_ISSUE_CASE
  }
  return hipGetLastError() == hipSuccess ? JATTN_SUCCESS : JATTN_ERROR_HIP;
}

extern "C" jattn_status jattn_probe_pingpong(int mode, int lds, int blocks, int iters, float seed, float* out,
                                             uint64_t* cycles, hipStream_t stream) {
  if (mode < JATTN_PROBE_PINGPONG_FREE || mode > JATTN_PROBE_PINGPONG_PHASED || (lds != 0 && lds != 1) ||
      blocks < 1 || iters < 1 || (int64_t)blocks * jattn::kIssueThreads >= ((int64_t)1 << 31) || out == nullptr ||
      cycles == nullptr || (reinterpret_cast<uintptr_t>(out) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(cycles) & 7u) != 0)
    return JATTN_ERROR_INVALID_VALUE;
  const dim3 grid(blocks), block(jattn::kIssueThreads);
  switch (mode * 2 + lds) {
#define JATTN_PP_CASE(M, LD)                                                                                 \
  case M * 2 + LD:                                                                                           \
    hipLaunchKernelGGL((jattn::probe_pingpong_kernel<M, LD>), grid, block, 0, stream, iters, seed, out, cycles); \
    break;
    JATTN_PP_CASE(JATTN_PROBE_PINGPONG_FREE, 0)
    JATTN_PP_CASE(JATTN_PROBE_PINGPONG_FREE, 1)
    JATTN_PP_CASE(JATTN_PROBE_PINGPONG_BARRIER, 0)
    JATTN_PP_CASE(JATTN_PROBE_PINGPONG_BARRIER, 1)
    JATTN_PP_CASE(JATTN_PROBE_PINGPONG_PHASED, 0)
    JATTN_PP_CASE(JATTN_PROBE_PINGPONG_PHASED, 1)
#undef JATTN_PP_CASE
  }
  return hipGetLastError() == hipSuccess ? JATTN_SUCCESS : JATTN_ERROR_HIP;
}
