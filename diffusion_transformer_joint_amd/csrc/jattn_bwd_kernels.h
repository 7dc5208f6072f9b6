// Kernels of the backward pass of QK-RMSNorm joint attention on gfx950 (the math and the kernel
// split are described at the top of jattn_bwd.hip). Instantiated by jattn_bwd.hip for head dims up
// to kNarrowMaxD and by jattn_bwd_wide.hip above it; the two files are compiled with different
// accumulator placement.
#pragma once

#include <type_traits>

#include "jattn_device.h"
#include "jattn_launch.h"

namespace jattn {

static_assert(kBwdRowsPerBlock == kBwdWaves * kWaveRows && kBwdWaves >= 2, "backward workgroup shape");

// Waves per SIMD the register allocation targets. dq kernel: two at every head dim (above D = 64 its
// tile reads the key and value row fragments one k-step at a time, so that they fit beside the dQ
// accumulators). dk/dv kernel: two up to D = 72, one above (from D = 80 its dK and dV accumulators
// and key/value fragments need the whole register file).
template <int D>
constexpr int dq_waves_per_eu() { return 2; }
template <int D>
constexpr int dkdv_waves_per_eu() { return D <= kNarrowMaxD ? 2 : 1; }
// Two waves per SIMD with tiles padded past 64 columns: the tightest case for LDS and registers.
template <int D, int WPE>
constexpr bool bwd_tight() { return Dims<D>::DM > 64 && WPE == 2; }
// LDS ring depth: four tile buffers (loads issued three tiles ahead; measured slightly faster than
// three), two in the tight case, whose padded tiles would otherwise not leave room for two workgroups per CU.
template <int D, int WPE>
constexpr int bwd_nbuf() { return bwd_tight<D, WPE>() || kBwdWaves < 4 ? 2 : 4; }


// LDS plan of the two main kernels. The swizzled layout (D = 64, 128) serves both row-fragment and
// transposed reads without bank conflicts; other head dims use padded rows.
template <int D>
struct DqCfg {
  using LK = Lay<D, kSwizzled>;  // normalised key rows: S (row fragments) and dQ (transposed)
  using LV = Lay<D, kSwizzled>;  // value rows: dP (row fragments)
  static constexpr int NB = bwd_nbuf<D, dq_waves_per_eu<D>()>();
  static constexpr int STAGE = NB * (LK::ELEMS + LV::ELEMS) * 2;
  // LDS bytes of the kernel (two-stream: the epilogue's per-stream column sums reuse the ring)
  template <bool S>
  static constexpr int bytes() {
    return S && colsum2_scratch_floats<D, kBwdWaves>() * 4 > STAGE ? colsum2_scratch_floats<D, kBwdWaves>() * 4
                                                                   : STAGE;
  }
};

template <int D>
struct DkdvCfg {
  using LQ = Lay<D, kSwizzled>;  // pre-scaled normalised query rows: S and dK
  using LO = Lay<D, kSwizzled>;  // dout rows: dP and dV
  static constexpr int NB = bwd_nbuf<D, dkdv_waves_per_eu<D>()>();
  static constexpr int STAGE = NB * (LQ::ELEMS + LO::ELEMS) * 2;
  static constexpr int STATS = NB * 2 * kTile * 4;  // -lse2 and -delta per streamed row
  template <bool S>
  static constexpr int bytes() {
    constexpr int scratch = (S ? colsum2_scratch_floats<D, kBwdWaves>() : colsum_scratch_floats<D, kBwdWaves>()) * 4;
    return STAGE + STATS > scratch ? STAGE + STATS : scratch;
  }
};

// A wave row in the C/D layout (pair j4 of tile mt holds d = 32 mt + 8 j4 + 4 g + [0..3]) as raw bf16
// pairs, for the RMSNorm backward of the epilogue. Where registers allow it the row is loaded in the
// prologue and kept through the tile loop: loading it after the loop leaves its latency, for every
// workgroup at once, between the last tile and the epilogue.
template <int D>
struct RowC {
  u32x2 w[Dims<D>::MT][4];
};
template <int D, int WPE>
constexpr bool keep_row_c() {
  // (no registers to spare in the tight case; at one wave per SIMD the loops use them better than the
  // row: without it, dq 7 % and dk/dv 4 % faster at D = 128)
  return WPE == 2 && !bwd_tight<D, WPE>();
}

template <int D>
__device__ __forceinline__ void load_row_c(RowC<D>& x, const uint16_t* __restrict__ row, bool valid, int g) {
#pragma unroll
  for (int mt = 0; mt < Dims<D>::MT; ++mt)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = mt * 32 + j4 * 8 + g * 4;
      x.w[mt][j4] = valid && d0 < D ? *reinterpret_cast<const u32x2*>(row + d0) : (u32x2){0u, 0u};
    }
}

// RMSNorm backward for one wave row held in the C/D layout (lane = row; register i of tile mt
// holds d = 32*mt + 8*(i/4) + 4*g + i%4; the other half of the row is in lane l^32). On entry dxn
// holds the gradient with respect to the normalised row divided by gpre[d] (the factor the MFMA
// operands left out; null = 1); xc is the raw row (zeros when not `valid`); `gain` is the row's own
// RMSNorm gain. If `exists`, writes the bf16 gradient row
// (zeros when not `valid`, i.e. a padded key) and, if xsrow is set, bf16(x * r * xs_mul * xs_gain[d])
// (xs_gain null = 1). With TSUM, dxn holds dxn * x * r on return (this row's term of the gain
// gradient; zeros for rows that are not valid).
template <int D, bool TSUM>
__device__ __forceinline__ void rmsnorm_backward_row(f32x16 (&dxn)[Dims<D>::MT], const RowC<D>& xc,
                                                     const float* __restrict__ gain, const float* __restrict__ gpre,
                                                     float r, bool valid, bool exists,
                                                     uint16_t* __restrict__ dxrow, uint16_t* __restrict__ xsrow,
                                                     float xs_mul, const float* __restrict__ xs_gain, int g) {
  using Dm = Dims<D>;
  float x[Dm::MT][16];
  float gd[Dm::MT][16];  // gain * (gradient with respect to the normalised row)
  float t = 0.f;
#pragma unroll
  for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = mt * 32 + j4 * 8 + g * 4;
      float xv[4];
      unpack4(xc.w[mt][j4], xv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = j4 * 4 + e;
        x[mt][i] = xv[e];
        gd[mt][i] = d0 < D ? gain[d0 + e] * (gpre ? gpre[d0 + e] : 1.f) * dxn[mt][i] : 0.f;
        t += gd[mt][i] * xv[e];
      }
    }
  t += __shfl_xor(t, 32);
  const float c3 = r * r * r * (1.0f / D) * t;
  const float xs = r * xs_mul;
#pragma unroll
  for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = mt * 32 + j4 * 8 + g * 4;
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = j4 * 4 + e;
        y[e] = valid ? r * gd[mt][i] - x[mt][i] * c3 : 0.f;
      }
      if (exists && d0 < D) {
        *reinterpret_cast<u32x2*>(dxrow + d0) = (u32x2){pack2(y[0], y[1]), pack2(y[2], y[3])};
        const int i = j4 * 4;
        if (xsrow) {
          float z[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] = x[mt][i + e] * xs * (xs_gain ? xs_gain[d0 + e] : 1.f);
          *reinterpret_cast<u32x2*>(xsrow + d0) = (u32x2){pack2(z[0], z[1]), pack2(z[2], z[3])};
        }
      }
      if constexpr (TSUM) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = j4 * 4 + e;
          dxn[mt][i] = valid ? dxn[mt][i] * x[mt][i] * r : 0.f;
        }
      }
    }
}

// Scheduling pattern for code emitted just before it: N groups of one MFMA followed by V VALU
// instructions, so that a stage's MFMAs issue under another stage's independent VALU work (one wave per
// SIMD has no second wave to fill the MFMA pipe while it runs its softmax).
template <int N, int V>
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);  // then V VALU instructions
  }
}

// Per-lane LDS byte offsets of a swizzled or padded tile's row fragments (row l32, k-step ks) and
// transposed fragments (column block mt, rows r and r + 8), computed once: rows 32 and 16 further on
// share the swizzle, so both halves and both 16-row steps are immediate offsets.
template <int D>
struct LaneOffs {
  uint32_t row[Dims<D>::KS];
  uint32_t tr[Dims<D>::MT][2];
  template <class LY>
  __device__ void init(int lane) {
    const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int ks = 0; ks < Dims<D>::KS; ++ks) row[ks] = 2u * (uint32_t)LY::off(l32, ks * 16 + g * 8);
    const int r = 4 * (lane >> 5) + ((lane & 15) >> 2);
    const int c = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
#pragma unroll
    for (int mt = 0; mt < Dims<D>::MT; ++mt) {
      tr[mt][0] = 2u * (uint32_t)LY::off(r, mt * 32 + c);
      tr[mt][1] = 2u * (uint32_t)LY::off(r + 8, mt * 32 + c);
    }
  }
};

// ------------------------------------------------------------------------------------------------
// dq kernel: query-parallel

// One 64-key tile: for both 32-key halves S'^T = Kr Q'^T and dP^T - Delta = V dO^T (lane = query),
// dS^T = P * (dP - Delta) with P = exp2(S' - lse2), then dQn^T += Kr^T dS^T. MASKED: keys at or
// past n are seeded with -inf (P = 0).
// The halves run one after the other (issuing the second half's row reads under the first half's
// products measured no faster). Above D = 64 the row fragments are read one k-step at a time (below).
// (The staged order of the one-wave-per-SIMD dk/dv tile, with the MFMAs of one stage under another's
// softmax, ran the dq kernel at one wave per SIMD in 577.5 us at B4 L2381 H24 D128; the streamed tile
// at two waves per SIMD takes 524.0 us.)
// W (local window): masked tiles also seed -inf outside the lane's query window qrow - wl .. qrow + wr.
template <int D, bool MASKED, bool W = false>
__device__ __forceinline__ void dq_tile(const __bf16* __restrict__ kt, const __bf16* __restrict__ vt,
                                        const bf16x8 (&qf)[Dims<D>::KS], const bf16x8 (&dof)[Dims<D>::KS],
                                        const f32x16& cs, const f32x16& cp, f32x16 (&acc)[Dims<D>::MT], int key0,
                                        int n, int lane, int qrow = 0, int wl = 0, int wr = 0) {
  using Dm = Dims<D>;
  using LK = typename DqCfg<D>::LK;
  using LV = typename DqCfg<D>::LV;
  constexpr int KS = Dm::KS, MT = Dm::MT;
  const int g = lane >> 5, l32 = lane & 31;
  bf16x8 kr[2][KS], vr[2][KS], f[2][2];
  f32x16 s[2], dp[2];
  auto rows = [&](int h) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kr[h][ks] = lds_row_frag<LK>(kt, h * 32 + l32, ks * 16 + g * 8);
      vr[h][ks] = lds_row_frag<LV>(vt, h * 32 + l32, ks * 16 + g * 8);
    }
  };
  auto scores = [&](int h) {
    s[h] = cs;
    dp[h] = cp;
    if constexpr (MASKED && W) {
      // keys key0 + c with c = h*32 + (i>>2)*8 + 4g + (i&3) are allowed for c in [clo, clo + span),
      // tested as one unsigned compare per element
      const int clo = qrow - wl - key0, span = max(min(n, qrow + wr + 1) - key0 - clo, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = h * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
        s[h][i] = (uint32_t)(c - clo) < (uint32_t)span ? s[h][i] : -INFINITY;
      }
    } else if constexpr (MASKED) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (key0 + h * 32 + (i >> 2) * 8 + g * 4 + (i & 3) >= n) s[h][i] = -INFINITY;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s[h] = mfma(kr[h][ks], qf[ks], s[h]);
      dp[h] = mfma(vr[h][ks], dof[ks], dp[h]);
    }
  };
  auto softmax = [&](int h) {
    float ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) ds[i] = fast_exp2(s[h][i]) * dp[h][i];
    f[h][0] = to_bf16x8(ds);
    f[h][1] = to_bf16x8(ds + 8);
  };
  auto accumulate = [&](int h) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[mt] = mfma(lds_tr_frag<LK>(kt, h * 32, mt * 32, lane), f[h][0], acc[mt]);
      acc[mt] = mfma(lds_tr_frag<LK>(kt, h * 32 + 16, mt * 32, lane), f[h][1], acc[mt]);
    }
  };
  if constexpr (KS > 4) {
    // Two waves per SIMD at wide head dims: each key and value row fragment is read from LDS just
    // before its MFMAs instead of a whole half at once, and the MFMA seeds are formed in each tile from
    // the row statistics rather than kept through the loop, so that the tile fits beside the dQ
    // accumulators in 256 registers.
    // (the lane index is made opaque too: the per-lane LDS offsets derived from it are then formed in
    // each tile instead of being hoisted out of the loop and spilled)
    float nl = cs[0], nd = cp[0];
    int ln = lane;
    asm volatile("" : "+v"(nl), "+v"(nd), "+v"(ln));
    const int gg = ln >> 5, r32 = ln & 31;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[h][i] = nl;
        dp[h][i] = nd;
      }
      if constexpr (MASKED && W) {
        const int clo = qrow - wl - key0, span = max(min(n, qrow + wr + 1) - key0 - clo, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = h * 32 + (i >> 2) * 8 + gg * 4 + (i & 3);
          s[h][i] = (uint32_t)(c - clo) < (uint32_t)span ? s[h][i] : -INFINITY;
        }
      } else if constexpr (MASKED) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key0 + h * 32 + (i >> 2) * 8 + gg * 4 + (i & 3) >= n) s[h][i] = -INFINITY;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 k1 = lds_row_frag<LK>(kt, h * 32 + r32, ks * 16 + gg * 8);
        const bf16x8 v1 = lds_row_frag<LV>(vt, h * 32 + r32, ks * 16 + gg * 8);
        s[h] = mfma(k1, qf[ks], s[h]);
        dp[h] = mfma(v1, dof[ks], dp[h]);
      }
      softmax(h);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt] = mfma(lds_tr_frag<LK>(kt, h * 32, mt * 32, ln), f[h][0], acc[mt]);
        acc[mt] = mfma(lds_tr_frag<LK>(kt, h * 32 + 16, mt * 32, ln), f[h][1], acc[mt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    rows(0);
    scores(0);
    softmax(0);
    accumulate(0);
    rows(1);
    scores(1);
    softmax(1);
    accumulate(1);
  }
}

// One work item of the dq kernel: query rows [128 blk, 128 blk + 128) of (sequence, head) pair bh.
// Varlen (V): a block past the end of its sequence has nothing to do (its statistics rows belong to
// the next pair).
template <int D, bool S, bool V, bool W>
__device__ __forceinline__ void dq_item(const BwdArgs& a, char* smem, int bh, int blk) {
  using Dm = Dims<D>;
  using Cfg = DqCfg<D>;
  using LK = typename Cfg::LK;
  using LV = typename Cfg::LV;
  constexpr int NB = Cfg::NB;
  __bf16* sk = reinterpret_cast<__bf16*>(smem);
  __bf16* sv = sk + NB * LK::ELEMS;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int H = a.H;
  const int b = bh / H, h = bh - b * H;
  // (fixed-length batches keep the offsets in their original form, e.g. (size_t)bh * L: written through
  // the sequence geometry instead, the compiler allocated the tile loop's registers differently and
  // the loop ran slower)
  const SeqGeom<V> seq(a.cu_seqlens, b, a.L, a.total, a.L);
  const int L = V ? seq.L : a.L;
  if (V && blk * kBwdRowsPerBlock >= L) return;  // (uniform over the workgroup)
  const int n = !V && a.valid_len ? min(max(a.valid_len[b], 0), L) : L;
  const size_t row0 = V ? seq.row0(h, H) : (size_t)bh * L;  // first workspace / LSE row of the pair
  const RowMap<S> map(V ? (size_t)seq.start : (size_t)b * (S ? a.n0 : L), (size_t)b * (L - a.n0), h, H, D,
                      S ? a.n0 : L);

  // start streaming the first key tiles before the per-row set-up
  const int ntiles = (n + kTile - 1) / kTile, nfull = n / kTile;
  DirectTile<D, LK, kBwdWaves> dk;
  DirectTile<D, LV, kBwdWaves> dv;
  dk.init(D, wave, lane);
  dv.init(map.rs, wave, lane);
  const uint16_t* kb = a.kr + row0 * D;
  auto issue = [&](int t, int buf) {
    dk.issue(tile_rsrc<D>(kb, D, t * kTile, n), sk + buf * LK::ELEMS, wave);
    dv.issue_blocks(S, a.v, a.v1, map.o0, map.o1, map.n0, map.rs, t * kTile, n, sv + buf * LV::ELEMS, wave,
                                 lane);
  };
  // (local window: the key tiles the block's query rows can reach)
  const TileRange tr = W ? window_tiles(blk * kBwdRowsPerBlock, min(L, (blk + 1) * kBwdRowsPerBlock), a.wl, a.wr, n, n)
                         : TileRange{0, 0, 0, 0};
  if constexpr (W) {
    for (int i = 0; i < NB - 1 && tr.lo + i < tr.hi; ++i) issue(tr.lo + i, i);
  } else {
    for (int t = 0; t < NB - 1 && t < ntiles; ++t) issue(t, t);
  }

  const int qrow = blk * kBwdRowsPerBlock + wave * kWaveRows + l32;
  const bool qvalid = qrow < L;
  // the row's Q gain (two-stream: its own stream's; the joint form folds both gains in)
  const float* gq = a.gains + (S ? map.block(qrow) * 2 * D : 0);
  const uint16_t* qptr = map.row(a.q, a.q1, qrow);
  // (The dO, O and LSE loads are issued after the Q normalisation: at two waves per SIMD the other wave
  // covers the waits, and issuing every row load first held the rows longer and made dq 2 % slower at
  // D = 64.)
  bf16x8 qf[Dm::KS], dof[Dm::KS], x[Dm::KS], o[Dm::KS];
  RowC<D> xq;
  float lse = 0.f;
  load_row_frags_raw<D>(x, qptr, qvalid, g);
  const float rq = rmsnorm_row_frags<D>(qf, x, gq, S ? nullptr : a.gains + D, a.c, a.eps, qvalid, g);
  load_row_frags_raw<D>(dof, map.row(a.dout, a.dout1, qrow), qvalid, g);
  if constexpr (keep_row_c<D, dq_waves_per_eu<D>()>()) load_row_c<D>(xq, qptr, qvalid, g);
  load_row_frags_raw<D>(o, map.row(a.out, a.out1, qrow), qvalid, g);
  float delta = 0.f;
#pragma unroll
  for (int ks = 0; ks < Dm::KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) delta += (float)dof[ks][e] * (float)o[ks][e];
  delta += __shfl_xor(delta, 32);
  if (qvalid) lse = a.lse[row0 + qrow];
  const float lse2 = lse * kLog2e;
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

  wait_vmem();
  __syncthreads();
  // One loop over the full tiles and a separate step for the partial one: a masked / unmasked
  // branch inside the loop makes the two bodies keep the accumulators in different registers, with
  // copies at the join.
  // a wave whose 32 query rows all lie past L keeps the ring going but skips the math
  const bool active = blk * kBwdRowsPerBlock + wave * kWaveRows < L;
  int cur = 0;
  auto step = [&](auto masked, int t) {
    const bool ahead = t + NB - 1 < ntiles;
    if (ahead) issue(t + NB - 1, cur == 0 ? NB - 1 : cur - 1);
    if (active)
      dq_tile<D, decltype(masked)::value>(sk + cur * LK::ELEMS, sv + cur * LV::ELEMS, qf, dof, cs, cp, acc,
                                          t * kTile, n, lane);
    ring_barrier<DirectTile<D, LK, kBwdWaves>::MIN_PER_WAVE + DirectTile<D, LV, kBwdWaves>::MIN_PER_WAVE, NB - 2>(ntiles - 2 - t);
    cur = cur + 1 == NB ? 0 : cur + 1;
  };
  if constexpr (!W) {
    for (int t = 0; t < nfull; ++t) step(std::false_type{}, t);
    if (nfull < ntiles) step(std::true_type{}, nfull);
  } else {
    auto wstep = [&](auto masked, int t) {
      if (t + NB - 1 < tr.hi) issue(t + NB - 1, cur == 0 ? NB - 1 : cur - 1);
      if (active)
        dq_tile<D, decltype(masked)::value, true>(sk + cur * LK::ELEMS, sv + cur * LV::ELEMS, qf, dof, cs, cp, acc,
                                                  t * kTile, n, lane, qrow, a.wl, a.wr);
      ring_barrier<DirectTile<D, LK, kBwdWaves>::MIN_PER_WAVE + DirectTile<D, LV, kBwdWaves>::MIN_PER_WAVE, NB - 2>(
          tr.hi - 2 - t);
      cur = cur + 1 == NB ? 0 : cur + 1;
    };
    int t = tr.lo;
    for (; t < tr.flo; ++t) wstep(std::true_type{}, t);
    for (; t < tr.fhi; ++t) wstep(std::false_type{}, t);
    for (; t < tr.hi; ++t) wstep(std::true_type{}, t);
  }

  // row statistics for the key-parallel kernel, for every row of the block (-inf / 0 past L)
  if (g == 0) {
    const size_t si = (V ? seq.stat0(b, h, H) : (size_t)bh * a.lp) + qrow;
    a.nlse2[si] = qvalid ? -lse2 : -INFINITY;
    a.ndelta[si] = qvalid ? -delta : 0.f;
  }
  // dQn = scale * (dS Kr) times g_k in the joint form (its streamed key rows carry no gain)
#pragma unroll
  for (int mt = 0; mt < Dm::MT; ++mt) acc[mt] *= a.scale;
  if constexpr (!keep_row_c<D, dq_waves_per_eu<D>()>()) load_row_c<D>(xq, qptr, qvalid, g);
  uint16_t* qsrow = a.qs + (row0 + qrow) * D;
  if constexpr (!S) {
    rmsnorm_backward_row<D, false>(acc, xq, a.gains, a.gains + D, rq, qvalid, qvalid, map.row(a.dq, a.dq1, qrow),
                                   qsrow, a.c, nullptr, g);
  } else {
    // Qs carries the row's own Q gain; the gain-gradient terms of the block go to the partial sets of
    // the two streams (rows below n0 - 128 blk are image rows)
    rmsnorm_backward_row<D, true>(acc, xq, gq, nullptr, rq, qvalid, qvalid, map.row(a.dq, a.dq1, qrow), qsrow, a.c,
                                  gq, g);
    const size_t set = (size_t)D * a.items, item = (size_t)bh * a.nblk + blk;
    const int split = min(max(map.n0 - blk * kBwdRowsPerBlock, 0), kBwdRowsPerBlock);
    block_column_sums2<D, kBwdWaves, true>(acc, reinterpret_cast<float*>(smem), a.part + item, a.part + 2 * set + item,
                                           (size_t)a.items, split, tid);
  }
}

template <int D, bool S, bool V, bool W>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(dq_waves_per_eu<D>())))
void bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[DqCfg<D>::template bytes<S>()];
  // (an item ends with its tile loop's barrier and, in the joint form, its epilogue does not touch
  // LDS, so the next item may refill the ring right away; the two-stream epilogue's column sums do)
  if constexpr (V) {
    for (PairIter it(a.B * a.H, a.nblk); it.valid(); it.next()) dq_item<D, S, V, W>(a, smem, it.pair(), it.blk());
  } else {
    for (ItemIter it(a.items); it.valid(); it.next()) {
      const int bh = it.item() / a.nblk;
      dq_item<D, S, V, W>(a, smem, bh, it.item() - bh * a.nblk);
      if constexpr (S) __syncthreads();
    }
  }
}

// ------------------------------------------------------------------------------------------------
// dkdv kernel: key-parallel

// One 64-query tile: for both 32-query halves S' = Qs Kf^T and dP - Delta = dO V^T (lane = key),
// P = exp2(S' - lse2), dS = P * (dP - Delta), then dV^T += dO^T P and dKn^T += Qs^T dS.
// sl / sd hold -lse2 and -Delta of the tile's rows. KMASK: this wave holds keys at or past n, whose
// P is forced to zero. WM (local window): P is also zero for the queries outside the window of this
// lane's key (queries key - wr .. key + wl see it); q0 is the tile's first query row. (Selected after
// the exp: a query with no key in its window has lse = -inf, so its S - lse is +inf.)
template <int D, bool KMASK, bool WM = false>
__device__ __forceinline__ void dkdv_tile(const __bf16* __restrict__ qt, const __bf16* __restrict__ ot,
                                          const float* __restrict__ sl, const float* __restrict__ sd,
                                          const bf16x8 (&kf)[Dims<D>::KS], const bf16x8 (&vf)[Dims<D>::KS],
                                          f32x16 (&dva)[Dims<D>::MT], f32x16 (&dka)[Dims<D>::MT], bool kvalid,
                                          int lane, int q0 = 0, int key = 0, int wl = 0, int wr = 0) {
  using Dm = Dims<D>;
  using LQ = typename DkdvCfg<D>::LQ;
  using LO = typename DkdvCfg<D>::LO;
  constexpr int KS = Dm::KS, MT = Dm::MT;
  const int g = lane >> 5, l32 = lane & 31;
  bf16x8 qr[2][KS], orr[2][KS], pf[2][2], df[2][2];
  f32x16 s[2], dp[2];
  auto rows = [&](int h) {  // statistics (the MFMA seeds) and row fragments
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(sl + h * 32 + j4 * 8 + g * 4);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(sd + h * 32 + j4 * 8 + g * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[h][j4 * 4 + e] = l4[e];
        dp[h][j4 * 4 + e] = d4[e];
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qr[h][ks] = lds_row_frag<LQ>(qt, h * 32 + l32, ks * 16 + g * 8);
      orr[h][ks] = lds_row_frag<LO>(ot, h * 32 + l32, ks * 16 + g * 8);
    }
  };
  auto scores = [&](int h) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s[h] = mfma(qr[h][ks], kf[ks], s[h]);
      dp[h] = mfma(orr[h][ks], vf[ks], dp[h]);
    }
  };
  auto probs = [&](int h) {
    float p[16], ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = fast_exp2(s[h][i]);
      if constexpr (KMASK) p[i] = kvalid ? p[i] : 0.f;
      if constexpr (WM) {
        // queries q0 + c with c in [key - wr - q0, key + wl - q0] see this key, i.e. 0 <= c + wr + q0 - key
        // <= wl + wr, tested as one unsigned compare per element against a lane offset
        const int c = h * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
        p[i] = (uint32_t)(c + wr + q0 - key) <= (uint32_t)(wl + wr) ? p[i] : 0.f;
      }
      ds[i] = p[i] * dp[h][i];
    }
    pf[h][0] = to_bf16x8(p);
    pf[h][1] = to_bf16x8(p + 8);
    df[h][0] = to_bf16x8(ds);
    df[h][1] = to_bf16x8(ds + 8);
  };
  auto accumulate = [&](int h) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      dva[mt] = mfma(lds_tr_frag<LO>(ot, h * 32, mt * 32, lane), pf[h][0], dva[mt]);
      dva[mt] = mfma(lds_tr_frag<LO>(ot, h * 32 + 16, mt * 32, lane), pf[h][1], dva[mt]);
      dka[mt] = mfma(lds_tr_frag<LQ>(qt, h * 32, mt * 32, lane), df[h][0], dka[mt]);
      dka[mt] = mfma(lds_tr_frag<LQ>(qt, h * 32 + 16, mt * 32, lane), df[h][1], dka[mt]);
    }
  };
  rows(0);
  scores(0);
  probs(0);
  accumulate(0);
  rows(1);
  scores(1);
  probs(1);
  accumulate(1);
}

// The dk/dv tile for the instantiations that run one wave per SIMD (D > 72): the same arithmetic as
// dkdv_tile with an explicit issue order, every LDS read a stage ahead of its use and the MFMAs of one
// stage under the VALU work of another:
//   statistics and rows of half 0 | scores(0) | transposed fragments of half 0, rows and statistics of
//   half 1 | probabilities(0) with scores(1) | probabilities(1) with accumulate(0) | transposed
//   fragments of half 1 | accumulate(1)
// With no second wave on the SIMD to run while one waits, the default schedule (each MFMA waits for
// the LDS read issued just before it, and the MFMA pipe idles through the softmax) leaves both
// exposed: at B4 L2381 H24 D128 the plain staged order took dk/dv 824 -> 749 us, the interleave
// 721 -> 688 us. (With two waves per SIMD the explicit order measured no faster and needs more
// registers, so those instantiations keep dkdv_tile.) LDS addresses come from LaneOffs.

template <int D, bool KMASK, bool WM = false>
__device__ __forceinline__ void dkdv_tile_staged(const __bf16* __restrict__ qt, const __bf16* __restrict__ ot,
                                                 const float* __restrict__ sl, const float* __restrict__ sd,
                                                 const bf16x8 (&kf)[Dims<D>::KS], const bf16x8 (&vf)[Dims<D>::KS],
                                                 f32x16 (&dva)[Dims<D>::MT], f32x16 (&dka)[Dims<D>::MT], bool kvalid,
                                                 int lane, const LaneOffs<D>& lo, int q0 = 0, int key = 0, int wl = 0,
                                                 int wr = 0) {
  using Dm = Dims<D>;
  using LQ = typename DkdvCfg<D>::LQ;
  static_assert(std::is_same<LQ, typename DkdvCfg<D>::LO>::value, "Qs and dO tiles share one layout");
  constexpr int KS = Dm::KS, MT = Dm::MT;
  const int g = lane >> 5;
  bf16x8 qr[2][KS], orr[2][KS], pf[2][2], df[2][2], tq[MT][2], to[MT][2];
  f32x16 s[2], dp[2];
  const char* qb = reinterpret_cast<const char*>(qt);
  const char* ob = reinterpret_cast<const char*>(ot);
  constexpr int RB = 32 * LQ::PITCH * 2;  // bytes between the two 32-row halves
  auto seeds = [&](int h) {
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(sl + h * 32 + j4 * 8 + g * 4);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(sd + h * 32 + j4 * 8 + g * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[h][j4 * 4 + e] = l4[e];
        dp[h][j4 * 4 + e] = d4[e];
      }
    }
  };
  auto rows = [&](int h) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qr[h][ks] = *reinterpret_cast<const bf16x8*>(qb + lo.row[ks] + h * RB);
      orr[h][ks] = *reinterpret_cast<const bf16x8*>(ob + lo.row[ks] + h * RB);
    }
  };
  auto scores = [&](int h) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s[h] = mfma(qr[h][ks], kf[ks], s[h]);
      dp[h] = mfma(orr[h][ks], vf[ks], dp[h]);
    }
  };
  auto tr = [&](const char* b, int mt, int r0) {  // rows r0 .. r0 + 15 of the tile, column block mt
    const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((JATTN_LDS i16x4*)(b + lo.tr[mt][0] + r0 * LQ::PITCH * 2));
    const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((JATTN_LDS i16x4*)(b + lo.tr[mt][1] + r0 * LQ::PITCH * 2));
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4, x), __builtin_bit_cast(bf16x4, y), 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto trload = [&](int h) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      to[mt][0] = tr(ob, mt, h * 32);
      to[mt][1] = tr(ob, mt, h * 32 + 16);
      tq[mt][0] = tr(qb, mt, h * 32);
      tq[mt][1] = tr(qb, mt, h * 32 + 16);
    }
  };
  auto probs = [&](int h) {
    float p[16], ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = fast_exp2(s[h][i]);
      if constexpr (KMASK) p[i] = kvalid ? p[i] : 0.f;
      if constexpr (WM) {
        // queries q0 + c with c in [key - wr - q0, key + wl - q0] see this key, i.e. 0 <= c + wr + q0 - key
        // <= wl + wr, tested as one unsigned compare per element against a lane offset
        const int c = h * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
        p[i] = (uint32_t)(c + wr + q0 - key) <= (uint32_t)(wl + wr) ? p[i] : 0.f;
      }
      ds[i] = p[i] * dp[h][i];
    }
    pf[h][0] = to_bf16x8(p);
    pf[h][1] = to_bf16x8(p + 8);
    df[h][0] = to_bf16x8(ds);
    df[h][1] = to_bf16x8(ds + 8);
  };
  auto accumulate = [&](int h) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      dva[mt] = mfma(to[mt][0], pf[h][0], dva[mt]);
      dva[mt] = mfma(to[mt][1], pf[h][1], dva[mt]);
      dka[mt] = mfma(tq[mt][0], df[h][0], dka[mt]);
      dka[mt] = mfma(tq[mt][1], df[h][1], dka[mt]);
    }
  };
  // (sched_barrier(0) keeps each stage's instructions in place: left alone, the scheduler sinks the
  // reads back down to their first use)
  seeds(0);
  rows(0);
  __builtin_amdgcn_sched_barrier(0);
  scores(0);
  __builtin_amdgcn_sched_barrier(0);
  trload(0);
  rows(1);
  seeds(1);
  __builtin_amdgcn_sched_barrier(0);
  probs(0);
  scores(1);
  interleave_mfma_valu<2 * KS, 3>();
  __builtin_amdgcn_sched_barrier(0);
  probs(1);
  accumulate(0);
  interleave_mfma_valu<4 * MT, 3>();
  __builtin_amdgcn_sched_barrier(0);
  trload(1);
  __builtin_amdgcn_sched_barrier(0);
  accumulate(1);
  __builtin_amdgcn_sched_barrier(0);
}

// One dk/dv tile: the staged form at one wave per SIMD, else the compiler's schedule.
template <int D, bool KMASK, bool WM = false>
__device__ __forceinline__ void dkdv_tile_any(const __bf16* __restrict__ qt, const __bf16* __restrict__ ot,
                                              const float* __restrict__ sl, const float* __restrict__ sd,
                                              const bf16x8 (&kf)[Dims<D>::KS], const bf16x8 (&vf)[Dims<D>::KS],
                                              f32x16 (&dva)[Dims<D>::MT], f32x16 (&dka)[Dims<D>::MT], bool kvalid,
                                              int lane, const LaneOffs<D>& lo, int q0 = 0, int key = 0, int wl = 0,
                                              int wr = 0) {
  if constexpr (dkdv_waves_per_eu<D>() == 1)
    dkdv_tile_staged<D, KMASK, WM>(qt, ot, sl, sd, kf, vf, dva, dka, kvalid, lane, lo, q0, key, wl, wr);
  else
    dkdv_tile<D, KMASK, WM>(qt, ot, sl, sd, kf, vf, dva, dka, kvalid, lane, q0, key, wl, wr);
}

// `active`: this wave holds at least one valid key (a wave of padded keys only keeps the ring going).
// Streams the query rows of (sequence, head) pair bh: Qs, dout (through `map`) and the statistics.
// W (local window): only the query tiles [tr.lo, tr.hi), the ends [tr.lo, tr.flo) and [tr.fhi, tr.hi)
// with the window mask (tile t in buffer (t - tr.lo) % NB); key is this lane's key row.
template <int D, bool S, bool V, bool W, bool KMASK>
__device__ __forceinline__ void dkdv_loop(const BwdArgs& a, char* smem, const RowMap<S>& map, int bh,
                                          const TileRange& tr, int key,
                                          const bf16x8 (&kf)[Dims<D>::KS], const bf16x8 (&vf)[Dims<D>::KS],
                                          f32x16 (&dva)[Dims<D>::MT], f32x16 (&dka)[Dims<D>::MT], bool kvalid,
                                          bool active, int tid) {
  using Cfg = DkdvCfg<D>;
  using LQ = typename Cfg::LQ;
  using LO = typename Cfg::LO;
  constexpr int NB = Cfg::NB;
  __bf16* sq = reinterpret_cast<__bf16*>(smem);
  __bf16* so = sq + NB * LQ::ELEMS;
  float* sl = reinterpret_cast<float*>(smem + Cfg::STAGE);  // [NB][kTile]
  float* sd = sl + NB * kTile;                                // [NB][kTile]
  const int lane = tid & 63, wave = wave_id();
  // (fixed-length batches: the original offset expressions, see dq_item)
  const int H = a.H, b = bh / H, h = bh - b * H;
  const SeqGeom<V> seq(a.cu_seqlens, b, a.L, a.total, a.L);
  const int L = V ? seq.L : a.L;
  const uint16_t* qb = a.qs + (V ? seq.row0(h, H) : (size_t)bh * L) * D;
  const size_t st0 = V ? seq.stat0(b, h, H) : (size_t)bh * a.lp;
  const int lp = V ? seq.lp : a.lp;
  DirectTile<D, LQ, kBwdWaves> dq;
  DirectTile<D, LO, kBwdWaves> dout;
  dq.init(D, wave, lane);
  const int rs = map.rs;
  dout.init(rs, wave, lane);
  const uint16_t* ob = a.dout + map.o0;  // (joint form)
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.nlse2 + st0, (uint32_t)lp * 4u);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.ndelta + st0, (uint32_t)lp * 4u);
  // Tile t: rows [64 t, 64 t + 64) of Qs and dO (zeros past L) and of the statistics (written by the
  // dq kernel for every row of its blocks, so 64 t + 63 < lp). Waves 0 and 1 carry the statistics.
  auto issue = [&](int t, int buf) {
    if (wave == 0)
      lds_load_dwords(rl, sl + buf * kTile, (uint32_t)(t * kTile + lane) * 4u);
    else if (wave == 1)
      lds_load_dwords(rd, sd + buf * kTile, (uint32_t)(t * kTile + lane) * 4u);
    dq.issue(tile_rsrc<D>(qb, D, t * kTile, L), sq + buf * LQ::ELEMS, wave);
    if constexpr (S)
      dout.issue_blocks(true, a.dout, a.dout1, map.o0, map.o1, map.n0, rs, t * kTile, L, so + buf * LO::ELEMS, wave,
                        lane);
    else
      dout.issue(tile_rsrc<D>(ob, rs, t * kTile, L), so + buf * LO::ELEMS, wave);
  };
  const int ntiles = (L + kTile - 1) / kTile;
  LaneOffs<D> lo;
  if constexpr (dkdv_waves_per_eu<D>() == 1) lo.template init<LQ>(lane);
  // Two waves per SIMD with a 4-buffer ring: two query tiles per barrier (each step computes tiles t and
  // t + 1 and loads t + 2 and t + 3 into the buffers the previous step used; 2 % faster at D = 64 than a
  // barrier per tile. The dq kernel measured slower that way and keeps one tile per barrier.)
  constexpr bool PAIRS = NB == 4 && !W && dkdv_waves_per_eu<D>() == 2;
  if constexpr (W) {
    for (int i = 0; i < NB - 1 && tr.lo + i < tr.hi; ++i) issue(tr.lo + i, i);
  } else {
    for (int t = 0; t < (PAIRS ? 2 : NB - 1) && t < ntiles; ++t) issue(t, t);
  }
  wait_vmem();
  __syncthreads();
  constexpr int PER = DirectTile<D, LQ, kBwdWaves>::MIN_PER_WAVE + DirectTile<D, LO, kBwdWaves>::MIN_PER_WAVE;
  int cur = 0;
  if constexpr (W) {
    auto wstep = [&](auto masked, int t) {
      if (t + NB - 1 < tr.hi) issue(t + NB - 1, cur == 0 ? NB - 1 : cur - 1);
      if (active)
        dkdv_tile_any<D, KMASK, decltype(masked)::value>(sq + cur * LQ::ELEMS, so + cur * LO::ELEMS, sl + cur * kTile,
                                                         sd + cur * kTile, kf, vf, dva, dka, kvalid, lane, lo, t * kTile,
                                                         key, a.wl, a.wr);
      if (wave < 2)
        ring_barrier<PER + 1, NB - 2>(tr.hi - 2 - t);
      else
        ring_barrier<PER, NB - 2>(tr.hi - 2 - t);
      cur = cur + 1 == NB ? 0 : cur + 1;
    };
    int t = tr.lo;
    for (; t < tr.flo; ++t) wstep(std::true_type{}, t);
    for (; t < tr.fhi; ++t) wstep(std::false_type{}, t);
    for (; t < tr.hi; ++t) wstep(std::true_type{}, t);
    return;
  }
  if constexpr (PAIRS) {
    for (int t = 0; t < ntiles; t += 2) {
      if (t + 2 < ntiles) issue(t + 2, (t + 2) & 3);
      if (t + 3 < ntiles) issue(t + 3, (t + 3) & 3);
      if (active) {
        const int b0 = t & 3;
        dkdv_tile_any<D, KMASK>(sq + b0 * LQ::ELEMS, so + b0 * LO::ELEMS, sl + b0 * kTile, sd + b0 * kTile, kf,
                                vf, dva, dka, kvalid, lane, lo);
        if (t + 1 < ntiles) {
          const int b1 = b0 + 1;
          dkdv_tile_any<D, KMASK>(sq + b1 * LQ::ELEMS, so + b1 * LO::ELEMS, sl + b1 * kTile, sd + b1 * kTile, kf,
                                  vf, dva, dka, kvalid, lane, lo);
        }
      }
      stream_barrier<0>();  // (also ends the item: the ring is free for the next one)
    }
    return;
  }
  for (int t = 0; t < ntiles; ++t) {
    const bool ahead = t + NB - 1 < ntiles;
    if (ahead) issue(t + NB - 1, cur == 0 ? NB - 1 : cur - 1);
    if (active)
      dkdv_tile_any<D, KMASK>(sq + cur * LQ::ELEMS, so + cur * LO::ELEMS, sl + cur * kTile, sd + cur * kTile, kf,
                              vf, dva, dka, kvalid, lane, lo);
    if (wave < 2)
      ring_barrier<PER + 1, NB - 2>(ntiles - 2 - t);  // (these waves also load a statistics row per tile)
    else
      ring_barrier<PER, NB - 2>(ntiles - 2 - t);
    cur = cur + 1 == NB ? 0 : cur + 1;
  }
}

// One work item of the dk/dv kernel: key rows [128 blk, 128 blk + 128) of (sequence, head) pair bh.
// (Varlen: a block past the end of its sequence takes the all-padding path below, which then writes
// no rows, only its zero partial sums.)
template <int D, bool S, bool V, bool W>
__device__ __forceinline__ void dkdv_item(const BwdArgs& a, char* smem, int bh, int blk, int item) {
  using Dm = Dims<D>;
  // (windowed form: the thread index is made opaque per item, so that the per-lane values derived from
  // it are formed in each item instead of being hoisted out of the item loop and kept, or spilled,
  // through it)
  int tid_ = threadIdx.x;
  if constexpr (W) asm volatile("" : "+v"(tid_));
  const int tid = tid_, lane = tid & 63, wave = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int H = a.H;
  const int b = bh / H, h = bh - b * H;
  const SeqGeom<V> seq(a.cu_seqlens, b, a.L, a.total, a.L);
  const int L = V ? seq.L : a.L;
  const int n = !V && a.valid_len ? min(max(a.valid_len[b], 0), L) : L;
  const RowMap<S> map(V ? (size_t)seq.start : (size_t)b * (S ? a.n0 : L), (size_t)b * (L - a.n0), h, H, D,
                      S ? a.n0 : L);
  const size_t set = (size_t)D * a.items;

  const int key = blk * kBwdRowsPerBlock + wave * kWaveRows + l32;
  const bool kin = key < L;      // row exists
  const bool kvalid = key < n;   // row is an unpadded key
  const size_t roff = map.o0 + (size_t)key * map.rs;  // (joint form)
  // (the joint form addresses its rows by one offset computed here: with pointers formed after the
  // tile loop instead, the compiler schedules the loop's LDS reads one at a time)

  if (blk * kBwdRowsPerBlock >= n) {
    // every key of this workgroup is padding: exact zeros, no dg contribution
    if (kin) {
      uint16_t* dkrow = map.row(a.dk, a.dk1, key);
      uint16_t* dvrow = S ? map.row(a.dv, a.dv1, key) : a.dv + roff;
#pragma unroll
      for (int c = g; c < Dm::NCH; c += 2) {
        *reinterpret_cast<u32x4*>(dkrow + c * 8) = (u32x4){0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(dvrow + c * 8) = (u32x4){0u, 0u, 0u, 0u};
      }
    }
    for (int d = tid; d < D; d += kBwdThreads) {
      if constexpr (S) {
        a.part[set + (size_t)d * a.items + item] = 0.f;
        a.part[3 * set + (size_t)d * a.items + item] = 0.f;
      } else {
        a.part[(size_t)d * a.items + item] = 0.f;
      }
    }
    return;
  }

  // the key's own K gain (two-stream) or both gains (joint form: the streamed Qs rows carry none)
  const float* gk = a.gains + (S ? map.block(key) * 2 * D : 0) + D;
  bf16x8 kf[Dm::KS], vf[Dm::KS], x[Dm::KS];
  load_row_frags_raw<D>(x, S ? map.row(a.k, a.k1, key) : a.k + roff, kvalid, g);
  const float rk =
      rmsnorm_row_frags<D>(kf, x, S ? gk : a.gains, S ? nullptr : a.gains + D, 1.f, a.eps, kvalid, g);
  load_row_frags_raw<D>(vf, S ? map.row(a.v, a.v1, key) : a.v + roff, kvalid, g);
  RowC<D> xk;
  if constexpr (keep_row_c<D, dkdv_waves_per_eu<D>()>()) load_row_c<D>(xk, S ? map.row(a.k, a.k1, key) : a.k + roff, kvalid, g);

  f32x16 dva[Dm::MT], dka[Dm::MT];
#pragma unroll
  for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dva[mt][i] = 0.f;
      dka[mt][i] = 0.f;
    }
  // waves whose 32 keys are all valid skip the key mask
  const bool active = blk * kBwdRowsPerBlock + wave * kWaveRows < n;
  // (local window: the query tiles the block's keys can be seen from; queries past L need no mask,
  // their statistics already give P = 0)
  const TileRange tr = W ? window_tiles(blk * kBwdRowsPerBlock, min(L, (blk + 1) * kBwdRowsPerBlock), a.wr, a.wl, L,
                                        L + 2 * kTile)
                         : TileRange{0, 0, 0, 0};
  if (blk * kBwdRowsPerBlock + (wave + 1) * kWaveRows <= n)
    dkdv_loop<D, S, V, W, false>(a, smem, map, bh, tr, key, kf, vf, dva, dka, kvalid, active, tid);
  else
    dkdv_loop<D, S, V, W, true>(a, smem, map, bh, tr, key, kf, vf, dva, dka, kvalid, active, tid);

  // dv (zeros at padded keys)
  if (kin) {
    uint16_t* dvrow = S ? map.row(a.dv, a.dv1, key) : a.dv + roff;
#pragma unroll
    for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int d0 = mt * 32 + j4 * 8 + g * 4;
        if (d0 < D) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = kvalid ? dva[mt][j4 * 4 + e] : 0.f;
          *reinterpret_cast<u32x2*>(dvrow + d0) = (u32x2){pack2(y[0], y[1]), pack2(y[2], y[3])};
        }
      }
  }
  // dKn = scale * dS^T Qn = ln(2) * dS^T Qs, times g_q in the joint form (the streamed query rows carry
  // scale * log2(e), and in the two-stream form also their own Q gain)
#pragma unroll
  for (int mt = 0; mt < Dm::MT; ++mt) dka[mt] *= kLn2;
  if (kin) {
    if constexpr (!keep_row_c<D, dkdv_waves_per_eu<D>()>()) load_row_c<D>(xk, map.row(a.k, a.k1, key), kvalid, g);
    rmsnorm_backward_row<D, true>(dka, xk, gk, S ? nullptr : a.gains, rk, kvalid, true, S ? map.row(a.dk, a.dk1, key) : a.dk + roff,
                                  nullptr, 0.f, nullptr, g);
  } else {
#pragma unroll
    for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) dka[mt][i] = 0.f;
  }
  __syncthreads();
  if constexpr (S) {
    const int split = min(max(map.n0 - blk * kBwdRowsPerBlock, 0), kBwdRowsPerBlock);
    block_column_sums2<D, kBwdWaves, true>(dka, reinterpret_cast<float*>(smem), a.part + set + item,
                                           a.part + 3 * set + item, (size_t)a.items, split, tid);
  } else {
    block_column_sums<D, kBwdWaves>(dka, reinterpret_cast<float*>(smem), a.part + item, (size_t)a.items, tid);
  }
}

template <int D, bool S, bool V, bool W>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(dkdv_waves_per_eu<D>())))
void bwd_dkdv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[DkdvCfg<D>::template bytes<S>()];
  if constexpr (V) {
    for (PairIter it(a.B * a.H, a.nblk); it.valid(); it.next()) {
      dkdv_item<D, S, V, W>(a, smem, it.pair(), it.blk(), it.pair() * a.nblk + it.blk());
      __syncthreads();  // the column-sum scratch overlaps the ring the next item refills
    }
  } else {
    for (ItemIter it(a.items); it.valid(); it.next()) {
      const int bh = it.item() / a.nblk;
      dkdv_item<D, S, V, W>(a, smem, bh, it.item() - bh * a.nblk, it.item());
      __syncthreads();  // the column-sum scratch overlaps the ring the next item refills
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Gain gradients from the per-workgroup partial sums (stored column-major, part[set][d][item]), each
// summed in a fixed order: block x sums row x of the partials; thread t sums items t, t + 256, ...
// (coalesced) in batches of eight whose loads are all issued before the first add (the kernel is
// latency-bound: a few thousand items take one or two round trips to memory), then the wave sums
// are combined by a fixed butterfly and in wave order.
// Joint form (x = d < D): dgains[0][d] = g_k[d] * T[d] and dgains[1][d] = g_q[d] * T[d] with T the
// total of set 0. Two-stream form (x = set * D + d < 4 D): dgains[x] = the total of row x, i.e.
// dgains[s][0] (Q gain of stream s) from set 2 s and dgains[s][1] from set 2 s + 1.
constexpr int kReduceThreads = 256;

template <bool S>
__global__ __launch_bounds__(kReduceThreads) void dg_reduce_kernel(const float* __restrict__ part,
                                                                   const float* __restrict__ gains, int items,
                                                                   int D, float* __restrict__ dgains) {
  __shared__ float wsum[kReduceThreads / 64];
  const int x = blockIdx.x, t = threadIdx.x;
  const float* p = part + (size_t)x * items;
  constexpr int kBatch = 8;
  float s = 0.f;
  for (int i0 = t; i0 < items; i0 += kBatch * kReduceThreads) {
    float v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = i0 + j * kReduceThreads;
      v[j] = i < items ? p[i] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) s += v[j];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  if ((t & 63) == 0) wsum[t >> 6] = s;
  __syncthreads();
  if (t == 0) {
    float total = 0.f;
#pragma unroll
    for (int w = 0; w < kReduceThreads / 64; ++w) total += wsum[w];
    if constexpr (S) {
      dgains[x] = total;
    } else {
      dgains[x] = gains[D + x] * total;
      dgains[D + x] = gains[x] * total;
    }
  }
}

template <int D, bool S, bool V, bool W>
static hipError_t launch_bwd_d(const BwdArgs& a, bool prenorm, const hipEvent_t* events, int n_events,
                               hipStream_t stream) {
  int stage = 0;
  auto recorded = [&](hipError_t e) {
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess && n_events > stage && events[stage]) e = hipEventRecord(events[stage], stream);
    ++stage;
    return e;
  };
  PrenormArgs p;
  p.k = a.k;
  p.k1 = a.k1;
  p.gains = a.gains;
  p.valid_len = a.valid_len;
  p.cu_seqlens = a.cu_seqlens;
  p.kr = a.kr;
  p.B = a.B;
  p.L = a.L;
  p.H = a.H;
  p.n0 = a.n0;
  p.total = a.total;
  p.eps = a.eps;
  hipError_t e = recorded(prenorm ? launch_prenorm(D, S ? kStreams : (V ? kVarlen : kJoint), p, stream) : hipSuccess);
  if (e != hipSuccess) return e;
  int grid = 0;
  if ((e = persistent_grid(reinterpret_cast<const void*>(bwd_dq_kernel<D, S, V, W>), a.items, kBwdThreads, &grid)) !=
      hipSuccess)
    return e;
  hipLaunchKernelGGL((bwd_dq_kernel<D, S, V, W>), dim3(grid), dim3(kBwdThreads), 0, stream, a);
  if ((e = recorded(hipSuccess)) != hipSuccess) return e;
  if ((e = persistent_grid(reinterpret_cast<const void*>(bwd_dkdv_kernel<D, S, V, W>), a.items, kBwdThreads, &grid)) !=
      hipSuccess)
    return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, S, V, W>), dim3(grid), dim3(kBwdThreads), 0, stream, a);
  if ((e = recorded(hipSuccess)) != hipSuccess) return e;
  hipLaunchKernelGGL(dg_reduce_kernel<S>, dim3(S ? kPartSets * D : D), dim3(kReduceThreads), 0, stream, a.part,
                     a.gains, a.items, D, a.dgains);
  return recorded(hipSuccess);
}

}  // namespace jattn
