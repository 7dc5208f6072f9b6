// Forward pass of QK-RMSNorm joint attention on gfx950.
//
// Definition (re-diffusion README: architecture flowchart, DiT-layer box -- one multi-head attention
// over the concatenated image and text tokens; design-notes table, "QK norm" row -- RMSNorm on Q and
// K; profiling section -- the attention as an explicit fp32 softmax over the score matrix, which
// this kernel never materialises):
//   out_i = sum_j softmax_j(scale * <Qn_i, Kn_j>) v_j over valid keys j < n_b,  lse_i = log sum_j exp(.)
//
// One workgroup = 4 waves; each wave owns QT = 1 tile of 32 queries (the tile loop is written for
// up to two) and streams all valid keys of the (batch, head) pair in tiles of 64 through a ring of
// LDS buffers (one barrier per tile). Per 32-key half and query tile a wave computes S'^T = Kr Q'^T
// (the result has the query on the lane), turns it into P in registers, and accumulates
// O^T += V^T P^T with V^T read by ds_read_b64_tr_b16 straight from the row-major V tile. Each K and V
// fragment read from LDS feeds QT MFMAs. (Two tiles per wave at 256 rows per workgroup and two waves
// per SIMD measured no faster than one tile at three waves per SIMD; the smaller blocks cut the
// windowed forward's reach by a quarter.)
//
// Both gains go to the query side: Q' = bf16(q * r_q * g_q * g_k * scale * log2(e)) lives in
// registers for the whole loop, and the staged key rows are only normalised, Kr = bf16(k * r_k), so
// S' = Q' Kr^T = scale * log2(e) * Qn Kn^T comes out in log2 units.
//
// Two-stream variant (S): image and text tokens stay in their own tensors (the per-stream QKV of
// the README's DiT-layer box, without the concatenation and split copies) and each stream has its
// own gain pair. Query rows, value tiles and output rows are addressed through a two-block row map;
// the K gain of each key's stream is applied by the prenorm kernel (Kr = bf16(k * r_k * g_k)) and
// the query side carries only its own Q gain.
//
// Softmax shift. QK-RMSNorm bounds every score: ||k_j * r_k|| <= sqrt(D) for any key, so
// |S'_ij| <= B_i = ||Q'_i|| * sqrt(D) (plus a margin for bf16 rounding; two-stream:
// B_i = max_s ||Q'_i * g_k,s|| * sqrt(D) over the two streams' K gains). When every row of the
// workgroup has B_i <= 48 (log2 units), the kernel uses the fixed shift B_i instead of a running
// maximum: the MFMA accumulator starts at -B_i, exp2 of the result lies in [2^-96, 1], and no row
// maximum, rescale or cross-lane exchange is needed inside the loop. Otherwise (large scale or gains)
// it runs the usual online softmax with a running maximum. Both give the same softmax up to rounding.
//
// Streaming: a prenorm kernel first writes Kr = bf16(k * r_k) (per (batch, head), contiguous rows)
// to the workspace. The forward kernel then streams Kr and V tiles straight from memory into a ring
// of LDS buffers with buffer loads that carry the LDS bit, issued NB - 1 tiles ahead. Their range ends
// at the last valid key, so later rows and padding columns land as zeros. No registers or VALU work
// are spent on staging, and the tile body is straight-line code.
#include <type_traits>

#include "jattn_device.h"
#include "jattn_launch.h"

namespace jattn {

constexpr float kBoundLimit = 48.f;

template <int D>
struct Fwd {
  static constexpr int QT = fwd_rows_per_block(D) / kBlockRows;  // 32-query tiles per wave
  static constexpr int ROWS = fwd_rows_per_block(D);
  using LK = Lay<D, kSwizzled>;  // key rows: row fragments (padded rows where D has no swizzle)
  // value rows: read transposed only (swizzled for D = 64, 128, else a pitch for transposed reads)
  using LV = Lay<D, (D == 64 || D == 128) ? kSwizzled : kTrRead>;
  // ring depth: three buffers for rows of up to 64 columns, two for wider rows; the workgroups per CU
  // that fwd_waves_per_eu assumes must fit in the 160 KB of LDS
  static constexpr int BUF = (LK::ELEMS + LV::ELEMS) * 2;  // bytes per ring buffer
  static constexpr int NB = Dims<D>::DM > 64 ? 2 : 3;
  static_assert(NB * BUF + 16 <= 160 * 1024 / fwd_waves_per_eu(D), "ring does not fit the workgroups per CU");
  static constexpr int STAGE = NB * (LK::ELEMS + LV::ELEMS) * 2;  // bytes
  static constexpr int BYTES = STAGE + 16;
  static_assert(QT == 1 || QT == 2, "query tiles per wave");
};

// Per-wave softmax state of QT query tiles.
template <int D>
struct FwdState {
  f32x16 o[Fwd<D>::QT][Dims<D>::MT];  // O^T accumulators (d x queries)
  float lsum[Fwd<D>::QT];             // partial row sums (this lane's half of the keys)
  float mrow[Fwd<D>::QT];             // shift (bounded) or running maximum, log2 units
};

// Softmax of one 32-key half for one query tile (S'^T in registers, lane = query) -> bf16 P
// fragments, with the running-maximum bookkeeping when the fixed shift is not usable.
template <int D, bool BOUNDED>
__device__ __forceinline__ void softmax_half(const f32x16& s, f32x16 (&o)[Dims<D>::MT], float& lsum, float& mrow,
                                             bf16x8& pf0, bf16x8& pf1) {
  using Dm = Dims<D>;
  float p[16];
  if constexpr (BOUNDED) {
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = fast_exp2(s[i]);
  } else {
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
    for (int mt = 0; mt < Dm::MT; ++mt) o[mt] *= alpha;
    mrow = mnew;
  }
  pack_probs(p, pf0, pf1, lsum);
}

// One 64-key tile from LDS (kt, vt). MASKED: keys at or past n get a -inf accumulator seed (p = 0),
// and with a local window (W) so do the keys outside each query's window qrow - wl .. qrow + wr.
template <int D, bool BOUNDED, bool MASKED, bool W = false>
__device__ __forceinline__ void fwd_tile(const __bf16* __restrict__ kt, const __bf16* __restrict__ vt,
                                         const bf16x8 (&qf)[Fwd<D>::QT][Dims<D>::KS],
                                         const f32x16 (&cinit)[Fwd<D>::QT], FwdState<D>& st, int key0, int n,
                                         int lane, const int* qrow = nullptr, int wl = 0, int wr = 0) {
  using Dm = Dims<D>;
  using LK = typename Fwd<D>::LK;
  using LV = typename Fwd<D>::LV;
  constexpr int QT = Fwd<D>::QT;
  const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // S'^T (keys x queries) = Kr Q'^T for this 32-key half and every query tile
    f32x16 s[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      s[qt] = cinit[qt];
      if constexpr (MASKED && W) {
        // keys key0 + c with c = h*32 + (i>>2)*8 + 4g + (i&3) are allowed for c in [clo, chi)
        const int clo = qrow[qt] - wl - key0, chi = min(n, qrow[qt] + wr + 1) - key0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = h * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
          s[qt][i] = ((c >= clo) & (c < chi)) ? s[qt][i] : -INFINITY;
        }
      } else if constexpr (MASKED) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key0 + h * 32 + (i >> 2) * 8 + g * 4 + (i & 3) >= n) s[qt][i] = -INFINITY;
      }
    }
#pragma unroll
    for (int ks = 0; ks < Dm::KS; ++ks) {
      const bf16x8 kf = lds_row_frag<LK>(kt, h * 32 + l32, ks * 16 + g * 8);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[qt] = mfma(kf, qf[qt][ks], s[qt]);
    }
    bf16x8 pf[QT][2];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
      softmax_half<D, BOUNDED>(s[qt], st.o[qt], st.lsum[qt], st.mrow[qt], pf[qt][0], pf[qt][1]);
    // O^T (d x queries) += V^T P^T; each V fragment serves every query tile
#pragma unroll
    for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 vf = lds_tr_frag<LV>(vt, h * 32 + kk * 16, mt * 32, lane);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) st.o[qt][mt] = mfma(vf, pf[qt][kk], st.o[qt][mt]);
      }
  }
}

// The LDS ring of key and value tiles: tile t lives in buffer t % NB. The first NB - 1 tiles are
// issued by the kernel before its prologue; each step issues the tile NB - 1 ahead.
template <int D, bool S>
struct FwdRing {
  using LK = typename Fwd<D>::LK;
  using LV = typename Fwd<D>::LV;
  static constexpr int NB = Fwd<D>::NB;
  static constexpr int PER = DirectTile<D, LK>::MIN_PER_WAVE + DirectTile<D, LV>::MIN_PER_WAVE;
  __bf16* sk;
  __bf16* sv;
  const uint16_t* kb;  // Kr rows of this (batch, head), row stride D
  const uint16_t* v0;  // value rows, two blocks (see RowMap)
  const uint16_t* v1;
  RowMap<S> map;
  int n, ntiles, wave, lane;
  DirectTile<D, LK> dk;
  DirectTile<D, LV> dv;
  __device__ FwdRing(const RowMap<S>& m) : map(m) {}
  __device__ __forceinline__ void issue(int t, int buf) {
    dk.issue(tile_rsrc<D>(kb, D, t * kTile, n), sk + buf * LK::ELEMS, wave);
    dv.issue_blocks(S, v0, v1, map.o0, map.o1, map.n0, map.rs, t * kTile, n, sv + buf * LV::ELEMS, wave, lane);
  }
};

// `active`: this wave has at least one query row inside the sequence (a wave past L only keeps the
// ring going: it issues its share of the loads and meets the barriers, but skips the math).
// (V is not used here; as a template argument it keeps each caller's instantiation its own, which
// the compiler's host-side pass needs for templates that reach the LDS-bound load builtins.)
// W (local window): the ring holds the tiles [tr.lo, tr.hi) only, tile t in buffer (t - tr.lo) % NB;
// the tiles [tr.flo, tr.fhi) run unmasked, the others with the window mask.
template <int D, bool S, bool V, bool W, bool BOUNDED>
__device__ __forceinline__ void fwd_loop(FwdRing<D, S>& ring, const bf16x8 (&qf)[Fwd<D>::QT][Dims<D>::KS],
                                         const float (&shift)[Fwd<D>::QT], FwdState<D>& st, bool active,
                                         int lane, const TileRange& tr, const int* qrow, int wl, int wr) {
  using LK = typename Fwd<D>::LK;
  using LV = typename Fwd<D>::LV;
  constexpr int QT = Fwd<D>::QT, NB = Fwd<D>::NB;
  const int n = ring.n, ntiles = ring.ntiles, nfull = n / kTile;
  f32x16 cinit[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int i = 0; i < 16; ++i) cinit[qt][i] = BOUNDED ? -shift[qt] : 0.f;
  int cur = 0;
  auto step = [&](auto masked, int t) {
    if (t + NB - 1 < ntiles) ring.issue(t + NB - 1, cur == 0 ? NB - 1 : cur - 1);
    if (active)
      fwd_tile<D, BOUNDED, decltype(masked)::value>(ring.sk + cur * LK::ELEMS, ring.sv + cur * LV::ELEMS, qf,
                                                    cinit, st, t * kTile, n, lane);
    ring_barrier<FwdRing<D, S>::PER, NB - 2>(ntiles - 2 - t);
    cur = cur + 1 == NB ? 0 : cur + 1;
  };
  if constexpr (!W) {
    for (int t = 0; t < nfull; ++t) step(std::false_type{}, t);
    if (nfull < ntiles) {
      if constexpr (BOUNDED) {
        // The last tile runs unmasked. Its rows past n arrived as zeros (K and V), so each such key's
        // score is exactly the accumulator seed -shift and its rounded probability p0 = bf16(2^-shift)
        // is the same for every one of them, while its V row adds nothing to O: the row sums only
        // need the masked keys' p0 taken out again. This lane holds the keys 8 k + 4 g + b (k < 8,
        // b < 4) of the tile; those at or past m0 = n - key0 are masked.
        step(std::false_type{}, nfull);
        const int m0 = n - nfull * kTile, g4 = 4 * (lane >> 5);
        int nm = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) nm += min(4, max(0, 8 * k + g4 + 4 - m0));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const float p0 = bf_lo(pack2(fast_exp2(-shift[qt]), 0.f));
          st.lsum[qt] -= (float)nm * p0;
        }
      } else {
        step(std::true_type{}, nfull);
      }
    }
  } else {
    auto wstep = [&](auto masked, int t) {
      if (t + NB - 1 < tr.hi) ring.issue(t + NB - 1, cur == 0 ? NB - 1 : cur - 1);
      if (active)
        fwd_tile<D, BOUNDED, decltype(masked)::value, true>(ring.sk + cur * LK::ELEMS, ring.sv + cur * LV::ELEMS, qf,
                                                            cinit, st, t * kTile, n, lane, qrow, wl, wr);
      ring_barrier<FwdRing<D, S>::PER, NB - 2>(tr.hi - 2 - t);
      cur = cur + 1 == NB ? 0 : cur + 1;
    };
    int t = tr.lo;
    for (; t < tr.flo; ++t) wstep(std::true_type{}, t);
    for (; t < tr.fhi; ++t) wstep(std::false_type{}, t);
    for (; t < tr.hi; ++t) wstep(std::true_type{}, t);
  }
}

// One work item: query rows [ROWS blk, ROWS blk + ROWS) of (sequence, head) pair bh.
// Varlen (V): the grid is sized for the longest sequence; a block past the end of its sequence has
// nothing to do.
template <int D, bool S, bool V, bool W>
__device__ __forceinline__ void fwd_item(const FwdArgs& a, char* smem, int bh, int blk) {
  using Dm = Dims<D>;
  constexpr int QT = Fwd<D>::QT;
  float* sbound = reinterpret_cast<float*>(smem + Fwd<D>::STAGE);
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), g = lane >> 5, l32 = lane & 31;
  const int H = a.H;
  const int b = bh / H, h = bh - b * H;
  const SeqGeom<V> seq(a.cu_seqlens, b, a.L, a.total, a.L);
  const int L = V ? seq.L : a.L;
  if (V && blk * Fwd<D>::ROWS >= L) return;  // (uniform over the workgroup)
  const int n = !V && a.valid_len ? min(max(a.valid_len[b], 0), L) : L;
  const size_t row0 = V ? seq.row0(h, H) : (size_t)bh * L;  // first workspace / LSE row of the pair
  const RowMap<S> map(V ? (size_t)seq.start : (size_t)b * (S ? a.n0 : L), (size_t)b * (L - a.n0), h, H, D,
                      S ? a.n0 : L);

  // start streaming the first key/value tiles before the per-row set-up
  FwdRing<D, S> ring(map);
  ring.sk = reinterpret_cast<__bf16*>(smem);
  ring.sv = ring.sk + Fwd<D>::NB * Fwd<D>::LK::ELEMS;
  ring.kb = a.kr + row0 * D;
  ring.v0 = a.v;
  ring.v1 = a.v1;
  ring.n = n;
  ring.ntiles = (n + kTile - 1) / kTile;
  ring.wave = wave;
  ring.lane = lane;
  ring.dk.init(D, wave, lane);
  ring.dv.init(map.rs, wave, lane);
  // (local window: the key tiles the block's query rows can reach)
  const TileRange tr = W ? window_tiles(blk * Fwd<D>::ROWS, min(L, (blk + 1) * Fwd<D>::ROWS), a.wl, a.wr, n, n)
                         : TileRange{0, 0, 0, 0};
  if constexpr (W) {
    for (int i = 0; i < Fwd<D>::NB - 1 && tr.lo + i < tr.hi; ++i) ring.issue(tr.lo + i, i);
  } else {
    for (int t = 0; t < Fwd<D>::NB - 1 && t < ring.ntiles; ++t) ring.issue(t, t);
  }

  // This wave's query rows, normalised with both gains (two-stream: its own stream's Q gain) and
  // pre-scaled, as B-operand fragments, and their score bounds in log2 units (margin covers the
  // bf16 rounding of Kr and Q').
  int qrow[QT];
  bf16x8 qf[QT][Dm::KS];
  float shift[QT];
  float wmax = 0.f;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    qrow[qt] = blk * Fwd<D>::ROWS + wave * 32 * QT + qt * 32 + l32;
    const bool qvalid = qrow[qt] < L;
    bf16x8 x[Dm::KS];
    load_row_frags_raw<D>(x, map.row(a.q, a.q1, qrow[qt]), qvalid, g);
    float qq = 0.f;
    if constexpr (!S) {
      rmsnorm_row_frags<D>(qf[qt], x, a.gains, a.gains + D, a.c, a.eps, qvalid, g);
#pragma unroll
      for (int ks = 0; ks < Dm::KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float y = (float)qf[qt][ks][e];
          qq += y * y;
        }
      qq += __shfl_xor(qq, 32);
    } else {
      const float* gs = a.gains + map.block(qrow[qt]) * 2 * D;
      rmsnorm_row_frags<D>(qf[qt], x, gs, nullptr, a.c, a.eps, qvalid, g);
      float q0 = 0.f, q1 = 0.f;  // |Q' * g_k|^2 for the K gains of both streams
#pragma unroll
      for (int ks = 0; ks < Dm::KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = (2 * ks + g) * 8 + e;
          if (d < D) {
            const float y = (float)qf[qt][ks][e];
            const float y0 = y * a.gains[D + d], y1 = y * a.gains[3 * D + d];
            q0 += y0 * y0;
            q1 += y1 * y1;
          }
        }
      q0 += __shfl_xor(q0, 32);
      q1 += __shfl_xor(q1, 32);
      qq = fmaxf(q0, q1);
    }
    shift[qt] = sqrtf(qq) * sqrtf((float)D) * (1.f + 1.f / 64.f);
    wmax = fmaxf(wmax, wave_max(shift[qt]));
  }
  if (lane == 0) sbound[wave] = wmax;
  wait_vmem();  // (the first tiles have landed in LDS as well)
  __syncthreads();
  const float bmax = fmaxf(fmaxf(sbound[0], sbound[1]), fmaxf(sbound[2], sbound[3]));

  FwdState<D> st;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.o[qt][mt][i] = 0.f;
    st.lsum[qt] = 0.f;
  }
  const bool active = blk * Fwd<D>::ROWS + wave * 32 * QT < L;  // wave-uniform
  if (bmax <= kBoundLimit) {  // uniform over the workgroup
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) st.mrow[qt] = shift[qt];
    fwd_loop<D, S, V, W, true>(ring, qf, shift, st, active, lane, tr, qrow, a.wl, a.wr);
  } else {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) st.mrow[qt] = -INFINITY;
    fwd_loop<D, S, V, W, false>(ring, qf, shift, st, active, lane, tr, qrow, a.wl, a.wr);
  }
  // (the output addresses are formed after the loop rather than kept from the prologue: at D = 64 the
  // windowed loop has no registers to spare for them)
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) asm volatile("" : "+v"(qrow[qt]));

#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float lsum = st.lsum[qt] + __shfl_xor(st.lsum[qt], 32);
    if (qrow[qt] >= L) continue;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    if (g == 0)
      a.lse[row0 + qrow[qt]] = lsum > 0.f ? (st.mrow[qt] + __log2f(lsum)) * kLn2 : -INFINITY;
    uint16_t* orow = map.row(a.out, a.out1, qrow[qt]);
#pragma unroll
    for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int d0 = mt * 32 + j4 * 8 + g * 4;
        if (d0 < D) {
          const f32x16& o = st.o[qt][mt];
          const u32x2 u = {pack2(o[j4 * 4 + 0] * inv, o[j4 * 4 + 1] * inv),
                           pack2(o[j4 * 4 + 2] * inv, o[j4 * 4 + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d0) = u;
        }
      }
  }
}

template <int D, bool S, bool V, bool W>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(fwd_waves_per_eu(D, W)))) void fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[Fwd<D>::BYTES];
  // one item per workgroup (a persistent grid measured slower here: the items are few and large),
  // numbered so that the row blocks of one (batch, head) pair share an XCD and its L2
  if constexpr (V) {
    const PairIter it(a.B * a.H, a.nblk);
    if (!it.valid()) return;
    fwd_item<D, S, V, W>(a, smem, it.pair(), it.blk());
  } else {
    const ItemIter it(a.items);
    if (!it.valid()) return;
    const int bh = it.item() / a.nblk;
    fwd_item<D, S, V, W>(a, smem, bh, it.item() - bh * a.nblk);
  }
}

template <int D, bool S, bool V, bool W>
static hipError_t launch_fwd_d(const FwdArgs& a, const hipEvent_t* events, int n_events, hipStream_t stream) {
  PrenormArgs p;
  p.k = a.k;
  p.k1 = a.k1;
  p.gains = a.gains;
  p.valid_len = a.valid_len;
  p.cu_seqlens = a.cu_seqlens;
  p.kr = const_cast<uint16_t*>(a.kr);
  p.B = a.B;
  p.L = a.L;
  p.H = a.H;
  p.n0 = a.n0;
  p.total = a.total;
  p.eps = a.eps;
  hipError_t e = launch_prenorm(D, S ? kStreams : (V ? kVarlen : kJoint), p, stream);  // (window: joint)
  if (e == hipSuccess && n_events > 0 && events[0]) e = hipEventRecord(events[0], stream);
  if (e != hipSuccess) return e;
  const int grid = V ? pair_grid(a.B * a.H, a.nblk) : grid_for_items(a.items);
  hipLaunchKernelGGL((fwd_kernel<D, S, V, W>), dim3(grid), dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e == hipSuccess && n_events > 1 && events[1]) e = hipEventRecord(events[1], stream);
  return e;
}

template <bool S, bool V, bool W>
static hipError_t launch_fwd_s(int D, const FwdArgs& a, const hipEvent_t* events, int n_events,
                               hipStream_t stream) {
  switch (D) {
#define JATTN_CASE(DD) \
  case DD: return launch_fwd_d<DD, S, V, W>(a, events, n_events, stream);
    JATTN_FOR_EACH_HEAD_DIM(JATTN_CASE)
#undef JATTN_CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd(int D, Variant var, const FwdArgs& a, const hipEvent_t* events, int n_events,
                      hipStream_t stream) {
  switch (var) {
    case kStreams: return launch_fwd_s<true, false, false>(D, a, events, n_events, stream);
    case kVarlen: return launch_fwd_s<false, true, false>(D, a, events, n_events, stream);
    case kWindow: return launch_fwd_s<false, false, true>(D, a, events, n_events, stream);
    default: return launch_fwd_s<false, false, false>(D, a, events, n_events, stream);
  }
}

}  // namespace jattn
