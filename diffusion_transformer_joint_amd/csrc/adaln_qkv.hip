// Kernels of the adaLN-modulated QKV projection (gfx950 / CDNA4): the adaLN modulation of the two
// token streams of an MM-DiT layer followed by their per-stream QKV projections, forward and
// backward (re-diffusion README: the DiT-layer box of the architecture flowchart applies adaLN with
// the conditioning vector to each stream and computes Q, K and V per stream before the joint
// attention; the design-notes table gives adaLN as scale + shift without gate).
//
//   h = LN(x) * (1 + scale_b) + shift_b            (LayerNorm over C channels, no affine parameters)
//   [q | k | v] = h W^T + bias                     (W [3C, C]; q, k, v land in the attention's layout)
//
// Forward: one pass over x writes h (bf16, the MFMA operand, also kept for the weight gradient) and
// the row statistics; one GEMM launch covers both streams, with the bias and the q/k/v split in its
// epilogue. Backward: W is transposed once (3C x C, small), dh = dY W runs as the same kind of GEMM
// as the forward, a row kernel applies the LayerNorm backward and sums the modulation gradients
// per chunk of rows, and dW = dY^T h is a split-K GEMM over the tokens; fixed-order reductions
// finish the modulation, weight and bias gradients, so every result is deterministic.
//
// GEMM structure: W waves split the output tile 2 x W/2 (A rows x B rows); both operands stream
// through an LDS ring in 64-wide contraction steps with direct-to-LDS buffer loads (no VGPR
// staging) into 64 x 64 swizzled sub-tiles; v_mfma_f32_32x32x16_bf16 with fp32 accumulators.
// Operands stored with the contraction index along memory rows (the weight gradient's) are read
// with ds_read_b64_tr_b16. The buffer descriptors of a tile's sub-tiles are set up once per tile and
// advanced per step with a pointer add: every scalar instruction of the step sits in the MFMA stream
// (recomputing them per step cost a third of the step at one wave per SIMD).
// Every GEMM runs 256 x 256 output tiles on 8 waves, two per SIMD, each wave 128 x 64 of the tile:
// a SIMD's second wave issues its MFMAs while the first waits on its LDS fragment reads, and the
// larger tile reads each operand fewer times. Measured at C = 3072 against one wave per SIMD on the
// same tile (and, for the projection and SwiGLU forward, 256 x 128 tiles): projection 681 -> 543 us,
// dh 610 -> 513, dW 699 -> 590, SwiGLU forward 1172 -> 933, SwiGLU d(hid) 624 -> 529, on one box.
// (8 waves on 256 x 128 tiles, one 32-row block of tokens per wave, made the SwiGLU forward slower:
// 1339 us.)
#include "adaln_launch.h"
#include "jattn_device.h"

namespace jattn {

using GL = Lay<64, kSwizzled>;     // one 64 x 64 bf16 sub-tile: 128-byte rows, swizzled 16-byte chunks
constexpr int kSub = DirectTile<64, GL, kGemmWaves>::ALLOC;  // elements per sub-tile in the LDS ring

// The sub-tiles of one operand in one output tile, as wave-uniform scalar state: S sub-tiles of 64
// operand rows each (rows mode: memory rows r0 + 64 s, contraction along the memory columns, through
// the column segments of the MatRef; transposed mode: memory columns c0 + 64 s, contraction along the
// memory rows). base[s] addresses the current step's sub-tile, range[s] the bytes from there that
// hold valid rows (later rows, and sub-tiles past the matrix width, read as zeros).
template <int S, bool TR>
struct OpStream {
  const uint16_t* base[S];
  uint32_t range[S];
  // rows mode: the segment and column of the current step
  const uint16_t *p0, *p1, *p2;

  // Segment k's pointer as arithmetic rather than a select: the compiler turns a select between two
  // members into a load at a computed offset, which keeps the whole object in scratch memory.
  __device__ __forceinline__ const uint16_t* seg_ptr(int k) const {
    const uintptr_t u = (uintptr_t)p0 * (uintptr_t)(k == 0) + (uintptr_t)p1 * (uintptr_t)(k == 1) +
                        (uintptr_t)p2 * (uintptr_t)(k == 2);
    return reinterpret_cast<const uint16_t*>(u);
  }
  size_t row_off[S];
  int seg, col, kseg, rs, rows;

  // pair: rows mode only; sub-tiles s >= S/2 start pair rows further (r0 then counts A rows per half)
  __device__ __forceinline__ void init(const MatRef& M, int r0, int k0, int pair = 0) {
    rs = M.rs;
    rows = M.rows;
    if constexpr (!TR) {
      p0 = M.p[0];
      p1 = M.p[1];
      p2 = M.p[2];
      seg = M.seg;
      kseg = k0 / M.seg;  // (once per tile)
      col = k0 - kseg * M.seg;
      const uint16_t* sp = seg_ptr(kseg);
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int row0 = pair ? (s < S / 2 ? r0 + 64 * s : pair + r0 + 64 * (s - S / 2)) : r0 + 64 * s;
        const int valid = M.rows - row0;
        row_off[s] = (size_t)row0 * M.rs;
        range[s] = __builtin_amdgcn_readfirstlane(valid > 0 ? (uint32_t)((valid - 1) * M.rs + 64) * 2u : 0u);
        base[s] = sp + row_off[s] + col;
      }
    } else {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int c0 = r0 + 64 * s;
        const int sg = c0 < M.width ? c0 / M.seg : 0;
        const uint16_t* sp = sg == 0 ? M.p[0] : sg == 1 ? M.p[1] : M.p[2];
        base[s] = sp + (c0 - sg * M.seg) + (size_t)k0 * M.rs;
        const int valid = M.rows - k0;
        range[s] = __builtin_amdgcn_readfirstlane(c0 < M.width && valid > 0 ? (uint32_t)((valid - 1) * M.rs + 64) * 2u
                                                                              : 0u);
      }
    }
  }

  // Move to the next contraction step.
  __device__ __forceinline__ void advance() {
    if constexpr (!TR) {
      col += kGemmK;
      if (col >= seg) {
        col = 0;
        ++kseg;
      }
      const uint16_t* sp = seg_ptr(kseg);
#pragma unroll
      for (int s = 0; s < S; ++s) base[s] = sp + row_off[s] + col;
    } else {
      const uint32_t step = (uint32_t)kGemmK * (uint32_t)rs * 2u;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        base[s] += (size_t)kGemmK * rs;
        range[s] = range[s] > step ? range[s] - step : 0u;
      }
    }
  }

  // (The base is wave-uniform by construction; saying so keeps the descriptor in scalar registers
  // instead of a loop over its per-lane values, which the compiler emits when it cannot prove it.)
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(int s) const {
    const uint64_t u = reinterpret_cast<uint64_t>(base[s]);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    return make_rsrc(reinterpret_cast<const void*>(lo | (hi << 32)), range[s]);
  }
};

// Row-staged epilogue I/O. An MFMA result tile leaves each lane with one token row and runs of 4
// columns; stored straight from there, every instruction writes 8 bytes into 32 different rows, and a
// workgroup's lines stay partly written until its last iteration. With many tiles in flight per XCD
// those lines were evicted half-written (3.7x the HBM writes of the SwiGLU outputs). So a wave
// stages 32 rows x 64 columns (bf16) in LDS, pitch kStgPitch elements, and moves whole 128-byte row
// pieces with 16-byte accesses: lane l takes row 8 it + l / 8, columns 8 (l % 8) .. + 7, 4
// instructions per block. (A wave's 128 columns go through in two such halves: with 8 waves, blocks
// of 32 x 128 would not fit beside each other in the ring.)
constexpr int kStgPitch = 72;              // 64 columns + 8: rows stay 16-byte aligned, 4-bank shift per row
constexpr int kStgElems = 32 * kStgPitch;  // one 32 x 64 block

// Store block `stg` (32 rows x 64 columns) to out + row * rs + col0, rows < nrows, columns < ncols
// (ncols - col0 a multiple of 8 or >= 64).
__device__ __forceinline__ void stg_store_rows(const __bf16* stg, uint16_t* __restrict__ out, size_t rs, int row0,
                                               int nrows, int col0, int ncols, int lane) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = 8 * it + (lane >> 3), c = 8 * (lane & 7);
    if (row0 + r < nrows && col0 + c < ncols)
      *reinterpret_cast<u32x4*>(out + (size_t)(row0 + r) * rs + col0 + c) =
          *reinterpret_cast<const u32x4*>(stg + r * kStgPitch + c);
  }
}

// Load a block the same way (rows >= nrows or columns >= ncols read as zeros), in two parts: the
// global loads into registers, then their LDS writes, so that a caller can issue the loads early.
__device__ __forceinline__ void stg_fetch_rows(u32x4 (&v)[4], const uint16_t* __restrict__ in, size_t rs, int row0,
                                               int nrows, int col0, int ncols, int lane) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = 8 * it + (lane >> 3), c = 8 * (lane & 7);
    v[it] = row0 + r < nrows && col0 + c < ncols ? *reinterpret_cast<const u32x4*>(in + (size_t)(row0 + r) * rs + col0 + c)
                                                   : (u32x4){0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void stg_put_rows(__bf16* stg, const u32x4 (&v)[4], int lane) {
#pragma unroll
  for (int it = 0; it < 4; ++it)
    *reinterpret_cast<u32x4*>(stg + (8 * it + (lane >> 3)) * kStgPitch + 8 * (lane & 7)) = v[it];
}

__device__ __forceinline__ void stg_load_rows(__bf16* stg, const uint16_t* __restrict__ in, size_t rs, int row0,
                                              int nrows, int col0, int ncols, int lane) {
  u32x4 v[4];
  stg_fetch_rows(v, in, rs, row0, nrows, col0, ncols, lane);
  stg_put_rows(stg, v, lane);
}

// sigmoid(x) = 1 / (1 + e^-x) with the hardware exp2 and reciprocal (about 1 ulp each): an IEEE
// division is a dependent chain of several instructions, and the SwiGLU epilogues take hundreds of
// them per wave.
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// Main loop of one output tile: acc[i][j] += sum over k in [kbeg, kend) of A-block i x B-block j,
// where the wave owns A rows wa * MA/2 + 32 i + [0, 32) and B rows wb * MB/WB + 32 j + [0, 32)
// (W waves: 2 along A, WB = W/2 along B).
// TR: operands stored with k along memory rows. NB: LDS stages in the ring.
// (Member functions of a class template rather than function templates: the host-side pass of the
// compiler rejects function templates that reach the LDS-DMA builtin from several kernels.)
template <int MA, int MB, int NB, bool TR, int W>
struct GemmCore {
  using GTW = DirectTile<64, GL, W>;
  static constexpr int WB = W / 2;                      // waves along the B operand
  static constexpr int SA = MA / 64, SB = MB / 64;     // sub-tiles per operand and stage
  static constexpr int STAGE = (SA + SB) * kSub;        // elements per stage
  static constexpr int IA = MA / 64, IB = MB / (32 * WB);  // 32-row MFMA blocks per wave and operand
  static constexpr int PER = (SA + SB) * GTW::PER_WAVE;  // loads each wave issues per stage
  static constexpr int BYTES = NB * STAGE * 2;
  static_assert(GTW::PER_WAVE == GTW::MIN_PER_WAVE, "every wave issues the same number of loads");
  static_assert(NB >= 2 && NB <= 5 && PER * (NB - 2) < 64, "ring depth");

  GTW ta, tb;
  int wa, wb, wave, lane;

  __device__ __forceinline__ GemmCore(const GemmProblem& p) {
    wave = wave_id();
    lane = threadIdx.x & 63;
    wa = wave & 1;
    wb = wave >> 1;
    ta.init(p.a.rs, wave, lane);
    tb.init(p.b.rs, wave, lane);
  }

  // Issue the loads of the step the streams point at.
  __device__ __forceinline__ void issue(const OpStream<SA, TR>& sa, const OpStream<SB, TR>& sb, __bf16* __restrict__ lds) const {
#pragma unroll
    for (int s = 0; s < SA; ++s) ta.issue(sa.rsrc(s), lds + s * kSub, wave);
#pragma unroll
    for (int s = 0; s < SB; ++s) tb.issue(sb.rsrc(s), lds + (SA + s) * kSub, wave);
  }

  // Operand fragment of the 32 rows starting at tile row r (a multiple of 32), k-step ks.
  __device__ __forceinline__ bf16x8 frag(const __bf16* __restrict__ op, int r, int ks) const {
    const __bf16* sub = op + (r >> 6) * kSub;
    if constexpr (TR)
      return lds_tr_frag<GL>(sub, ks * 16, r & 63, lane);
    else
      return lds_row_frag<GL>(sub, (r & 63) + (lane & 31), ks * 16 + 8 * (lane >> 5));
  }

  __device__ __forceinline__ void load(const __bf16* __restrict__ st, int ks, bf16x8 (&fa)[IA], bf16x8 (&fb)[IB]) const {
#pragma unroll
    for (int i = 0; i < IA; ++i) fa[i] = frag(st, wa * (MA / 2) + 32 * i, ks);
#pragma unroll
    for (int j = 0; j < IB; ++j) fb[j] = frag(st + SA * kSub, wb * (MB / WB) + 32 * j, ks);
  }

  // One contraction step (4 k-steps of 16). The fragments of k-step ks + 1 are read before the
  // MFMAs of k-step ks start, into the other register set, so those MFMAs wait only for the older
  // reads: with one wave per SIMD nothing else hides the LDS latency. The scheduling fences keep that
  // order; left alone, the compiler keeps a few fragment registers and waits for each read right
  // before its MFMAs.
  // `before_last` runs after the last k-step's fragments are read and before its MFMAs: the ring
  // barrier goes there, so those MFMAs overlap the next stage's first fragment reads.
  template <class F>
  __device__ __forceinline__ void step(const __bf16* __restrict__ st, f32x16 (&acc)[IA][IB], F before_last) const {
    constexpr int KS = kGemmK / 16;
    bf16x8 fa[2][IA], fb[2][IB];
    load(st, 0, fa[0], fb[0]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = ks & 1;
      if (ks + 1 < KS) load(st, ks + 1, fa[c ^ 1], fb[c ^ 1]);
      else before_last();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < IA; ++i)
#pragma unroll
        for (int j = 0; j < IB; ++j) acc[i][j] = mfma(fa[c][i], fb[c][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// Ring over the contraction steps [kbeg, kend) of one tile; `visit(stage, t)` runs after step t's
// tile has landed and before its MFMAs (the weight-gradient kernel sums its B tiles there).
template <int MA, int MB, int NB, bool TR, int W, class Visit>
__device__ __forceinline__ void gemm_tile(const GemmCore<MA, MB, NB, TR, W>& g, const GemmProblem& p, int m0, int n0,
                                          int kbeg, int kend, __bf16* __restrict__ lds,
                                          f32x16 (&acc)[MA / 64][MB / (16 * W)], Visit& visit) {
  using GC = GemmCore<MA, MB, NB, TR, W>;
#pragma unroll
  for (int i = 0; i < GC::IA; ++i)
#pragma unroll
    for (int j = 0; j < GC::IB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int nk = max(0, (kend - kbeg + kGemmK - 1) / kGemmK);
  OpStream<GC::SA, TR> sa;
  OpStream<GC::SB, TR> sb;
  sa.init(p.a, m0, kbeg, TR ? 0 : p.pair_off);
  sb.init(p.b, n0, kbeg);
#pragma unroll
  for (int t = 0; t < NB - 1; ++t)
    if (t < nk) {
      g.issue(sa, sb, lds + t * GC::STAGE);
      sa.advance();
      sb.advance();
    }
  ring_barrier<GC::PER, NB - 2>(min(NB - 2, nk - 1));
  for (int t = 0; t < nk; ++t) {
    const int ahead = t + NB - 1;
    if (ahead < nk) {
      g.issue(sa, sb, lds + (ahead % NB) * GC::STAGE);
      sa.advance();
      sb.advance();
    }
    const __bf16* st = lds + (t % NB) * GC::STAGE;
    visit(st, t);
    g.step(st, acc, [&]() { ring_barrier<GC::PER, NB - 2>(max(0, min(NB - 2, nk - t - 2))); });
  }
}

// The problem of stream s as a register copy, field by field with constant indices. (Selecting a
// reference to a.pr[s] made the compiler copy the kernel arguments to scratch memory to index them.)
__device__ __forceinline__ MatRef pick(const MatRef& x, const MatRef& y, bool s) {
  MatRef m;
  m.p[0] = s ? y.p[0] : x.p[0];
  m.p[1] = s ? y.p[1] : x.p[1];
  m.p[2] = s ? y.p[2] : x.p[2];
  m.seg = s ? y.seg : x.seg;
  m.rs = s ? y.rs : x.rs;
  m.rows = s ? y.rows : x.rows;
  m.width = s ? y.width : x.width;
  return m;
}

__device__ __forceinline__ GemmProblem pick(const GemmArgs& a, bool s) {
  const GemmProblem &x = a.pr[0], &y = a.pr[1];
  GemmProblem p;
  p.a = pick(x.a, y.a, s);
  p.b = pick(x.b, y.b, s);
  p.M = s ? y.M : x.M;
  p.N = s ? y.N : x.N;
  p.K = s ? y.K : x.K;
  p.tiles_m = s ? y.tiles_m : x.tiles_m;
  p.tiles_n = s ? y.tiles_n : x.tiles_n;
  p.splits = s ? y.splits : x.splits;
  p.kchunk = s ? y.kchunk : x.kchunk;
  p.ntiles = s ? y.ntiles : x.ntiles;
  p.out[0] = s ? y.out[0] : x.out[0];
  p.out[1] = s ? y.out[1] : x.out[1];
  p.out[2] = s ? y.out[2] : x.out[2];
  p.out_seg = s ? y.out_seg : x.out_seg;
  p.bias = s ? y.bias : x.bias;
  p.colsum = s ? y.colsum : x.colsum;
  p.aux = s ? y.aux : x.aux;
  p.pair_off = s ? y.pair_off : x.pair_off;
  return p;
}

// Output tile of workgroup blockIdx.x. Workgroup w runs on XCD w % 8 as that XCD's (w / 8)-th. Each
// problem's tiles are dealt to the XCDs in contiguous ranges, problem by problem, so every XCD gets
// the same share of each stream (with one list for both, the XCDs holding the short text-stream
// tiles idled while the others ran the image stream's). Within a range, tiles go in groups of
// kGroupM A-tiles: consecutive tiles walk the group's A-tiles for one B-tile, then the next B-tile,
// so the ~32 workgroups an XCD runs at once share 4 blocks of A rows and ~8 of B rows in its L2
// (A-tile fastest over all of A re-streamed the forward's weight once per block of tokens). The
// weight-gradient GEMMs take groups of 16 (C = 3072: dW 604 -> 577 us, dW12 991 -> 924, dW2
// 601 -> 576 on one box); for the others 16 measured slower (du 878 -> 979 us) and 8 the same as 4.
constexpr int kGroupM = 4, kGroupMW = 16;  // (kGroupMW: the weight-gradient GEMMs)

struct TileId {
  int s, tm, tn, sp;
  bool ok;
  __device__ explicit TileId(const GemmArgs& a, int group_m = kGroupM) {
    const int x = (int)(blockIdx.x & 7), j = (int)(blockIdx.x >> 3);
    const int nt0 = a.pr[0].ntiles, nt1 = a.pr[1].ntiles;
    const int per0 = (nt0 + 7) >> 3, per1 = (nt1 + 7) >> 3;
    s = j < per0 ? 0 : 1;
    int t = s ? x * per1 + (j - per0) : x * per0 + j;
    ok = s ? (j - per0 < per1 && t < nt1) : t < nt0;
    if (!ok) {
      s = tm = tn = sp = 0;
      return;
    }
    const int tiles_m = s ? a.pr[1].tiles_m : a.pr[0].tiles_m, tiles_n = s ? a.pr[1].tiles_n : a.pr[0].tiles_n;
    const int per_split = tiles_m * tiles_n;
    sp = t / per_split;
    t -= sp * per_split;
    const int group = t / (group_m * tiles_n), first = group * group_m;
    const int gm = min(tiles_m - first, group_m);
    const int r = t - group * group_m * tiles_n;
    tm = first + r % gm;
    tn = r / gm;
  }
};

__host__ __device__ inline int gemm_grid(const GemmArgs& a) {
  return 8 * ((a.pr[0].ntiles + 7) / 8 + (a.pr[1].ntiles + 7) / 8);
}

struct NoVisit {
  __device__ void operator()(const __bf16*, int) {}
};

// ---------------------------------------------------------------------------------------------
// Forward: adaLN modulation. A wave takes MR consecutive token rows (4 for C <= 1024, 2 up to 2048,
// 1 above, where the registers of more rows would halve the waves per SIMD): the loads of all of them are
// issued first, and a sample's shift and scale are loaded again only where the sample changes (one
// row per wave made the launch tens of thousands of short load-reduce-store chains).

template <int U>
constexpr int mod_rows_per_wave() { return U <= 2 ? 4 : U <= 4 ? 2 : 1; }

template <int U>  // 16-byte chunks per lane (C <= 512 U)
__global__ __launch_bounds__(256) void modulate_kernel(ModulateArgs a) {
  constexpr int MR = mod_rows_per_wave<U>();
  const int lane = threadIdx.x & 63;
  const int total = a.T[0] + a.T[1];
  const int row0 = ((int)blockIdx.x * 4 + wave_id()) * MR;
  if (row0 >= total) return;
  const int C = a.C, nch = C >> 3;
  u32x4 v[MR][U];
#pragma unroll
  for (int k = 0; k < MR; ++k) {
    const int row = row0 + k;
    const int s = row >= a.T[0] ? 1 : 0;
    const int r = row - (s ? a.T[0] : 0);
    const uint16_t* x = (s ? a.x[1] : a.x[0]) + (size_t)r * C;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c8 = lane + 64 * u;
      v[k][u] = row < total && c8 < nch ? *reinterpret_cast<const u32x4*>(x + c8 * 8) : (u32x4){0u, 0u, 0u, 0u};
    }
  }
  f32x4 shv4[U][2], scv4[U][2];
  int cur_s = -1, cur_b = -1;
#pragma unroll
  for (int k = 0; k < MR; ++k) {
    const int row = row0 + k;
    if (row >= total) break;
    const int s = row >= a.T[0] ? 1 : 0;
    const int r = row - (s ? a.T[0] : 0);
    const int b = r / (s ? a.n[1] : a.n[0]);
    if (s != cur_s || b != cur_b) {  // (wave-uniform)
      const float* m = (s ? a.mod[1] : a.mod[0]) + (size_t)b * 2 * C;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c8 = lane + 64 * u;
        if (c8 < nch) {
          shv4[u][0] = *reinterpret_cast<const f32x4*>(m + c8 * 8);
          shv4[u][1] = *reinterpret_cast<const f32x4*>(m + c8 * 8 + 4);
          scv4[u][0] = *reinterpret_cast<const f32x4*>(m + C + c8 * 8);
          scv4[u][1] = *reinterpret_cast<const f32x4*>(m + C + c8 * 8 + 4);
        }
      }
      cur_s = s;
      cur_b = b;
    }
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float f[8];
      unpack8(v[k][u], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += f[e];
    }
    const float mean = wave_sum(sum) / (float)C;
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (lane + 64 * u < nch) {
        float f[8];
        unpack8(v[k][u], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += (f[e] - mean) * (f[e] - mean);
      }
    }
    const float rstd = 1.f / sqrtf(wave_sum(ss) / (float)C + a.eps);
    uint16_t* h = (s ? a.h[1] : a.h[0]) + (size_t)r * C;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c8 = lane + 64 * u;
      if (c8 < nch) {
        const f32x4 sh0 = shv4[u][0], sh1 = shv4[u][1], sc0 = scv4[u][0], sc1 = scv4[u][1];
        const float shv[8] = {sh0[0], sh0[1], sh0[2], sh0[3], sh1[0], sh1[1], sh1[2], sh1[3]};
        const float scv[8] = {sc0[0], sc0[1], sc0[2], sc0[3], sc1[0], sc1[1], sc1[2], sc1[3]};
        float f[8], o[8];
        unpack8(v[k][u], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (f[e] - mean) * rstd * (1.f + scv[e]) + shv[e];
        *reinterpret_cast<u32x4*>(h + c8 * 8) =
            (u32x4){pack2(o[0], o[1]), pack2(o[2], o[3]), pack2(o[4], o[5]), pack2(o[6], o[7])};
      }
    }
    if (lane == 0) {
      float* st = (s ? a.stats[1] : a.stats[0]) + 2 * (size_t)r;
      st[0] = mean;
      st[1] = rstd;
    }
  }
}

// Forward GEMM: MFMA-A = W rows (output columns), MFMA-B = h rows (tokens), so each lane ends with
// one token and runs of 4 consecutive output columns, which go out through the row-staged blocks
// into q, k or v (bf16).
template <int MA, int MB, int NB, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(W / 4, W / 4))) void qkv_gemm_kernel(
    GemmArgs a) {
  using GC = GemmCore<MA, MB, NB, false, W>;
  __shared__ __attribute__((aligned(16))) __bf16 smem[GC::BYTES / 2];
  __shared__ __attribute__((aligned(16))) float bias_lds[MA];
  const TileId id(a);
  if (!id.ok) return;
  const GemmProblem p = pick(a, id.s != 0);
  const GC g(p);
  const int m0 = id.tm * MA, n0 = id.tn * MB;
  // The tile's MA bias values go straight to LDS (one dword per lane, wave w the w-th 64), issued
  // before the ring's first loads: each wave's loads complete in order, so the ring's first wait
  // covers them too.
  static_assert(MA <= 64 * 4, "one bias load per wave");
  if (p.bias && g.wave < MA / 64) {
    const int nb = min(MA, p.M - m0);
    lds_load_dwords(make_rsrc(p.bias + m0, (uint32_t)__builtin_amdgcn_readfirstlane(nb * 4)), bias_lds + 64 * g.wave,
                    (uint32_t)(64 * g.wave + g.lane) * 4u);
  }
  f32x16 acc[GC::IA][GC::IB];
  NoVisit none;
  gemm_tile(g, p, m0, n0, 0, p.K, smem, acc, none);
  // Row-staged epilogue, one 32-token x 64-column block at a time: the residual rows (if any) come
  // in through the block, the sums replace them, and whole rows go out. A block never straddles q, k
  // and v (the segment width is a multiple of 64).
  static_assert(GC::IA == 4 && W * kStgElems * 2 <= GC::BYTES, "128 columns and one staged block per wave");
  __bf16* stg = smem + g.wave * kStgElems;  // (the ring's last barrier has passed)
  const int tl = g.lane & 31;
#pragma unroll
  for (int j = 0; j < GC::IB; ++j) {
    const int t0 = n0 + g.wb * (MB / GC::WB) + 32 * j;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int nb = m0 + g.wa * (MA / 2) + 64 * h;  // the block's first output column (wave-uniform)
      if (t0 >= p.N || nb >= p.M) continue;
      const int t = nb >= 2 * p.out_seg ? 2 : nb >= p.out_seg ? 1 : 0, c0 = nb - t * p.out_seg;
      uint16_t* out = static_cast<uint16_t*>(t == 0 ? p.out[0] : t == 1 ? p.out[1] : p.out[2]);
      if (p.aux) {  // the residual (same layout as the output)
        stg_load_rows(stg, p.aux, p.out_seg, t0, p.N, c0, p.out_seg, g.lane);
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are visible to its lanes
      }
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int jl = 32 * ii + 8 * q + 4 * (g.lane >> 5);  // column within the block
          const f32x4 b = p.bias ? *reinterpret_cast<const f32x4*>(bias_lds + g.wa * (MA / 2) + 64 * h + jl)
                                 : (f32x4){0.f, 0.f, 0.f, 0.f};
          u32x2* ps = reinterpret_cast<u32x2*>(stg + tl * kStgPitch + jl);
          float r[4] = {0.f, 0.f, 0.f, 0.f};
          if (p.aux) unpack4(*ps, r);
          const f32x16& v = acc[2 * h + ii][j];
          *ps = (u32x2){pack2(v[4 * q] + b[0] + r[0], v[4 * q + 1] + b[1] + r[1]),
                        pack2(v[4 * q + 2] + b[2] + r[2], v[4 * q + 3] + b[3] + r[3])};
        }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      stg_store_rows(stg, out, p.out_seg, t0, p.N, c0, p.out_seg, g.lane);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // (the next block overwrites this one)
    }
  }
}

// SwiGLU forward of the MLP: [a | g] = u W12^T + b12 and hid = silu(a) * g. The A tile holds 128 rows
// j0.. of W1 (waves wa = 0) and the same 128 rows of W3 (waves wa = 1, pair_off = F rows further),
// so a and g of one (token, j) sit in the same lane and register of the two waves of a pair; the
// wa = 1 waves hand their accumulators over through LDS. Writes [a | g] (bf16 [T, 2F], kept for the
// backward) and hid (bf16 [T, F]).
template <int MA, int MB, int NB, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(W / 4, W / 4))) void swiglu_gemm_kernel(
    GemmArgs a) {
  using GC = GemmCore<MA, MB, NB, false, W>;
  constexpr int H = MA / 2;  // columns j per tile
  static_assert(GC::IA * 16 * 64 * W * 4 <= GC::BYTES, "LDS hand-over fits the ring");
  __shared__ __attribute__((aligned(16))) __bf16 smem[GC::BYTES / 2];
  __shared__ __attribute__((aligned(16))) float bias_lds[MA];  // [b1 of the tile | b3 of the tile]
  const TileId id(a);
  if (!id.ok) return;
  const GemmProblem p = pick(a, id.s != 0);
  const GC g(p);
  const int Fh = p.pair_off, j0 = id.tm * H, n0 = id.tn * MB;
  if (p.bias && g.wave < 4) {  // wave w < 4: 64 bias values, b1 for w < 2, b3 for w >= 2 (before the ring's loads)
    const int jw = j0 + 64 * (g.wave & 1), nb = max(0, min(64, Fh - jw));
    lds_load_dwords(make_rsrc(p.bias + (g.wave < 2 ? 0 : Fh) + jw, (uint32_t)__builtin_amdgcn_readfirstlane(nb * 4)),
                    bias_lds + 64 * g.wave, (uint32_t)g.lane * 4u);
  }
  f32x16 acc[GC::IA][GC::IB];
  NoVisit none;
  gemm_tile(g, p, j0, n0, 0, p.K, smem, acc, none);
  // Hand-over: each wave of a pair (same wb) finishes token block jb = wa of the pair's IB = 2 blocks;
  // it gives its accumulators of the other block to its partner through LDS.
  static_assert(GC::IB == 2 && GC::IA == 4, "two token blocks and 128 columns per wave");
  static_assert(MA == 256 && W == 8, "tile of 128 columns j; 8 waves (the hand-over slots)");
  float* xch = reinterpret_cast<float*>(smem);  // (the ring's last barrier has passed)
  const int give = 1 - g.wa;
#pragma unroll
  for (int i = 0; i < GC::IA; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      xch[(((g.wb * 2 + g.wa) * GC::IA + i) * 16 + e) * 64 + g.lane] = give == 0 ? acc[i][0][e] : acc[i][1][e];
  __syncthreads();
  const int jb = g.wa, partner = 1 - g.wa;  // this wave's token block; the partner's slot in LDS
  float other[GC::IA][16];
#pragma unroll
  for (int i = 0; i < GC::IA; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) other[i][e] = xch[(((g.wb * 2 + partner) * GC::IA + i) * 16 + e) * 64 + g.lane];
  __syncthreads();  // (every hand-over read is done: the LDS now holds the staged output blocks)
  // The wave's 32 tokens x 128 columns of a, g and hid leave through staged blocks, 64 columns at a time.
  constexpr int HALVES = 2, COLS = 64, P = kStgPitch, ELEMS = kStgElems;
  static_assert(W * 3 * ELEMS * 2 <= GC::BYTES, "three staged blocks per wave");
  __bf16* s_a = smem + g.wave * 3 * ELEMS;
  __bf16* s_g = s_a + ELEMS;
  __bf16* s_h = s_g + ELEMS;
  const int t0 = n0 + g.wb * (MB / GC::WB) + 32 * jb;
  uint16_t* ag = static_cast<uint16_t*>(p.out[0]);
  uint16_t* hid = static_cast<uint16_t*>(p.out[1]);
#pragma unroll
  for (int h = 0; h < HALVES; ++h) {
#pragma unroll
    for (int ii = 0; ii < GC::IA / HALVES; ++ii)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = (GC::IA / HALVES) * h + ii;
        const int jl = 32 * i + 8 * q + 4 * (g.lane >> 5), tl = g.lane & 31;  // jl: column within the tile
        const f32x4 b1 = p.bias ? *reinterpret_cast<const f32x4*>(bias_lds + jl) : (f32x4){0.f, 0.f, 0.f, 0.f};
        const f32x4 b3 = p.bias ? *reinterpret_cast<const f32x4*>(bias_lds + H + jl) : (f32x4){0.f, 0.f, 0.f, 0.f};
        float av[4], gv[4], hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // a (W1 rows) is held by the wa = 0 wave, g (W3 rows) by the wa = 1 wave
          const float mine = jb == 0 ? acc[i][0][4 * q + e] : acc[i][1][4 * q + e];
          const float oth = other[i][4 * q + e];
          av[e] = (g.wa == 0 ? mine : oth) + b1[e];
          gv[e] = (g.wa == 0 ? oth : mine) + b3[e];
          hv[e] = av[e] * sigmoid_fast(av[e]) * gv[e];
        }
        const int o = tl * P + jl - COLS * h;
        *reinterpret_cast<u32x2*>(s_a + o) = (u32x2){pack2(av[0], av[1]), pack2(av[2], av[3])};
        *reinterpret_cast<u32x2*>(s_g + o) = (u32x2){pack2(gv[0], gv[1]), pack2(gv[2], gv[3])};
        *reinterpret_cast<u32x2*>(s_h + o) = (u32x2){pack2(hv[0], hv[1]), pack2(hv[2], hv[3])};
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staged blocks are complete
    const int c0 = j0 + COLS * h;
    stg_store_rows(s_a, ag, 2 * (size_t)Fh, t0, p.N, c0, Fh, g.lane);
    stg_store_rows(s_g, ag + Fh, 2 * (size_t)Fh, t0, p.N, c0, Fh, g.lane);
    stg_store_rows(s_h, hid, (size_t)Fh, t0, p.N, c0, Fh, g.lane);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // (the next half's writes overwrite these LDS blocks)
  }
}

// ---------------------------------------------------------------------------------------------
// Backward.

// src_i [R, Cc] -> dst_i [Cc, R] through a padded LDS tile, 64 x 64 elements per workgroup.
__global__ __launch_bounds__(256) void transpose_w_kernel(TransposeArgs a) {
  __shared__ uint16_t t[64][66];
  const int b = (int)blockIdx.x;
  int i = 0;
#pragma unroll
  for (int k = 1; k < 6; ++k) i += (k < a.n && b >= a.start[k]) ? 1 : 0;
  const int R = a.rows[i], Cc = a.cols[i], tiles_c = Cc / 64, id = b - a.start[i];
  const int r0 = (id / tiles_c) * 64, c0 = (id % tiles_c) * 64;
  const uint16_t* src = a.src[i];
  uint16_t* dst = a.dst[i];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) t[r][tx] = src[(size_t)(r0 + r) * Cc + c0 + tx];
  __syncthreads();
  for (int c = ty; c < 64; c += 4) dst[(size_t)(c0 + c) * R + r0 + tx] = t[tx][c];
}

// dh = dY W as MFMA-A = W^T rows (channels), MFMA-B = dY rows (tokens; k runs over the three tensors
// dq, dk, dv): fp32 stores of 4 consecutive channels per lane.
// SWIGLU: the MLP's d(hid) GEMM, whose epilogue applies the SwiGLU backward (p.aux = the forward's [a | g]).
template <int MA, int MB, int NB, bool SWIGLU, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(W / 4, W / 4))) void dh_gemm_kernel(
    GemmArgs a) {
  using GC = GemmCore<MA, MB, NB, false, W>;
  __shared__ __attribute__((aligned(16))) __bf16 smem[GC::BYTES / 2];
  const TileId id(a);
  if (!id.ok) return;
  const GemmProblem p = pick(a, id.s != 0);
  const GC g(p);
  const int m0 = id.tm * MA, n0 = id.tn * MB;
  // SWIGLU: the epilogue's blocks k = 0..3 are (32-token block jb, 64-column half h) = (k / 2, k % 2);
  // the a and g rows of block 0 are loaded before the main loop, and each later block's while the
  // block before it is processed.
  auto blk_t0 = [&](int k) { return n0 + g.wb * (MB / GC::WB) + 32 * (k >> 1); };
  auto blk_j0 = [&](int k) { return m0 + g.wa * (MA / 2) + 64 * (k & 1); };
  u32x4 ra[4], rg[4];
  if constexpr (SWIGLU) {
    stg_fetch_rows(ra, p.aux, 2 * (size_t)p.M, blk_t0(0), p.N, blk_j0(0), p.M, g.lane);
    stg_fetch_rows(rg, p.aux + p.M, 2 * (size_t)p.M, blk_t0(0), p.N, blk_j0(0), p.M, g.lane);
  }
  f32x16 acc[GC::IA][GC::IB];
  NoVisit none;
  gemm_tile(g, p, m0, n0, 0, p.K, smem, acc, none);
  if constexpr (SWIGLU) {  // acc = d(hid)[tok][j]; with the forward's a and g, write [da | dg]
    // Per block of 32 tokens: the a and g rows go through this wave's LDS blocks (coalesced loads),
    // da and dg replace them in place, and whole rows go back out (see the row-staged epilogue I/O),
    // 64 columns at a time.
    constexpr int HALVES = 2, P = kStgPitch, ELEMS = kStgElems;
    static_assert(MA / 2 == 128 && GC::IB == 2 && W * 2 * ELEMS * 2 <= GC::BYTES, "two staged blocks per wave");
    const int Fh = p.M;
    uint16_t* __restrict__ dag = static_cast<uint16_t*>(p.out[0]);
    __bf16* sa = smem + g.wave * 2 * ELEMS;  // (the ring's last barrier has passed)
    __bf16* sg = sa + ELEMS;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int jb = k >> 1, h = k & 1, t0 = blk_t0(k), jw = blk_j0(k);  // jw: the block's first column j
      stg_put_rows(sa, ra, g.lane);
      stg_put_rows(sg, rg, g.lane);
      if (k < 3) {
        stg_fetch_rows(ra, p.aux, 2 * (size_t)Fh, blk_t0(k + 1), p.N, blk_j0(k + 1), Fh, g.lane);
        stg_fetch_rows(rg, p.aux + Fh, 2 * (size_t)Fh, blk_t0(k + 1), p.N, blk_j0(k + 1), Fh, g.lane);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are visible to its lanes
#pragma unroll
      for (int ii = 0; ii < GC::IA / HALVES; ++ii)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = (GC::IA / HALVES) * h + ii;
          const int jl = 32 * ii + 8 * q + 4 * (g.lane >> 5), tl = g.lane & 31;  // jl: column within the block
          u32x2* pa = reinterpret_cast<u32x2*>(sa + tl * P + jl);
          u32x2* pg = reinterpret_cast<u32x2*>(sg + tl * P + jl);
          float av[4], gv[4], da[4], dg[4];
          unpack4(*pa, av);
          unpack4(*pg, gv);
          const f32x16& v = acc[i][jb];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sgm = sigmoid_fast(av[e]);
            da[e] = v[4 * q + e] * gv[e] * sgm * (1.f + av[e] * (1.f - sgm));
            dg[e] = v[4 * q + e] * av[e] * sgm;
          }
          *pa = (u32x2){pack2(da[0], da[1]), pack2(da[2], da[3])};
          *pg = (u32x2){pack2(dg[0], dg[1]), pack2(dg[2], dg[3])};
        }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      stg_store_rows(sa, dag, 2 * (size_t)Fh, t0, p.N, jw, Fh, g.lane);
      stg_store_rows(sg, dag + Fh, 2 * (size_t)Fh, t0, p.N, jw, Fh, g.lane);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // (the next block's loads overwrite these LDS blocks)
    }
    return;
  } else {
    float* dh = static_cast<float*>(p.out[0]);
#pragma unroll
    for (int i = 0; i < GC::IA; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = m0 + g.wa * (MA / 2) + 32 * i + 8 * q + 4 * (g.lane >> 5);
        if (c >= p.M) continue;
#pragma unroll
        for (int j = 0; j < GC::IB; ++j) {
          const int tok = n0 + g.wb * (MB / GC::WB) + 32 * j + (g.lane & 31);
          if (tok < p.N) {
            const f32x16& v = acc[i][j];
            *reinterpret_cast<f32x4*>(dh + (size_t)tok * p.out_seg + c) =
                (f32x4){v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
          }
        }
      }
  }
}

// Column sums of the B tiles (dY over the tokens, for the bias gradient), in the workgroups of
// A-tile 0 only: thread t sums 8 consecutive columns over rows t / (MB/8) + (256 / (MB/8)) * i.
template <int MB, int THREADS>
struct ColSumVisit {
  static constexpr int CH = MB / 8, RG = THREADS / CH;
  float acc[8];  // this thread's 8 column sums
  int sb_off;    // element offset of the B operand inside a stage
  bool on;
  __device__ __forceinline__ void operator()(const __bf16* st, int) {
    if (!on) return;
    const int c8 = (int)threadIdx.x % CH, rg = (int)threadIdx.x / CH;
    const __bf16* sub = st + sb_off + (c8 * 8 / 64) * kSub;
#pragma unroll
    for (int i = 0; i < kGemmK / RG; ++i) {
      const bf16x8 f = lds_row_frag<GL>(sub, rg + RG * i, (c8 * 8) & 63);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += (float)f[e];
    }
  }
};

// dW = dY^T h as split-K over the tokens: MFMA-A = h^T (channels), MFMA-B = dY^T (output columns),
// both read transposed from [64 tokens x 64] sub-tiles. Each split writes its fp32 partial
// [splits, 3C, C] (lane = output column, 4 consecutive channels per store) and, in the workgroups
// of A-tile 0, its partial column sums of dY.
template <int MA, int MB, int NB, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(W / 4, W / 4))) void dw_gemm_kernel(
    GemmArgs a) {
  using GC = GemmCore<MA, MB, NB, true, W>;
  using CS = ColSumVisit<MB, 64 * W>;
  __shared__ __attribute__((aligned(16))) __bf16 smem[GC::BYTES / 2];
  const TileId id(a, kGroupMW);
  if (!id.ok) return;
  const GemmProblem p = pick(a, id.s != 0);
  const GC g(p);
  const int m0 = id.tm * MA, n0 = id.tn * MB;
  const int kbeg = id.sp * p.kchunk, kend = min(p.K, kbeg + p.kchunk);
  f32x16 acc[GC::IA][GC::IB];
  const bool sums = p.colsum != nullptr && id.tm == 0;
  CS cs{{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, GC::SA * kSub, sums};
  gemm_tile(g, p, m0, n0, kbeg, kend, smem, acc, cs);
  float* part = static_cast<float*>(p.out[0]) + (size_t)id.sp * p.N * p.M;
#pragma unroll
  for (int i = 0; i < GC::IA; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = m0 + g.wa * (MA / 2) + 32 * i + 8 * q + 4 * (g.lane >> 5);
      if (c >= p.M) continue;
#pragma unroll
      for (int j = 0; j < GC::IB; ++j) {
        const int n = n0 + g.wb * (MB / GC::WB) + 32 * j + (g.lane & 31);
        if (n < p.N) {
          const f32x16& v = acc[i][j];
          *reinterpret_cast<f32x4*>(part + (size_t)n * p.M + c) = (f32x4){v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
        }
      }
    }
  if (sums) {  // combine the row groups' column sums in LDS (the ring's last barrier has passed)
    float* red = reinterpret_cast<float*>(smem);
    const int c8 = (int)threadIdx.x % CS::CH, rg = (int)threadIdx.x / CS::CH;
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rg * MB + c8 * 8 + e] = cs.acc[e];
    __syncthreads();
    if ((int)threadIdx.x < MB) {
      float t = 0.f;
      for (int r = 0; r < CS::RG; ++r) t += red[r * MB + threadIdx.x];
      const int n = n0 + (int)threadIdx.x;
      if (n < p.N) p.colsum[(size_t)id.sp * p.N + n] = t;
    }
  }
}

// LayerNorm backward and the modulation gradients' partial sums. Workgroup = (stream, sample,
// chunk of kBwdRowChunk rows); wave w takes rows w, w + 4, ...; lane l holds channels 4 l + 256 u.
// With g = dh (1 + scale):  dx = rstd (g - mean(g) - xhat mean(g xhat)),  and the chunk's partial
// sums of dh (shift gradient) and dh xhat (scale gradient) per channel, combined over the 4 waves
// in a fixed order.
template <int U>  // float4 chunks per lane (C <= 256 U)
__global__ __launch_bounds__(256) void rows_bwd_kernel(RowsBwdArgs a) {
  __shared__ float red[2 * 4096];
  const int s = (int)blockIdx.x >= a.blocks0 ? 1 : 0;
  const int blk = (int)blockIdx.x - (s ? a.blocks0 : 0);
  const int chunks = s ? a.chunks[1] : a.chunks[0], n = s ? a.n[1] : a.n[0];
  const int b = blk / chunks, ch = blk - b * chunks;
  const int C = a.C, lane = threadIdx.x & 63, wave = wave_id();
  const int r_lo = ch * kBwdRowChunk, r_hi = min(n, r_lo + kBwdRowChunk);
  const uint16_t* x = s ? a.x[1] : a.x[0];
  const float* dh = s ? a.dh[1] : a.dh[0];
  const float* st = s ? a.stats[1] : a.stats[0];
  uint16_t* dx = s ? a.dx[1] : a.dx[0];
  const float* sc = (s ? a.mod[1] : a.mod[0]) + (size_t)b * 2 * C + C;
  float s1[U][4], acc0[U][4], acc1[U][4];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = 4 * lane + 256 * u;
    const f32x4 v = c < C ? *reinterpret_cast<const f32x4*>(sc + c) : (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s1[u][e] = 1.f + v[e];
      acc0[u][e] = acc1[u][e] = 0.f;
    }
  }
  // A wave takes rounds of RPW rows (r, r + 4, ...). For C <= 1024 the loads of the next round are
  // issued before the current round is computed (two row buffers), so each wave keeps up to 2 RPW
  // rows in flight through its whole chunk instead of waiting for every round's loads.
  constexpr int RPW = U <= 4 ? 2 : 1;
  struct Rows {
    f32x4 dv[RPW][U];
    u32x2 xv[RPW][U];
    f32x2 ms[RPW];
  };
  auto load = [&](Rows& rb, int r0) {
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const int r = r0 + 4 * q;
      if (r < r_hi) {
        const size_t row = (size_t)b * n + r;
        rb.ms[q] = *reinterpret_cast<const f32x2*>(st + 2 * row);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = 4 * lane + 256 * u;
          if (c < C) {
            rb.dv[q][u] = *reinterpret_cast<const f32x4*>(dh + row * C + c);
            rb.xv[q][u] = *reinterpret_cast<const u32x2*>(x + row * C + c);
          }
        }
      }
    }
  };
  // (g and xhat are recomputed for the output rather than kept: registers hold two row buffers, and
  // the kernel is bound by memory, not arithmetic)
  auto compute = [&](const Rows& rb, int r0) {
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const int r = r0 + 4 * q;
      if (r >= r_hi) break;
      const size_t row = (size_t)b * n + r;
      const float mean = rb.ms[q][0], rstd = rb.ms[q][1];
      float sg = 0.f, sgx = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = 4 * lane + 256 * u;
        if (c < C) {
          const f32x4 d = rb.dv[q][u];
          float xf[4];
          unpack4(rb.xv[q][u], xf);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float xh = (xf[e] - mean) * rstd, g = d[e] * s1[u][e];
            sg += g;
            sgx += g * xh;
            acc0[u][e] += d[e];
            acc1[u][e] += d[e] * xh;
          }
        }
      }
      const float mg = wave_sum(sg) / (float)C, mgx = wave_sum(sgx) / (float)C;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = 4 * lane + 256 * u;
        if (c < C) {
          const f32x4 d = rb.dv[q][u];
          float xf[4], o[4];
          unpack4(rb.xv[q][u], xf);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = rstd * (d[e] * s1[u][e] - mg - (xf[e] - mean) * rstd * mgx);
          *reinterpret_cast<u32x2*>(dx + row * C + c) = (u32x2){pack2(o[0], o[1]), pack2(o[2], o[3])};
        }
      }
    }
  };
  constexpr int STEP = 4 * RPW;  // rows between a wave's consecutive rounds
  Rows ra;
  int r0 = r_lo + wave;
  if constexpr (U <= 4) {
    Rows rb;
    if (r0 < r_hi) load(ra, r0);
    for (; r0 < r_hi; r0 += 2 * STEP) {
      if (r0 + STEP < r_hi) load(rb, r0 + STEP);
      compute(ra, r0);
      if (r0 + 2 * STEP < r_hi) load(ra, r0 + 2 * STEP);
      if (r0 + STEP < r_hi) compute(rb, r0 + STEP);
    }
  } else {  // (wider rows: the accumulators leave room for one row buffer only)
    for (; r0 < r_hi; r0 += STEP) {
      load(ra, r0);
      compute(ra, r0);
    }
  }
  // waves add their sums into LDS one after the other (fixed order)
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = 4 * lane + 256 * u;
        if (c < C)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            red[c + e] = (w ? red[c + e] : 0.f) + acc0[u][e];
            red[C + c + e] = (w ? red[C + c + e] : 0.f) + acc1[u][e];
          }
      }
    }
    __syncthreads();
  }
  float* part = (s ? a.part[1] : a.part[0]) + ((size_t)b * chunks + ch) * 2 * C;
  for (int i = threadIdx.x; i < 2 * C; i += 256) part[i] = red[i];
}

// Modulation gradient [B, 2, C] of each stream: the sum over the chunks of [B, chunks, 2, C]
// partials, in chunk order (inner = 2C).
__global__ __launch_bounds__(256) void mod_reduce_kernel(ReduceArgs a) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int s = e >= a.len[0] ? 1 : 0;
  const int64_t i = e - (s ? a.len[0] : 0);
  if (i >= a.len[s ? 1 : 0]) return;
  const int inner = s ? a.inner[1] : a.inner[0], count = s ? a.count[1] : a.count[0];
  const int64_t outer = i / inner, in = i - outer * inner;
  const float* p = (s ? a.part[1] : a.part[0]) + outer * count * inner + in;
  // eight independent loads in flight per round, summed in chunk order
  float t = 0.f;
  int c = 0;
  for (; c + 8 <= count; c += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(c + u) * inner];
#pragma unroll
    for (int u = 0; u < 8; ++u) t += v[u];
  }
  for (; c < count; ++c) t += p[(int64_t)c * inner];
  (s ? a.out[1] : a.out[0])[i] = t;
}

__global__ __launch_bounds__(256) void w_reduce_kernel(ReduceArgs a) {
  const int64_t e4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int64_t l0 = a.len[0], l1 = a.len[1];
  if (e4 < l0 + l1) {
    const int s = e4 >= l0 ? 1 : 0;
    const int64_t i = e4 - (s ? l0 : 0), len = s ? l1 : l0;
    const int count = s ? a.count[1] : a.count[0];
    const float* p = (s ? a.part[1] : a.part[0]) + i;
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < count; ++c) t += *reinterpret_cast<const f32x4*>(p + (int64_t)c * len);
    *reinterpret_cast<f32x4*>((s ? a.out[1] : a.out[0]) + i) = t;
  }
  // bias gradient: the first workgroups also reduce the column sums (clen = 3C per stream)
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t c0 = a.cout[0] ? a.clen[0] : 0, c1 = a.cout[1] ? a.clen[1] : 0;
  if (j < c0 + c1) {
    const int s = j >= c0 ? 1 : 0;
    const int64_t i = j - (s ? c0 : 0), len = s ? c1 : c0;
    const int count = s ? a.count[1] : a.count[0];
    const float* p = (s ? a.cpart[1] : a.cpart[0]) + i;
    float t = 0.f;
    for (int c = 0; c < count; ++c) t += p[(int64_t)c * len];
    (s ? a.cout[1] : a.cout[0])[i] = t;
  }
}

// ---------------------------------------------------------------------------------------------
// Launchers

constexpr int kQkvNB = 2, kSwigluNB = 2, kDhNB = 2, kDwNB = 2;

// (Every launcher returns without a launch when there is no work: a grid of 0 workgroups is an
// invalid launch configuration.)
void launch_modulate(const ModulateArgs& a, hipStream_t stream) {
  const int rows = a.T[0] + a.T[1];
  if (rows == 0) return;
  const dim3 block(256);
  auto grid = [&](int per_wave) { return dim3((rows + 4 * per_wave - 1) / (4 * per_wave)); };
  if (a.C <= 1024)
    hipLaunchKernelGGL(modulate_kernel<2>, grid(mod_rows_per_wave<2>()), block, 0, stream, a);
  else if (a.C <= 2048)
    hipLaunchKernelGGL(modulate_kernel<4>, grid(mod_rows_per_wave<4>()), block, 0, stream, a);
  else
    hipLaunchKernelGGL(modulate_kernel<8>, grid(mod_rows_per_wave<8>()), block, 0, stream, a);
}

void launch_qkv_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.ntiles == 0) return;
  hipLaunchKernelGGL((qkv_gemm_kernel<kQkvMA, kQkvMB, kQkvNB, kGemmWaves>), dim3(gemm_grid(a)), dim3(64 * kGemmWaves), 0,
                     stream, a);
}

void launch_dh_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.ntiles == 0) return;
  hipLaunchKernelGGL((dh_gemm_kernel<kDhMA, kDhMB, kDhNB, false, kGemmWaves>), dim3(gemm_grid(a)), dim3(64 * kGemmWaves), 0, stream,
                     a);
}

void launch_dhid_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.ntiles == 0) return;
  hipLaunchKernelGGL((dh_gemm_kernel<kDhMA, kDhMB, kDhNB, true, kGemmWaves>), dim3(gemm_grid(a)), dim3(64 * kGemmWaves), 0, stream,
                     a);
}

void launch_dw_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.ntiles == 0) return;
  hipLaunchKernelGGL((dw_gemm_kernel<kDwMA, kDwMB, kDwNB, kGemmWaves>), dim3(gemm_grid(a)), dim3(64 * kGemmWaves), 0, stream,
                     a);
}

void launch_transpose_w(const TransposeArgs& a, hipStream_t stream) {
  if (a.n == 0 || a.start[a.n] == 0) return;
  hipLaunchKernelGGL(transpose_w_kernel, dim3(a.start[a.n]), dim3(256), 0, stream, a);
}

void launch_swiglu_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.ntiles == 0) return;
  hipLaunchKernelGGL((swiglu_gemm_kernel<kSwigluMA, kSwigluMB, kSwigluNB, kGemmWaves>), dim3(gemm_grid(a)), dim3(64 * kGemmWaves), 0,
                     stream, a);
}

void launch_rows_bwd(const RowsBwdArgs& a, hipStream_t stream) {
  const dim3 grid(a.blocks0 + a.B * a.chunks[1]), block(256);
  if (grid.x == 0) return;
  if (a.C <= 1024)
    hipLaunchKernelGGL(rows_bwd_kernel<4>, grid, block, 0, stream, a);
  else if (a.C <= 2048)
    hipLaunchKernelGGL(rows_bwd_kernel<8>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(rows_bwd_kernel<16>, grid, block, 0, stream, a);
}

void launch_mod_reduce(const ReduceArgs& a, hipStream_t stream) {
  const int64_t n = (int64_t)a.len[0] + a.len[1];
  if (n == 0) return;
  hipLaunchKernelGGL(mod_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
}

void launch_w_reduce(const ReduceArgs& a, hipStream_t stream) {
  const int64_t n4 = ((int64_t)a.len[0] + a.len[1]) / 4;
  const int64_t nc = (int64_t)(a.cout[0] ? a.clen[0] : 0) + (a.cout[1] ? a.clen[1] : 0);
  const int64_t threads = n4 > nc ? n4 : nc;
  if (threads == 0) return;
  hipLaunchKernelGGL(w_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
}

}  // namespace jattn
