// Device-side building blocks shared by the forward and backward kernels (gfx950 / CDNA4).
//
// MFMA conventions used throughout (v_mfma_f32_32x32x16_bf16, one wave of 64 lanes):
//   A operand: lane l holds row m = l%32 and the 8 contraction values k = 8*(l/32) + [0..7].
//   B operand: lane l holds column n = l%32 and the 8 contraction values k = 8*(l/32) + [0..7].
//   C/D:       lane l, register i holds element (m, n) = (8*(i/4) + 4*(l/32) + i%4, l%32).
// So a product X * Y^T where X and Y are both stored row-major over the contraction index maps
// directly onto the instruction, and the result has the n index on the lane.
//
// A C/D tile can be fed back as the B operand of a second product that contracts over m, with the
// contraction slots permuted: registers i = 0..7 of lane l carry m = 8*(t/4) + 4*(l/32) + t%4 for
// slot t = i, registers 8..15 the same plus 16. The A operand of that second product must use the
// same permutation; ds_read_b64_tr_b16 produces exactly that from a row-major LDS tile (see
// lds_tr_frag), so no LDS round trip or register shuffle is needed between the two products.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define JATTN_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kThreads = 256;  // 4 waves per workgroup
constexpr int kWaveRows = 32;  // rows (queries or keys) owned by one wave
constexpr int kBlockRows = 128;  // rows owned by one workgroup
constexpr int kTile = 64;      // rows of the streamed operand staged per LDS tile

// Head-dim dependent sizes. D is a multiple of 8 (16-byte rows chunks in HBM).
template <int D>
struct Dims {
  static_assert(D % 8 == 0 && D >= 32 && D <= 128, "unsupported head dim");
  static constexpr int NCH = D / 8;                   // 16-byte chunks per row
  static constexpr int DK = (D + 15) / 16 * 16;       // contraction width (k-steps of 16)
  static constexpr int KS = DK / 16;                  // MFMA k-steps over d
  static constexpr int DM = (D + 31) / 32 * 32;       // output width (32-row MFMA tiles over d)
  static constexpr int MT = DM / 32;                  // MFMA tiles over d
  static constexpr int PITCH = DM + 8;                // LDS row pitch in bf16 (16-byte skew)
  static constexpr int TPR = NCH >= 8 ? 8 : NCH;      // staging threads per row
  static constexpr int CPT = (NCH + TPR - 1) / TPR;   // staging chunks per thread
  static constexpr int RPP = kThreads / TPR;          // rows staged per pass
  static constexpr int PASSES = kTile / RPP;          // passes per tile
  static constexpr int TILE_ELEMS = kTile * PITCH;
  static_assert((TPR & (TPR - 1)) == 0 && kTile % RPP == 0, "staging layout");
};

// ---------------------------------------------------------------------------------------------
// MFMA and conversions

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const u32x4& u, float (&f)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = bf_lo(u[j]);
    f[2 * j + 1] = bf_hi(u[j]);
  }
}

__device__ __forceinline__ void unpack4(const u32x2& u, float (&f)[4]) {
  f[0] = bf_lo(u[0]);
  f[1] = bf_hi(u[0]);
  f[2] = bf_lo(u[1]);
  f[3] = bf_hi(u[1]);
}

// Round two floats to bf16 (round to nearest even) and pack them into one dword.
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float* f) {
  const u32x4 u = {pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round 16 probabilities to bf16 (the two B-operand fragments of a 32-row step) and add the rounded
// values to `sum` with v_dot2c_f32_bf16 against (1, 1). The softmax denominator is then the sum of
// exactly the weights the PV product applies, so every output row is a convex combination of the
// value rows (one valid key gives out = v exactly).
// (The packed words go through a plain scalar array: a bit cast applied to an ext-vector element
// subscript selects element 0 for every index.)
__device__ __forceinline__ void pack_probs(const float (&p)[16], bf16x8& f0, bf16x8& f1, float& sum) {
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = pack2(p[2 * j], p[2 * j + 1]);
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t wj = w[j];
    sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wj), one, sum, false);
  }
  const u32x4 a = {w[0], w[1], w[2], w[3]}, b = {w[4], w[5], w[6], w[7]};
  f0 = __builtin_bit_cast(bf16x8, a);
  f1 = __builtin_bit_cast(bf16x8, b);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

// ---------------------------------------------------------------------------------------------
// LDS fragment reads

// B/A operand fragment of 8 contiguous bf16 from a row-major LDS tile.
__device__ __forceinline__ bf16x8 lds_row_frag(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Transposed operand fragment from a row-major LDS tile T[row][col] (pitch in elements).
// ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element i%4 of the 8-byte chunk
// addressed by lane 4*t + i/4, for t = 0..3. If lane j of the group addresses T[r0 + j/4][c0 + 4*(j%4)],
// lane i receives T[r0 + t][c0 + i] for t = 0..3: four consecutive rows of one column.
// Lane l of the wave gets column c = col0 + l%32 and rows
//   row0 + 4*(l/32) + [0..3]  (elements 0..3)  and  row0 + 8 + 4*(l/32) + [0..3]  (elements 4..7),
// the contraction-slot order of a C/D tile reused as a B operand (see the file header).
__device__ __forceinline__ bf16x8 lds_tr_frag(const __bf16* tile, int pitch, int row0, int col0,
                                              int lane) {
  const __bf16* p = tile + (row0 + 4 * (lane >> 5) + ((lane & 15) >> 2)) * pitch + col0 +
                    ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((JATTN_LDS i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((JATTN_LDS i16x4*)(p + 8 * pitch));
  const bf16x4 a = __builtin_bit_cast(bf16x4, lo);
  const bf16x4 b = __builtin_bit_cast(bf16x4, hi);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------------------------------------
// Staging of a kTile-row tile of a [L, H, D] strided bf16 tensor into LDS.
// Thread t covers row p*RPP + t/TPR (pass p) and chunks t%TPR + j*TPR (j < CPT).

template <int D>
struct TileRegs {
  u32x4 r[Dims<D>::PASSES][Dims<D>::CPT];
};

// Load rows [row0, row0 + kTile) of the tensor at `base` (row stride `rs` elements); rows at or past
// `nrows` read as zeros.
template <int D>
__device__ __forceinline__ void tile_load(TileRegs<D>& t, const uint16_t* __restrict__ base, int rs,
                                          int row0, int nrows, int tid) {
  using Dm = Dims<D>;
  const int rr = tid / Dm::TPR, cc = tid % Dm::TPR;
#pragma unroll
  for (int p = 0; p < Dm::PASSES; ++p) {
    const int row = row0 + p * Dm::RPP + rr;
#pragma unroll
    for (int j = 0; j < Dm::CPT; ++j) {
      const int c = cc + j * Dm::TPR;
      if (row < nrows && c < Dm::NCH)
        t.r[p][j] = *reinterpret_cast<const u32x4*>(base + row * rs + c * 8);
      else
        t.r[p][j] = (u32x4){0u, 0u, 0u, 0u};
    }
  }
}

// Store the tile unchanged.
template <int D>
__device__ __forceinline__ void tile_store_raw(const TileRegs<D>& t, __bf16* lds, int tid) {
  using Dm = Dims<D>;
  const int rr = tid / Dm::TPR, cc = tid % Dm::TPR;
#pragma unroll
  for (int p = 0; p < Dm::PASSES; ++p)
#pragma unroll
    for (int j = 0; j < Dm::CPT; ++j) {
      const int c = cc + j * Dm::TPR;
      if (c < Dm::NCH)
        *reinterpret_cast<u32x4*>(lds + (p * Dm::RPP + rr) * Dm::PITCH + c * 8) = t.r[p][j];
    }
}

// Per-thread gain multipliers for the staged chunks: gm[j][e] = mul * gain[(cc + j*TPR)*8 + e].
template <int D>
__device__ __forceinline__ void stage_gains(float (&gm)[Dims<D>::CPT][8], const float* __restrict__ gain,
                                            float mul, int tid) {
  using Dm = Dims<D>;
  const int cc = tid % Dm::TPR;
#pragma unroll
  for (int j = 0; j < Dm::CPT; ++j) {
    const int c = cc + j * Dm::TPR;
#pragma unroll
    for (int e = 0; e < 8; ++e) gm[j][e] = c < Dm::NCH ? mul * gain[c * 8 + e] : 0.f;
  }
}

// Store the tile RMS-normalised over D: x * rsqrt(mean(x^2) + eps) * gm. Rows at or past `nrows`
// (relative row index >= nrows - row0) are written as zeros.
template <int D>
__device__ __forceinline__ void tile_store_rmsnorm(const TileRegs<D>& t, __bf16* lds,
                                                   const float (&gm)[Dims<D>::CPT][8], float eps,
                                                   int row0, int nrows, int tid) {
  using Dm = Dims<D>;
  const int rr = tid / Dm::TPR, cc = tid % Dm::TPR;
#pragma unroll
  for (int p = 0; p < Dm::PASSES; ++p) {
    float x[Dm::CPT][8];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < Dm::CPT; ++j) {
      unpack8(t.r[p][j], x[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[j][e] * x[j][e];
    }
#pragma unroll
    for (int m = 1; m < Dm::TPR; m <<= 1) ss += __shfl_xor(ss, m);
    const bool valid = row0 + p * Dm::RPP + rr < nrows;
    const float r = valid ? rsqrtf(ss * (1.0f / D) + eps) : 0.f;
#pragma unroll
    for (int j = 0; j < Dm::CPT; ++j) {
      const int c = cc + j * Dm::TPR;
      if (c < Dm::NCH) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = x[j][e] * r * gm[j][e];
        *reinterpret_cast<bf16x8*>(lds + (p * Dm::RPP + rr) * Dm::PITCH + c * 8) = to_bf16x8(y);
      }
    }
  }
}

// Zero the columns [D, DM) of `ntiles` LDS tiles (only head dims that are not a multiple of 32
// have them). Staging never writes those columns, so this is done once per kernel.
template <int D>
__device__ __forceinline__ void zero_pad_columns(__bf16* lds, int ntiles, int tid) {
  using Dm = Dims<D>;
  if constexpr (Dm::DM > D) {
    constexpr int W = Dm::DM - D;  // multiple of 8
    for (int idx = tid; idx < ntiles * kTile * (W / 8); idx += kThreads) {
      const int row = idx / (W / 8), c = idx % (W / 8);
      *reinterpret_cast<u32x4*>(lds + row * Dm::PITCH + D + c * 8) = (u32x4){0u, 0u, 0u, 0u};
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Wave-row fragments: lane l holds row (row0 + l%32) in the B-operand layout over d,
// i.e. d = 16*ks + 8*(l/32) + [0..7] for each k-step ks.

template <int D>
__device__ __forceinline__ void load_row_chunks(float (&x)[Dims<D>::KS][8],
                                                const uint16_t* __restrict__ row, bool valid, int g) {
  using Dm = Dims<D>;
#pragma unroll
  for (int ks = 0; ks < Dm::KS; ++ks) {
    const int c = 2 * ks + g;
    if (valid && c < Dm::NCH)
      unpack8(*reinterpret_cast<const u32x4*>(row + c * 8), x[ks]);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) x[ks][e] = 0.f;
  }
}

template <int D>
__device__ __forceinline__ void load_row_frags_raw(bf16x8 (&f)[Dims<D>::KS],
                                                   const uint16_t* __restrict__ row, bool valid, int g) {
  using Dm = Dims<D>;
#pragma unroll
  for (int ks = 0; ks < Dm::KS; ++ks) {
    const int c = 2 * ks + g;
    u32x4 u = {0u, 0u, 0u, 0u};
    if (valid && c < Dm::NCH) u = *reinterpret_cast<const u32x4*>(row + c * 8);
    f[ks] = __builtin_bit_cast(bf16x8, u);
  }
}

// RMS-normalise a wave row held as in load_row_chunks (the other half of the row sits in lane l^32)
// and round x * r * gain * mul to bf16 fragments. Returns r (0 for invalid rows).
template <int D>
__device__ __forceinline__ float rmsnorm_row_frags(bf16x8 (&f)[Dims<D>::KS], const float (&x)[Dims<D>::KS][8],
                                                   const float* __restrict__ gain, float mul, float eps,
                                                   bool valid, int g) {
  using Dm = Dims<D>;
  float ss = 0.f;
#pragma unroll
  for (int ks = 0; ks < Dm::KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[ks][e] * x[ks][e];
  ss += __shfl_xor(ss, 32);
  const float r = valid ? rsqrtf(ss * (1.0f / D) + eps) : 0.f;
#pragma unroll
  for (int ks = 0; ks < Dm::KS; ++ks) {
    const int c = 2 * ks + g;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = c < Dm::NCH ? x[ks][e] * r * (mul * gain[c * 8 + e]) : 0.f;
    f[ks] = to_bf16x8(y);
  }
  return r;
}

// ---------------------------------------------------------------------------------------------
// Grid mapping. Workgroups are dispatched round-robin over the 8 XCDs (workgroup i -> XCD i % 8).
// Work items are numbered so that consecutive items (the row blocks of one (batch, head) pair) land
// on the same XCD, which keeps that pair's streamed operands in one L2.
__device__ __forceinline__ bool map_item(int items, int nblk, int& bh, int& blk, int& item) {
  const int per = (items + 7) >> 3;
  item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (item >= items) return false;
  bh = item / nblk;
  blk = item - bh * nblk;
  return true;
}

__host__ __device__ inline int grid_for_items(int items) { return ((items + 7) >> 3) << 3; }

// ---------------------------------------------------------------------------------------------
// Deterministic per-workgroup column sums of a [4 waves x 32 rows x D] set of values held in the
// C/D layout of MT tiles (lane = row, register = d). `scr` must hold 128*DM + 8*DM floats and is
// only touched after the caller's barrier. Writes the D sums to out[0..D).
template <int D>
__device__ __forceinline__ void block_column_sums(const f32x16 (&v)[Dims<D>::MT], float* scr,
                                                  float* __restrict__ out, int tid) {
  using Dm = Dims<D>;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  float* rows = scr;                        // [128][DM]
  float* segs = scr + kBlockRows * Dm::DM;  // [SEGS][DM]
#pragma unroll
  for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int d = mt * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
      rows[(wave * 32 + l32) * Dm::DM + d] = v[mt][i];
    }
  __syncthreads();
  constexpr int COLS = Dm::DM <= 32 ? 32 : (Dm::DM <= 64 ? 64 : 128);  // power of two >= DM
  constexpr int SEGS = kThreads / COLS;
  constexpr int RPS = kBlockRows / SEGS;
  {
    const int col = tid % COLS, seg = tid / COLS;
    if (col < Dm::DM) {
      float s = 0.f;
#pragma unroll 8
      for (int r = 0; r < RPS; ++r) s += rows[(seg * RPS + r) * Dm::DM + col];
      segs[seg * Dm::DM + col] = s;
    }
  }
  __syncthreads();
  for (int d = tid; d < D; d += kThreads) {
    float s = 0.f;
#pragma unroll
    for (int seg = 0; seg < SEGS; ++seg) s += segs[seg * Dm::DM + d];
    out[d] = s;
  }
}

}  // namespace jattn
