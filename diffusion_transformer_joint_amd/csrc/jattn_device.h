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
constexpr int kThreads = 256;  // 4 waves per workgroup (forward and prenorm kernels)
constexpr int kWaveRows = 32;  // rows (queries or keys) owned by one wave
constexpr int kBlockRows = 128;  // rows owned by one workgroup of 4 waves
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
  static constexpr int TPR = NCH >= 8 ? 8 : 4;        // staging threads per row (a power of two)
  static constexpr int CPT = (NCH + TPR - 1) / TPR;   // staging chunks per thread
  static constexpr int RPP = kThreads / TPR;          // rows staged per pass
  static constexpr int PASSES = kTile / RPP;          // passes per tile
  static_assert((TPR & (TPR - 1)) == 0 && kTile % RPP == 0, "staging layout");
};


// ---------------------------------------------------------------------------------------------
// LDS tile layouts (kTile rows of up to DM bf16 columns). Each knows where logical (row, column)
// lives; columns [D, DM) of the padded layouts are zero. Bank model: 64 four-byte banks; a b128
// read is served 16 lanes at a time and a b64 transpose read 32 lanes at a time.
//
// kRowRead  - rows read as 16-byte fragments (lane = row, ds_read_b128). Pitch DM + 8: 16 rows at
//             one column hit 16 different 4-bank groups.
// kTrRead   - rows read by ds_read_b64_tr_b16 (32 lanes = 4 rows x 64 bytes). Pitch chosen so that
//             4 consecutive rows start 16 banks apart: 64 mod 256 bytes or 192 mod 256 bytes.
// kSwizzled - read both ways (D = 64 and 128 only; other head dims fall back to kRowRead). Pitch DM,
//             16-byte chunk c of row r stored at chunk c ^ f(r): f gives 16 consecutive rows distinct
//             (row parity, chunk) bank groups for b128 reads, and 4 consecutive rows disjoint 4-chunk
//             blocks for transpose reads.
enum LayoutKind { kRowRead = 0, kTrRead = 1, kSwizzled = 2 };

template <int D, int KIND>
struct Lay {
  using Dm = Dims<D>;
  static constexpr bool SWZ = KIND == kSwizzled && (D == 64 || D == 128);
  static constexpr int tr_pitch() {
    int p = Dm::DM * 2;  // bytes
    while (p % 256 != 64 && p % 256 != 192) p += 64;
    return p / 2;
  }
  static constexpr int PITCH = SWZ ? Dm::DM : (KIND == kTrRead ? tr_pitch() : Dm::DM + 8);
  static constexpr int ELEMS = kTile * PITCH;
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (!SWZ) return 0;
    else if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    else return ((r & 3) << 2) | ((r >> 2) & 3);
  }
  // element offset of logical (row r, column col); col % 4 == 0
  __device__ static __forceinline__ int off(int r, int col) {
    return r * PITCH + (((col >> 3) ^ swz(r)) << 3) + (col & 7);
  }
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

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

// ---------------------------------------------------------------------------------------------
// LDS fragment reads

// Operand fragment of 8 contiguous bf16 (columns col .. col+7, col % 8 == 0) of one LDS tile row.
template <class LY>
__device__ __forceinline__ bf16x8 lds_row_frag(const __bf16* __restrict__ tile, int r, int col) {
  return *reinterpret_cast<const bf16x8*>(tile + LY::off(r, col));
}

// Transposed operand fragment from an LDS tile T[row][col].
// ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element i%4 of the 8-byte chunk
// addressed by lane 4*t + i/4, for t = 0..3. If lane j of the group addresses T[r0 + j/4][c0 + 4*(j%4)],
// lane i receives T[r0 + t][c0 + i] for t = 0..3: four consecutive rows of one column.
// Lane l of the wave gets column c = col0 + l%32 and rows
//   row0 + 4*(l/32) + [0..3]  (elements 0..3)  and  row0 + 8 + 4*(l/32) + [0..3]  (elements 4..7),
// the contraction-slot order of a C/D tile reused as a B operand (see the file header).
template <class LY>
__device__ __forceinline__ bf16x8 lds_tr_frag(const __bf16* __restrict__ tile, int row0, int col0, int lane) {
  const int r = row0 + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int col = col0 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((JATTN_LDS i16x4*)(tile + LY::off(r, col)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((JATTN_LDS i16x4*)(tile + LY::off(r + 8, col)));
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

// Buffer resource over `nbytes` bytes from `base` (raw buffer, no stride). Loads at byte offsets at or
// past nbytes return zeros, so tile loads need no bounds branches.
constexpr int kBufferWord3 = 0x00020000;  // gfx9 buffer descriptor word 3: 32-bit data, no swizzle
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, kBufferWord3);
}

// Bytes covering rows [0, nrows) of a [rows][D] bf16 view with row stride rs elements.
template <int D>
__device__ __forceinline__ uint32_t rows_bytes(int nrows, int rs) {
  return nrows > 0 ? (uint32_t)((nrows - 1) * rs + D) * 2u : 0u;
}

// Buffer resource for the tile starting at row `row0` of a [rows][D] view (row stride rs elements)
// whose rows [0, nrows) are valid: later rows read as zeros.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int rs, int row0, int nrows) {
  const uint32_t total = rows_bytes<D>(nrows, rs), start = (uint32_t)row0 * (uint32_t)rs * 2u;
  // (the range is wave-uniform; saying so keeps the descriptor in scalar registers, where the
  // buffer instructions need it, instead of a loop over its distinct per-lane values)
  const uint32_t range = __builtin_amdgcn_readfirstlane(total > start ? total - start : 0u);
  return make_rsrc(base + (size_t)row0 * rs, range);
}

// Load rows [row0, row0 + kTile) through a buffer resource that covers the valid rows only; rows
// outside it read as zeros.
template <int D>
__device__ __forceinline__ void tile_load_buf(TileRegs<D>& t, __amdgpu_buffer_rsrc_t rsrc, int rs, int row0,
                                              int tid) {
  using Dm = Dims<D>;
  const int rr = tid / Dm::TPR, cc = tid % Dm::TPR;
#pragma unroll
  for (int p = 0; p < Dm::PASSES; ++p) {
    const uint32_t row = (uint32_t)(row0 + p * Dm::RPP + rr);
#pragma unroll
    for (int j = 0; j < Dm::CPT; ++j) {
      const uint32_t c = (uint32_t)(cc + j * Dm::TPR);
      // chunks past the row (head dims that are not a multiple of 64) read as zeros
      const uint32_t off = c < (uint32_t)Dm::NCH ? (row * (uint32_t)rs + c * 8u) * 2u : 0xFFFFFFF0u;
      t.r[p][j] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
    }
  }
}

// Direct-to-LDS tile loads (buffer_load_dwordx4 ... lds): one wave instruction writes the 16 bytes
// of lane l to LDS at base + 16*l, so the tile's physical 16-byte chunks, taken in LDS order, are
// covered by NWL consecutive wave loads. Each lane precomputes (once) the global offset of the
// logical chunk that belongs at its physical position -- undoing the layout's swizzle -- or an
// out-of-range offset (zeros) for padding positions. Per tile only the buffer resource changes.
// The data bypasses VGPRs; completion is covered by the s_waitcnt vmcnt before the next barrier.
template <int D, class LY, int W = 4>
struct DirectTile {  // W waves share the loads of a tile
  using Dm = Dims<D>;
  static constexpr int HEAD_DIM = D;
  static constexpr int CPR = LY::PITCH / 8;                 // physical chunks per row (incl. padding)
  static constexpr int NWL = (kTile * CPR + 63) / 64;       // wave loads per tile
  static constexpr int PER_WAVE = (NWL + W - 1) / W;        // most loads one wave issues
  static constexpr int MIN_PER_WAVE = NWL / W;              // fewest loads one wave issues
  static constexpr int ALLOC = NWL * 512;                   // elements one tile buffer occupies
  uint32_t voff[PER_WAVE];

  __device__ __forceinline__ void init(int rs, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int p = (wave + W * j) * 64 + lane;  // physical chunk index in the tile
      const int row = p / CPR, pc = p - row * CPR;
      const int lc = pc ^ LY::swz(row & (kTile - 1));
      const bool real = wave + W * j < NWL && row < kTile && pc * 8 < Dm::DM && lc < Dm::NCH;
      voff[j] = real ? (uint32_t)(row * rs + lc * 8) * 2u : 0xFFFFFFF0u;
    }
  }
  // Issue this wave's share of the tile whose first row is addressed by `rsrc`.
  // (The restrict qualifiers here and on the tile readers let the compiler see that reads of the
  // current tile do not depend on the loads in flight into another buffer; without them it waits
  // for every outstanding load before each transposed LDS read.)
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rsrc, __bf16* __restrict__ lds, int wave) const {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int i = wave + W * j;
      if (NWL % W == 0 || i < NWL)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (JATTN_LDS void*)(lds + i * 512), 16, voff[j], 0, 0, 0);
    }
  }
  // Issue a tile whose rows [0, split) come from `r0` (addressed from the tile's first row) and rows
  // [split, kTile) from `r1` (addressed from tile row `split`); 0 < split < kTile. Each lane loads
  // through the resource of its own row, with the other lanes switched off, so a wave may issue up
  // to two loads where `issue` issues one. Lanes of padding positions keep an out-of-range offset
  // under either resource and still write zeros.
  __device__ __forceinline__ void issue_split(__amdgpu_buffer_rsrc_t r0, __amdgpu_buffer_rsrc_t r1, int split,
                                              int rs, __bf16* __restrict__ lds, int wave, int lane) const {
    const uint32_t shift = (uint32_t)split * (uint32_t)rs * 2u;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int i = wave + W * j;
      if (NWL % W == 0 || i < NWL) {
        const int row = (i * 64 + lane) / CPR;
        if (row < split)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r0, (JATTN_LDS void*)(lds + i * 512), 16, voff[j], 0, 0, 0);
        if (row >= split)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r1, (JATTN_LDS void*)(lds + i * 512), 16, voff[j] - shift, 0, 0,
                                                   0);
      }
    }
  }
  // Issue the tile of rows [row0, row0 + kTile) of a tensor stored in two row blocks (see RowMap:
  // rows [0, n0) at p0 + o0, rows [n0, ...) at p1 + o1, row stride rs) whose rows [0, n) are valid
  // (later rows read as zeros). A tile inside one block takes one resource; the (at most one per
  // sequence) tile across the block boundary is split per lane. two = false: block 0 only (callers
  // pass a compile-time constant). n and n0 are wave-uniform.
  // (An ordinary member rather than a member template: the host-side pass of the compiler rejected
  // calls of such a member template from the dk/dv loop.)
  __device__ __forceinline__ void issue_blocks(bool two, const uint16_t* p0, const uint16_t* p1, size_t o0, size_t o1,
                                               int n0, int rs, int row0, int n, __bf16* __restrict__ lds, int wave,
                                               int lane) const {
    if (!two || row0 + kTile <= n0 || n <= n0)  // (no valid row in block 1: it is never addressed)
      issue(tile_rsrc<D>(p0 + o0, rs, row0, two ? min(n, n0) : n), lds, wave);
    else if (row0 >= n0)
      issue(tile_rsrc<D>(p1 + o1, rs, row0 - n0, n - n0), lds, wave);
    else
      issue_split(tile_rsrc<D>(p0 + o0, rs, row0, min(n, n0)), tile_rsrc<D>(p1 + o1, rs, 0, n - n0), n0 - row0, rs,
                  lds, wave, lane);
  }
};

// Direct-to-LDS load of one dword per lane: lane l's word (byte offset voff in rsrc) lands at dst[l].
__device__ __forceinline__ void lds_load_dwords(__amdgpu_buffer_rsrc_t rsrc, float* __restrict__ dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (JATTN_LDS void*)dst, 4, voff, 0, 0, 0);
}


// Addresses of the rows of one (sequence, head) pair of a per-token tensor (token rows of H * D
// elements) stored in two row blocks: rows [0, n0) of the sequence start at token row base0 of
// block 0, rows [n0, ...) at token row base1 of block 1. The joint layout is a single block
// (base0 = b * L, n0 = L); the two-stream layout has base0 = b * N_img, base1 = b * N_txt; a packed
// variable-length batch has base0 = the sequence's first token row. o0 / o1: element offsets of row 0
// in block 0 and of row n0 in block 1. With S = false only block 0 exists and no per-row selection
// is made.
template <bool S>
struct RowMap {
  size_t o0, o1;
  int n0, rs;
  __device__ RowMap(size_t base0, size_t base1, int h, int H, int D, int n_0) {
    n0 = n_0;
    rs = H * D;
    o0 = (base0 * H + h) * D;
    o1 = (base1 * H + h) * D;
  }
  template <class T>
  __device__ __forceinline__ T* row(T* p0, T* p1, int r) const {
    if constexpr (!S) return p0 + o0 + (size_t)r * rs;
    else return r < n0 ? p0 + o0 + (size_t)r * rs : p1 + o1 + (size_t)(r - n0) * rs;
  }
  __device__ __forceinline__ int block(int r) const { return S && r >= n0 ? 1 : 0; }
};

// Geometry of sequence b and the offsets of one of its heads in the library's own arrays.
// Fixed-length batch (V = false): rows [b L, b L + L) of the token tensors. Packed variable-length
// batch (V = true): rows [start, start + L) with start = clamp(cu[b], 0, total) and
// L = clamp(cu[b + 1], start, min(total, start + maxlen)) - start, so that no value of the device
// array can address outside the tensors. In both forms the rows of one (sequence, head) are
// contiguous in the workspaces ([rows, D], from row start * H + h * L) and in the LSE (from element
// start * H + h * L); the fixed form is exactly [B, H, L] there. The row statistics of (sequence,
// head) take lp = L rounded up to 128-row blocks from row (start + 128 b) * H + h * lp (fixed form:
// (b H + h) lp), which leaves room for every sequence's rounding.
template <bool V>
struct SeqGeom {
  int L, start, lp;
  __device__ SeqGeom(const int32_t* cu, int b, int Lfix, int total, int maxlen) {
    if constexpr (V) {
      start = min(max(cu[b], 0), total);
      const int end = min(max(cu[b + 1], start), min(total, start + maxlen));
      L = end - start;
    } else {
      L = Lfix;
      start = b * Lfix;
    }
    lp = (L + 127) / 128 * 128;
  }
  __device__ __forceinline__ size_t row0(int h, int H) const { return (size_t)start * H + (size_t)h * L; }
  __device__ __forceinline__ size_t stat0(int b, int h, int H) const {
    return V ? ((size_t)start + 128 * (size_t)b) * H + (size_t)h * lp : ((size_t)b * H + h) * lp;
  }
};

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Workgroup barrier for the tile-streaming loops: each wave first waits until at most N of its
// vector memory operations are outstanding (they retire in issue order, so every load older than the
// N most recent has landed in LDS) and until its LDS reads have returned, then meets the others.
// __syncthreads() would add a memory-model fence that waits for all outstanding loads, including
// those of tiles further ahead. The asm statement is also a compiler barrier for memory accesses.
template <int N>
__device__ __forceinline__ void stream_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// End-of-step barrier of the tile rings. At the end of step t the tile t + 1 must have landed in LDS;
// the k tiles after it whose loads are already issued (k <= NB - 2) may stay in flight, and each
// wave issued at least PER loads for each of them. k is wave-uniform.
template <int PER, int MAXK>
__device__ __forceinline__ void ring_barrier(int k) {
  static_assert(MAXK >= 0 && MAXK <= 3, "ring depth");
  if constexpr (MAXK >= 3) {
    if (k >= 3) return stream_barrier<3 * PER>();
  }
  if constexpr (MAXK >= 2) {
    if (k >= 2) return stream_barrier<2 * PER>();
  }
  if constexpr (MAXK >= 1) {
    if (k >= 1) return stream_barrier<PER>();
  }
  stream_barrier<0>();
}

// Store the tile unchanged.
template <int D, class LY>
__device__ __forceinline__ void tile_store_raw(const TileRegs<D>& t, __bf16* lds, int tid) {
  using Dm = Dims<D>;
  const int rr = tid / Dm::TPR, cc = tid % Dm::TPR;
#pragma unroll
  for (int p = 0; p < Dm::PASSES; ++p)
#pragma unroll
    for (int j = 0; j < Dm::CPT; ++j) {
      const int c = cc + j * Dm::TPR;
      if (c < Dm::NCH)
        *reinterpret_cast<u32x4*>(lds + LY::off(p * Dm::RPP + rr, c * 8)) = t.r[p][j];
    }
}

// Sum over each aligned group of N lanes (N = 4 or 8) with DPP lane moves: no LDS traffic.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8, "group size");
  // quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2), row_half_mirror (lane i <-> 7-i)
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  if constexpr (N == 8)
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  return x;
}

// Sum of squares of the 8 bf16 values in a 16-byte chunk, accumulated in fp32 with v_dot2c_f32_bf16.
__device__ __forceinline__ float sumsq8(const u32x4& u, float acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = u[j];
    const bf16x2 v = __builtin_bit_cast(bf16x2, w);
    acc = __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
  }
  return acc;
}

// Store the tile with every row RMS-normalised over D and multiplied by `mul`:
// x * rsqrt(mean(x^2) + eps) * mul (gains are applied elsewhere). Rows at or past `nrows`
// (relative row index >= nrows - row0) are written as zeros.
template <int D, class LY>
__device__ __forceinline__ void tile_store_rmsnorm(const TileRegs<D>& t, __bf16* lds, float mul, float eps,
                                                   int row0, int nrows, int tid) {
  using Dm = Dims<D>;
  const int rr = tid / Dm::TPR, cc = tid % Dm::TPR;
#pragma unroll
  for (int p = 0; p < Dm::PASSES; ++p) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < Dm::CPT; ++j) ss = sumsq8(t.r[p][j], ss);
    ss = group_sum<Dm::TPR>(ss);
    const bool valid = row0 + p * Dm::RPP + rr < nrows;
    const float r = valid ? rsqrtf(ss * (1.0f / D) + eps) * mul : 0.f;
#pragma unroll
    for (int j = 0; j < Dm::CPT; ++j) {
      const int c = cc + j * Dm::TPR;
      if (c < Dm::NCH) {
        float x[8];
        unpack8(t.r[p][j], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= r;
        *reinterpret_cast<bf16x8*>(lds + LY::off(p * Dm::RPP + rr, c * 8)) = to_bf16x8(x);
      }
    }
  }
}

// Zero the columns [D, DM) of `ntiles` consecutive LDS tiles of layout LY (only head dims that are
// not a multiple of 32 have them). Staging never writes those columns, so this is done once.
template <int D, class LY>
__device__ __forceinline__ void zero_pad_columns(__bf16* lds, int ntiles, int tid) {
  using Dm = Dims<D>;
  if constexpr (Dm::DM > D) {
    constexpr int W = Dm::DM - D;  // multiple of 8
    for (int idx = tid; idx < ntiles * kTile * (W / 8); idx += kThreads) {
      const int row = idx / (W / 8), c = idx % (W / 8);
      *reinterpret_cast<u32x4*>(lds + (row / kTile) * LY::ELEMS + LY::off(row % kTile, D + c * 8)) =
          (u32x4){0u, 0u, 0u, 0u};
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Wave-row fragments: lane l holds row (row0 + l%32) in the B-operand layout over d,
// i.e. d = 16*ks + 8*(l/32) + [0..7] for each k-step ks.

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

// RMS-normalise a wave row held as in load_row_frags_raw (the other half of the row sits in lane
// l^32) and round x * r * mul * ga[d] * gb[d] to bf16 fragments (gb may be null). Returns r (0 for
// invalid rows). The row stays in its bf16 form and is widened where it is used: widened copies
// made at the load would either be made inside the per-lane load branch, which then waits there for
// its load (one memory round trip per chunk), or hold a second copy of the row in registers.
template <int D>
__device__ __forceinline__ float rmsnorm_row_frags(bf16x8 (&f)[Dims<D>::KS], const bf16x8 (&x)[Dims<D>::KS],
                                                   const float* __restrict__ ga, const float* __restrict__ gb,
                                                   float mul, float eps, bool valid, int g) {
  using Dm = Dims<D>;
  float ss = 0.f;
#pragma unroll
  for (int ks = 0; ks < Dm::KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = (float)x[ks][e];
      ss += v * v;
    }
  ss += __shfl_xor(ss, 32);
  const float r = valid ? rsqrtf(ss * (1.0f / D) + eps) : 0.f;
#pragma unroll
  for (int ks = 0; ks < Dm::KS; ++ks) {
    const int c = 2 * ks + g;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = c * 8 + e;
      y[e] = c < Dm::NCH ? (float)x[ks][e] * r * mul * ga[d] * (gb ? gb[d] : 1.f) : 0.f;
    }
    f[ks] = to_bf16x8(y);
  }
  return r;
}

// ---------------------------------------------------------------------------------------------
// Grid mapping. Workgroups are dispatched round-robin over the 8 XCDs (workgroup i -> XCD i % 8).
__host__ __device__ inline int grid_for_items(int items) { return ((items + 7) >> 3) << 3; }

// Persistent grids: gridDim.x (a multiple of 8) workgroups stay resident and loop over the items.
// Workgroup w serves XCD w % 8, whose items are the contiguous range [x * per, (x + 1) * per) with
// per = ceil(items / 8) -- so the row blocks of one (batch, head) pair share an L2 -- taking every
// (gridDim.x / 8)-th of them. Looping instead of launching one workgroup per item lets the stores of
// one item drain under the next item's work and keeps the workgroups of a CU from running their
// memory-bound prologues and epilogues in lockstep.
struct ItemIter {
  int per, base, j, step, items;
  __device__ explicit ItemIter(int n_items) : items(n_items) {
    per = (n_items + 7) >> 3;
    base = (int)(blockIdx.x & 7) * per;
    j = (int)(blockIdx.x >> 3);
    step = (int)(gridDim.x >> 3);
  }
  __device__ bool valid() const { return j < per && base + j < items; }
  __device__ int item() const { return base + j; }
  __device__ void next() { j += step; }
};

// Streamed tiles a block of rows [r0, r1) reaches under a local window, where row r may see streamed
// rows r - before .. r + after. Streamed rows at or past n_reach are never read; tiles [lo, flo) and
// [fhi, hi) need an element mask, tiles [flo, fhi) are allowed for every (row, streamed row) pair
// and have no streamed row at or past n_full. lo = hi when nothing is reachable. All bounds are
// wave-uniform; the arguments stay far from integer overflow (window bounds are at most L).
struct TileRange {
  int lo, flo, fhi, hi;
};
__device__ __forceinline__ TileRange window_tiles(int r0, int r1, int before, int after, int n_reach, int n_full) {
  TileRange t;
  const int j0 = max(0, r0 - before), j1 = min(n_reach, r1 + after);
  if (j1 <= j0) {
    t.lo = t.flo = t.fhi = t.hi = 0;
    return t;
  }
  t.lo = j0 / kTile;
  t.hi = (j1 + kTile - 1) / kTile;
  const int a = r1 - 1 - before;                        // a full tile starts at or after the last row's first
  const int fl = a > 0 ? (a + kTile - 1) / kTile : 0;   // allowed streamed row ...
  const int b = min(n_full, r0 + after + 1);            // ... and ends at or before the first row's last one
  t.flo = min(max(fl, t.lo), t.hi);
  t.fhi = min(max(b > 0 ? b / kTile : 0, t.flo), t.hi);
  return t;
}

// Item order of the packed variable-length kernels. Sequences differ in length, and the work of a row
// block grows with its sequence's length, so contiguous item ranges per XCD (ItemIter) would give
// one XCD the long sequences and another the short ones. Here the (sequence, head) pairs are dealt
// round-robin over the XCDs (pair p to XCD p % 8): every XCD gets about the same share of every
// sequence, and the nblk row blocks of one pair stay on one XCD and its L2. Workgroup w serves XCD
// w % 8 and takes its items j = w / 8, w / 8 + gridDim.x / 8, ... (one item per workgroup for a grid
// of 8 * ceil(npairs / 8) * nblk).
struct PairIter {
  int x, j, step, per, nblk;
  __device__ PairIter(int npairs, int nblk_) : nblk(nblk_) {
    x = (int)(blockIdx.x & 7);
    j = (int)(blockIdx.x >> 3);
    step = (int)(gridDim.x >> 3);
    per = npairs > x ? ((npairs - x + 7) >> 3) * nblk_ : 0;
  }
  __device__ bool valid() const { return j < per; }
  __device__ int pair() const { return x + 8 * (j / nblk); }
  __device__ int blk() const { return j % nblk; }
  __device__ void next() { j += step; }
};
__host__ __device__ inline int pair_grid(int npairs, int nblk) { return 8 * ((npairs + 7) / 8) * nblk; }

// ---------------------------------------------------------------------------------------------
// Deterministic per-workgroup column sums of a [W waves x 32 rows x D] set of values held in the
// C/D layout of MT tiles (lane = row, register = d). `scr` must hold colsum_scratch_floats<D, W>()
// floats and is only touched after the caller's barrier. Writes the sum of column d to out[d * stride].
// Rows are staged with an odd pitch (DM + 1 floats): the 32 lanes of a wave write 32 different rows
// of one column, which then fall in 32 different banks.
template <int D, int W>
__host__ __device__ constexpr int colsum_scratch_floats() {
  return 32 * W * (Dims<D>::DM + 1) + 8 * Dims<D>::DM;
}

template <int D, int W>
__host__ __device__ constexpr int colsum2_scratch_floats() {
  return 32 * W * (Dims<D>::DM + 1) + 16 * Dims<D>::DM;
}

// As block_column_sums, with the rows split in two groups: rows [0, split) of the block (row index
// 32 * wave + lane % 32) are summed into out0, rows [split, 32 W) into out1 (TWO only; without TWO
// every row goes to out0 and out1 is not touched). Scratch: colsum2_scratch_floats<D, W>() floats.
template <int D, int W, bool TWO>
__device__ __forceinline__ void block_column_sums2(const f32x16 (&v)[Dims<D>::MT], float* scr,
                                                   float* __restrict__ out0, float* __restrict__ out1, size_t stride,
                                                   int split, int tid) {
  using Dm = Dims<D>;
  constexpr int P = Dm::DM + 1, ROWS = 32 * W, THREADS = 64 * W;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  float* rows = scr;             // [ROWS][P]
  float* segs = scr + ROWS * P;  // [TWO + 1][SEGS][DM]
#pragma unroll
  for (int mt = 0; mt < Dm::MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int d = mt * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
      rows[(wave * 32 + l32) * P + d] = v[mt][i];
    }
  __syncthreads();
  constexpr int COLS = Dm::DM <= 32 ? 32 : (Dm::DM <= 64 ? 64 : 128);  // power of two >= DM
  constexpr int SEGS = THREADS / COLS;
  constexpr int RPS = ROWS / SEGS;
  static_assert(SEGS >= 1 && SEGS <= 8 && ROWS % SEGS == 0, "column-sum split");
  {
    const int col = tid % COLS, seg = tid / COLS;
    if (col < Dm::DM) {
      if constexpr (!TWO) {
        float s = 0.f;
#pragma unroll 8
        for (int r = 0; r < RPS; ++r) s += rows[(seg * RPS + r) * P + col];
        segs[seg * Dm::DM + col] = s;
      } else {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll 8
        for (int r = 0; r < RPS; ++r) {
          const float x = rows[(seg * RPS + r) * P + col];
          if (seg * RPS + r < split) s0 += x;
          else s1 += x;
        }
        segs[seg * Dm::DM + col] = s0;
        segs[(SEGS + seg) * Dm::DM + col] = s1;
      }
    }
  }
  __syncthreads();
  for (int d = tid; d < D; d += THREADS) {
    float s = 0.f;
#pragma unroll
    for (int seg = 0; seg < SEGS; ++seg) s += segs[seg * Dm::DM + d];
    out0[d * stride] = s;
    if constexpr (TWO) {
      float t = 0.f;
#pragma unroll
      for (int seg = 0; seg < SEGS; ++seg) t += segs[(SEGS + seg) * Dm::DM + d];
      out1[d * stride] = t;
    }
  }
}

template <int D, int W>
__device__ __forceinline__ void block_column_sums(const f32x16 (&v)[Dims<D>::MT], float* scr,
                                                  float* __restrict__ out, size_t stride, int tid) {
  block_column_sums2<D, W, false>(v, scr, out, nullptr, stride, 32 * W, tid);
}

}  // namespace jattn
