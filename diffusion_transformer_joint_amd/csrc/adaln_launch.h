// Internal interface between the C ABIs (adaln_api.cpp, mlp_api.cpp) and the kernels of the
// adaLN-modulated QKV projection and of the MLP block after the attention (adaln_qkv.hip).
//
// Per token stream s (image = 0, text = 1) with T_s = B * n_s token rows and C channels:
//   x_s    bf16 [T_s, C]         input rows (sample b = row / n_s)
//   mod_s  fp32 [B, 2, C]        per-sample shift (row 0) and scale (row 1)
//   w_s    bf16 [3C, C]          projection weight (torch Linear layout), bias_s fp32 [3C] or null
//   h_s    bf16 [T_s, C]         LN(x) * (1 + scale) + shift, rounded once (forward workspace)
//   stats  fp32 [T_s, 2]         per-row (mean, rstd) of x (forward workspace)
//   q/k/v  bf16 [T_s, C] each    columns [0, C), [C, 2C), [2C, 3C) of h w^T + bias
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace jattn {

constexpr int kGemmWaves = 8;      // waves per GEMM workgroup, 2 x 4 over the output tile
constexpr int kGemmK = 64;         // contraction columns staged per step
constexpr int kBwdRowChunk = 64;   // token rows of one sample per workgroup of the row backward

// A bf16 matrix M[rows][width] in memory whose columns are split into segments of `seg` columns,
// segment i stored at p[i] (row stride rs elements). Rows at or past `rows` read as zeros.
struct MatRef {
  const uint16_t* p[3];
  int seg, rs, rows, width;
};

// One stream's GEMM  out[m][n] = sum_k A[m][k] B[n][k]  (the MFMA's A and B operands), where each
// operand is either stored with k along its memory columns (rows mode: A[m][k] = M[m][k]) or along
// its memory rows (transposed mode: A[m][k] = M[k][m]).
struct GemmProblem {
  MatRef a, b;
  int M, N, K;
  int tiles_m, tiles_n, splits, kchunk;  // kchunk: contraction length of one split (multiple of kGemmK)
  int ntiles;                            // tiles_m * tiles_n * splits
  void* out[3];                          // epilogue targets (see the kernels)
  int out_seg;                           // columns per output tensor
  const float* bias;                     // bf16-output and SwiGLU epilogues (or null)
  float* colsum;                         // weight-gradient kernel: [splits, N] sums of B over k (or null)
  const uint16_t* aux;                   // bf16-output kernel: residual added to the output (or null);
                                         // fp32-output kernel: the forward's [a | g] for the SwiGLU backward
  int pair_off;                          // SwiGLU forward: A tile = rows [j0, j0 + MA/2) and the same rows
                                         // + pair_off (W1 and W3 of W12); 0 elsewhere
};

struct GemmArgs {
  GemmProblem pr[2];
  int ntiles;  // pr[0].ntiles + pr[1].ntiles
};

struct ModulateArgs {
  const uint16_t* x[2];
  const float* mod[2];
  uint16_t* h[2];
  float* stats[2];
  int n[2], T[2];
  int C;
  float eps;
};

struct RowsBwdArgs {
  const uint16_t* x[2];
  const float* mod[2];
  const float* stats[2];
  const float* dh[2];     // [T_s, C] fp32
  uint16_t* dx[2];
  float* part[2];         // [B, chunks_s, 2, C]
  int n[2], chunks[2];    // chunks_s = ceil(n_s / kBwdRowChunk)
  int B, C;
  int blocks0;            // workgroups of stream 0 (B * chunks_0)
};

// Fixed-order sums of per-chunk or per-split partials.
//   modulation: out_s [B, 2, C] = sum over count_s chunks of part_s [B, count_s, 2C]  (len_s = 2BC,
//               inner = 2C)
//   weight:     out_s [3C, C] = sum over count_s splits of part_s [count_s, len_s] (len_s = 3C^2), and
//               cout_s [3C] = sum over the splits of cpart_s [count_s, clen_s] (clen_s = 3C; cout_s
//               may be null)
struct ReduceArgs {
  const float* part[2];
  const float* cpart[2];
  float* out[2];
  float* cout[2];
  int count[2];
  int len[2];
  int inner[2];
  int clen[2];
};

// Up to 6 bf16 matrices src_i [rows_i, cols_i] -> dst_i [cols_i, rows_i] (sizes multiples of 64), one
// 64 x 64 tile per workgroup; start_i = first workgroup of matrix i, start_n = total.
struct TransposeArgs {
  const uint16_t* src[6];
  uint16_t* dst[6];
  int rows[6], cols[6];
  int start[7];
  int n;
};

void launch_modulate(const ModulateArgs& a, hipStream_t stream);
void launch_qkv_gemm(const GemmArgs& a, hipStream_t stream);
void launch_swiglu_gemm(const GemmArgs& a, hipStream_t stream);
void launch_dh_gemm(const GemmArgs& a, hipStream_t stream);
void launch_dhid_gemm(const GemmArgs& a, hipStream_t stream);  // dh GEMM with the SwiGLU-backward epilogue
void launch_dw_gemm(const GemmArgs& a, hipStream_t stream);
void launch_transpose_w(const TransposeArgs& a, hipStream_t stream);
void launch_rows_bwd(const RowsBwdArgs& a, hipStream_t stream);
void launch_mod_reduce(const ReduceArgs& a, hipStream_t stream);
void launch_w_reduce(const ReduceArgs& a, hipStream_t stream);

// Output-tile sizes of the three GEMMs (MFMA-A rows x MFMA-B rows per workgroup).
constexpr int kQkvMA = 256, kQkvMB = 256;
constexpr int kSwigluMA = 256, kSwigluMB = 256;  // 128 columns j of W1 and the same 128 of W3 per tile
constexpr int kDhMA = 256, kDhMB = 256;
constexpr int kDwMA = 256, kDwMB = 256;

}  // namespace jattn
