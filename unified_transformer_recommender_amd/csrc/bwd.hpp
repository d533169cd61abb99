// Argument blocks and launchers of the training-step kernels: the backward pass of the block stack
// with activation recomputation (fun-rec-mdbook 7.5.3, closing paragraph: mixed-precision training
// with activation recomputation; the paper-daily deep reading 4.3, system-efficiency table).
//
// Layout vocabulary.
//   Row views address activations by (sequence b, position t) exactly as in the forward (RowView).
//   Feature-major ("transposed") copies hold, for one weight set, every token's value of feature f
//   in one contiguous run, so that a weight gradient dW = sum_tokens dY^T X is a contraction over
//   contiguous memory: element (group j, token r, feature f) at base + j * g + f * ld + r, where the
//   token index r enumerates the set's rows (S rows: r = b * rows + (t - t0); NS token j: r = b)
//   and ld is a multiple of 64 whose padding columns hold zeros.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace ot {

// Row i of group j of a matrix: base + j * g + (i / rpb) * sb + (i % rpb) * rs (elements).
struct Mat2 {
  const void *base;
  long long g, sb;
  int rpb, rs;
};

// Feature-major copy: element (j, r, f) at base + j * g + f * ld + r (elements).
struct MatT {
  void *base;
  long long g, ld;
};

// ---------------------------------------------------------------------------------------------
// NT contraction on MFMA, grouped: for group j of a job,
//   C(j, r, n) = sum_k A(j, r)[k] * B(j, n)[k],   r < m (token operand), n < n_feat (multiple of 64)
// over k in [0, k_len) (a multiple of 128 bytes), optionally split into n_split contiguous ranges.
// Epilogues:
//   STORE   out(j, r)[n] = C (+ bias[j][n]) (+ resid(j, r)[n]); fp32 or storage dtype; plus outT
//   GELU    out = C + bias (storage dtype, the pre-activation); outT = GELU(C + bias)
//   DGELU   v = C * GELU'(Z(j, r, n)); out = v (storage dtype) and outT = v, where the
//           pre-activation Z = sum_k A2(j, r)[k] * B2(j, n)[k] + bias(j)[n] over k in [0, k_len2) is
//           formed by a first contraction of the same shape into registers (not read from memory)
//           (GELU: the erf form with fp32 storage; with bf16 storage the fitted form the bf16
//           forward evaluates, and its exact derivative)
//   PARTIAL out(j, r)[n] at out.base + split * part_split: the split's fp32 partial sum; with
//           rowsum set, the workgroups of feature tile 0 also write sum_k A(j, r)[k] over their
//           range to rowsum[split * rowsum_split + j * m + r]
// ---------------------------------------------------------------------------------------------
enum GemmEpi { EPI_STORE = 0, EPI_GELU = 1, EPI_DGELU = 2, EPI_PARTIAL = 3 };

struct GemmJob {
  Mat2 a, b;
  int m, n_feat, k_len, n_groups;
  int n_split;
  int tile0, m_tiles, n_tiles;   // tiles = n_split * n_groups * m_tiles * n_tiles
  int epi;
  const void *bias; long long bias_g;   // storage dtype [group][n_feat], or null (DGELU: Z's bias)
  Mat2 resid; int resid_f32;            // STORE: rows added to C (base null: none)
  Mat2 a2, b2; int k_len2;              // DGELU: the pre-activation's operands (no split)
  Mat2 out; int out_f32;                // row-major output (base null: none)
  MatT outT;                            // feature-major output, storage dtype (base null: none)
  long long part_split;                 // PARTIAL: elements between splits
  float *rowsum; long long rowsum_split;
};

constexpr int GEMM_MAX_JOBS = 8;
struct GemmArgs {
  GemmJob job[GEMM_MAX_JOBS];
  int n_jobs;
};

hipError_t launch_gemm(int dtype, const GemmArgs &a, int grid, hipStream_t s);
int gemm_tokens_per_tile();     // rows of the token operand per workgroup
int gemm_features_per_tile();   // rows of the feature operand per workgroup

// Sum of split partials: dst[e] = sum_{s < n_split} src[s * split + e] for e < count (fp32).
constexpr int RED_MAX_JOBS = 16;
struct RedJob {
  const float *src; long long split; int n_split;
  float *dst; long long count;
  long long start;   // first element of this job in the launch's flat index
};
struct RedArgs {
  RedJob job[RED_MAX_JOBS];
  int n_jobs;
  long long total;
};
hipError_t launch_reduce(const RedArgs &a, hipStream_t s);

// Weight copies for the backward products: dst[set][c][dst_off + r] = src[set][r][c] for r < rows,
// c < cols (storage dtype; dst rows are dst_ld elements long).
constexpr int TR_MAX_JOBS = 8;
struct TrJob {
  const void *src; void *dst;
  int rows, cols, sets;
  long long src_set, dst_set;
  int dst_ld, dst_off;
  int tile0;   // first workgroup (32 x 32 tiles, set-major)
};
struct TrArgs {
  TrJob job[TR_MAX_JOBS];
  int n_jobs;
};
hipError_t launch_transpose(int dtype, const TrArgs &a, int grid, hipStream_t s);

// Zero fill of up to FILL_MAX_JOBS strided regions: for row i < rows of group j < groups, elements
// [c0, c1) of base + j * g + i * ld (bytes per element: esz). start: the job's first segment
// (groups * rows segments per job) in the launch; total: segments of the launch.
constexpr int FILL_MAX_JOBS = 32;
struct FillJob {
  void *base; long long g, ld;
  int groups, rows, c0, c1, esz;
  long long start;
};
struct FillArgs {
  FillJob job[FILL_MAX_JOBS];
  int n_jobs;
  long long total;
};
hipError_t launch_fill(const FillArgs &a, hipStream_t s);

// ---------------------------------------------------------------------------------------------
// Row kernels: 32 rows of one row set per workgroup (a wave takes 8 rows, one at a time).
//   NORM_FWD  y = Norm(x) g (+ b): out_t (storage rows) and/or outT
//   NORM_BWD  dx = Norm'(x)^T dy (+ res(b, t) for t >= res_from): out_f32, out_t, outT; per tile
//             column sums of dy * xhat and dy to colpart[tile][2][d]
//   CONVERT   fp32 rows x to out_t and/or outT
//   DOT       D[b][h][t - d_p0] = sum over head h of x * dy (both storage dtype), and outT = x
// ---------------------------------------------------------------------------------------------
enum RowsMode { ROWS_NORM_FWD = 0, ROWS_NORM_BWD = 1, ROWS_CONVERT = 2, ROWS_DOT = 3 };

struct RowsJob {
  RowSet rs;
  int tile0, m_tiles;    // 32-row tiles per group
  long long tr_g, tr_ld; // outT addressing of this job
  void *outT;
};
struct RowsArgs {
  int mode, n_jobs;
  RowsJob job[2];
  int d, layer, n_heads;
  float eps;
  RowView x; int x_f32;
  RowView dy;            // NORM_BWD: fp32; DOT: storage dtype
  RowView res; int res_from;
  const void *gamma, *beta;
  RowView out_f32, out_t;
  float *colpart;
  float *dvec; long long d_sb; int d_R, d_p0;
};
hipError_t launch_rows(int dtype, const RowsArgs &a, int grid, hipStream_t s);

// Column sums of the NORM_BWD partials: dst_g[f] = sum_tiles colpart[tile][0][f], dst_b likewise
// with [1] (dst_b may be null). More than COLSUM_PER tiles are first summed in ranges of that many
// into scratch ([ceil(n_tiles / COLSUM_PER)][2][d] floats).
constexpr int COLSUM_PER = 64;
hipError_t launch_colsum(const float *colpart, int n_tiles, int d, float *dst_g, float *dst_b, float *scratch,
                         hipStream_t s);

// ---------------------------------------------------------------------------------------------
// Attention backward for one block (per head, base 2 as in the forward: queries stored multiplied
// by log2(e) / sqrt(d_head), lse the base-2 log-sum-exp of each query's scores):
//   P = exp2(Qs K^T - lse) over visible keys (key position <= query position)
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),  D = rowsum(dO * O)
//   dQ = dS K / sqrt(d_head),   dK = dS^T Qs / log2(e)
// Queries: q[b][h][i][dh] at positions p0 + i (i < R). Keys/values: k, v [b][h][t][dh] (t < T).
// dO [b][i][d] rows. Outputs: dK, dV, dQ rows of dqkv [b][t][3d] (columns 0, d, 2d), and their
// feature-major copies: position t < s is S token b * s + t, t >= s is NS group t - s token b.
// The dQ copy holds zeros at the S positions before p0 (they issue no query; written with dK).
// ---------------------------------------------------------------------------------------------
struct AttnBwdArgs {
  int n_seq, n_heads, d_model;
  int T, s, R, p0;
  const void *q, *k, *v; long long q_sb, kv_sb;
  const void *dout;      // [b][R][d]
  const float *lse, *dvec;   // [b][h][R]
  void *dqkv;            // [b][T][3d]
  void *tS[3]; long long tS_ld;         // feature-major S parts of dK, dV, dQ
  void *tN[3]; long long tN_g, tN_ld;   // feature-major NS parts
  int n_kblocks, n_qblocks;
};
hipError_t launch_attn_bwd(int dtype, int d_head, const AttnBwdArgs &a, hipStream_t s);
constexpr int ATTB_WAVES = 4;   // waves per attention-backward workgroup (32 keys or queries each)

}  // namespace ot
