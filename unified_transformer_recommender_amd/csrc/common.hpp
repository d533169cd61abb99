// Shared device types, MFMA tile traits and kernel argument blocks (gfx950 / CDNA4).
//
// Tile vocabulary used by every kernel: one wave (64 lanes) owns 32x32 fp32 accumulator tiles of
// the MFMA 32x32 family. Lane l holds column (l % 32) of a tile and rows
//     8 * (v / 4) + 4 * (l / 32) + (v % 4),   v = 0..15
// of it. A-operand fragments hold row (l % 32) and B-operand fragments column (l % 32); both hold
// the k elements [KPL * (l / 32), KPL * (l / 32) + KPL) of the instruction's k-chunk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ot {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// ---------------------------------------------------------------------------------------------
// MFMA traits: 32x32 output tile, k-chunk of KSTEP per instruction, KPL k elements per lane.
// ---------------------------------------------------------------------------------------------
template <typename T> struct Mma;

template <> struct Mma<bf16> {
  static constexpr int KPL = 8;
  static constexpr int KSTEP = 16;
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag zero() { return frag{}; }
};

template <> struct Mma<float> {
  static constexpr int KPL = 1;
  static constexpr int KSTEP = 2;
  typedef float frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag zero() { return 0.0f; }
};

// Row of the accumulator element v held by a lane in lane-group g (= lane / 32).
__device__ __forceinline__ constexpr int acc_row(int v, int g) { return 8 * (v >> 2) + 4 * g + (v & 3); }

// ---------------------------------------------------------------------------------------------
// conversions
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// 16-byte vector load / store (both pointers 16-byte aligned).
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

// ---------------------------------------------------------------------------------------------
// Row sets. A row set enumerates (sequence b, position t, parameter group) triples:
//   group j in [0, n_groups); row r in [0, n_seq * rows):
//     b = r / rows,  t = t0 + j * t_step + r % rows,  parameter set = wg0 + j
// S rows of a block: n_groups = 1, rows = count, t_step = 0, wg0 = 0.
// NS rows of a block: n_groups = l_ns, rows = 1, t0 = s, t_step = 1, wg0 = 1.
// ---------------------------------------------------------------------------------------------
struct RowSet {
  int n_seq, rows, n_groups, t0, t_step, wg0;
};

// Strided view of a row-major activation buffer addressed by (b, t):
//   element (b, t, c) at base + b * sb + (t - t_off) * rs + c
struct RowView {
  void *base;
  long long sb;
  int t_off;
  int rs;
};

// Head-split view: element (b, t, col) with h = col / d_head, c = col % d_head at
//   base + b * sb + h * sh + (t - t_off) * d_head + c
struct HeadView {
  void *base;
  long long sb, sh;
  int t_off;
};

// ---------------------------------------------------------------------------------------------
// Fused pre-norm 1 + mixed Q/K/V launch over the rows of a block: job 0 = S rows (parameter set
// 0), job 1 = NS rows (sets 1..l_ns). K and V are produced for every row, Q for rows at
// positions >= q_from.
// ---------------------------------------------------------------------------------------------
struct QkvJob {
  RowSet rs;
  int tile_start;          // first workgroup of this job
  int m_tiles;             // token tiles per group
  int q_from;              // first position that issues a query
  HeadView k, v, q;        // head-split outputs
};

struct QkvArgs {
  int n_jobs;
  QkvJob job[2];
  int d_model, d_head;
  RowView x;               // block input rows (storage dtype in block 0, else fp32)
  const void *wq, *wk, *wv;   // [G][d][d] storage dtype
  const void *gamma, *beta;   // norm1 [d]
  int layer;
  float eps;
};

// ---------------------------------------------------------------------------------------------
// Fused post-attention launch (W^O + residual + norm2 + mixed FFN + residual) over the query rows
// of a block: job 0 = tail S rows (parameter set 0), job 1 = NS rows (sets 1..l_ns).
// ---------------------------------------------------------------------------------------------
struct PostJob {
  RowSet rs;
  int tile_start;          // first workgroup of this job
  int m_tiles;             // token tiles per group
};

struct PostArgs {
  int n_jobs;
  PostJob job[2];
  int d_model, d_ff;
  RowView o;               // attention output rows (storage dtype)
  RowView resid;           // block input rows (storage dtype in block 0, else fp32)
  RowView out;             // X' rows (fp32)
  const void *wo, *w1, *b1, *w2, *b2;   // [G][..] storage dtype
  const void *gamma, *beta;             // norm2 [d]
  int layer;
  float eps;
};

// ---------------------------------------------------------------------------------------------
// Attention launch.
//   Queries: q[b][h][i][dh] for i < R at positions p0 + i.
//   Keys 0..n_pre-1 (the "prefix"): k_pre + grp * pre_sb + h * pre_sh + key * dh, where grp is
//   the sequence (forward mode) or the user (Stage II mode) of the workgroup.
//   Stage II only: keys n_pre..n_pre+R-1 are the sequence's own rows:
//     k_own + b * own_sb + h * own_sh + j * dh.
//   Output o[b][i][h * dh + c] (row stride d).
// Forward mode groups a workgroup's queries as 128 consecutive rows of one sequence; Stage II
// mode groups 4 * (32 / R) candidates of one user (sequence b = user * n_cand + cand).
// ---------------------------------------------------------------------------------------------
struct AttnArgs {
  int n_seq_grp;           // forward: sequences; stage II: users
  int n_heads, d_model;
  int R, p0;
  int n_qblocks;
  int n_cand;              // stage II: candidates per user
  int n_pre;               // prefix keys
  const void *q; long long q_sb, q_sh;
  const void *k_pre, *v_pre; long long pre_sb, pre_sh;
  const void *k_own, *v_own; long long own_sb, own_sh;
  void *o; long long o_sb;
  float scale_log2;        // log2(e) / sqrt(d_head)
};

}  // namespace ot
