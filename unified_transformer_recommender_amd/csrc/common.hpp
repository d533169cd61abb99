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
// synchronisation and instruction-scheduling helpers
// ---------------------------------------------------------------------------------------------
// s_waitcnt constraining only the vector-memory counter (gfx9 encoding: vmcnt bits [3:0] and
// [15:14]). Vector-memory loads complete in issue order, so waiting for <= N outstanding means
// every load but the last N issued has landed (for direct-to-LDS loads: its LDS bytes are written).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads and writes have completed.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier with no memory fence. __syncthreads() also waits for every outstanding
// vector-memory access of the wave (vmcnt(0)), which would drain loads issued several chunks
// ahead; here the caller states exactly what must have completed (wait_vm / wait_lgkm0) before
// arriving. The empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct global->LDS load of 16 bytes per lane: lane i's bytes land at LDS byte address
// lds_base + 16 i (lds_base is wave-uniform). Written as inline assembly so that the compiler's
// wait-count bookkeeping does not see an outstanding LDS write: with the builtin, every later LDS
// read waits for lgkmcnt(0), which serialises the operand reads of the MFMA loops. The caller
// waits for completion explicitly (wait_vm) before the data is read; the asm has no outputs.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(src) : "memory", "m0");
}
// The same with a wave-uniform base address in SGPRs and a 32-bit per-lane byte offset (the
// load's scalar-base form): no per-lane 64-bit address arithmetic per load.
__device__ __forceinline__ void dma16s(const void *sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_base), "v"(voff), "s"(sbase) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) void *)p;
}

// Instruction order for an unrolled block of NR LDS reads feeding NM MFMAs: PD reads first, then
// one read after every MFMA, then the remaining MFMAs. Each MFMA's operand was requested PD
// instructions earlier, which hides the LDS latency behind the matrix pipe (the default schedule
// keeps only one read in flight to save registers). Place after the block, in the same basic block.
template <int NR, int NM, int PD>
__device__ __forceinline__ void sched_lds_mfma() {
  constexpr int P = PD < NR ? PD : NR;   // never more reads ahead than the block has
  static_assert(NR - P <= NM, "schedule shape");
  __builtin_amdgcn_sched_group_barrier(0x100, P, 0);
#pragma unroll
  for (int i = 0; i < NR - P; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NM - (NR - P), 0);
}

// ---------------------------------------------------------------------------------------------
// Transposed bf16 MFMA fragments from a row-major LDS tile [token][ROW] (ROW elements per row,
// features 0..31 used), by the transposing LDS read ds_read_b64_tr_b16. In each 16-lane group,
// lane i of the read receives element i % 4 of the 8-byte runs that lanes i / 4, 4 + i / 4,
// 8 + i / 4 and 12 + i / 4 of the group point at (measured on gfx950). Source lane s of the group
// that holds output lanes (features 16 h .. 16 h + 15, lane half g) points at
// tile[t0 + 4 g + s / 4][16 h + 4 (s % 4)], so output lane (lc, g) receives tokens
// t0 + 4 g + 0..3 of feature lc. Two reads, at t0 + 16 mc and t0 + 16 mc + 8, give the fragment of
// the 32-token k index in the accumulator-row order acc_row (tokens 16 mc + 4 g + 0..3 and
// 16 mc + 8 + 4 g + 0..3): the order in which a lane holds probabilities or score gradients, so
// they serve directly as the other operand.
// ---------------------------------------------------------------------------------------------
// Element offset of this lane's source address for the tokens starting at t0.
template <int ROW>
__device__ __forceinline__ int tr_src(int t0, int lane) {
  return (t0 + 4 * (lane >> 5) + ((lane >> 2) & 3)) * ROW + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
}
// k-chunk mc of the fragment; src = tile + tr_src<ROW>(t0, lane).
template <int ROW>
__device__ __forceinline__ bf16x8 tr_frag(const bf16 *src, int mc) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4 lds_s4;
  const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(src + 16 * mc * ROW));
  const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(src + (16 * mc + 8) * ROW));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

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
// GELU, the erf form 0.5 x (1 + erf(x / sqrt 2)).
// gelu_as (fp32 paths): erf by Abramowitz & Stegun 7.1.26 (|error| <= 1.5e-7): with
// z = |x| / sqrt 2, t = 1 / (1 + p z),
//   GELU(x) = max(x, 0) - |x| * 0.5 t (a1 + t(a2 + t(a3 + t(a4 + t a5)))) * exp(-x^2 / 2).
// gelu_fit (bf16 paths, whose activations are rounded to bf16 right after): a fitted sigmoid form
// with half the instructions (|error| <= 2.71e-4).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float gelu_as(float x) {
  // Abramowitz & Stegun 7.1.26 coefficients, halved so that q = 0.5 t P(t)
  constexpr float p = 0.3275911f * 0.70710678118654752f;   // p / sqrt(2): t = 1 / (1 + p |x| / sqrt 2)
  constexpr float a1 = 0.5f * 0.254829592f, a2 = 0.5f * -0.284496736f, a3 = 0.5f * 1.421413741f,
                  a4 = 0.5f * -1.453152027f, a5 = 0.5f * 1.061405429f;
  constexpr float neg_half_log2e = -0.72134752044448170f;   // -0.5 * log2(e)
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(p, ax, 1.0f));
  const float q = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
  const float e = __builtin_amdgcn_exp2f(x * x * neg_half_log2e);
  return fmaf(-ax * q, e, fmaxf(x, 0.0f));
}

// GELU for the bf16 path, whose hidden activations are rounded to bf16 (relative step 2^-8)
// before the down-projection: x sigma(z) with z = x (A1 + A3 x^2), the two coefficients a minimax
// fit to the erf form on [-12, 12] (max |error| 2.71e-4 there; z is monotone in x, so the limits
// x -> +-inf give x and 0). sigma(z) = 1 / (1 + 2^(-z log2 e)): 5 VALU and 2 transcendental
// instructions per value.
constexpr float GELU_FIT_A1 = 1.6003141571088118f;
constexpr float GELU_FIT_A3 = 0.06940178685506644f;
__device__ __forceinline__ float gelu_fit(float x) {
  constexpr float L = -1.4426950408889634f;   // -log2(e)
  const float x2 = x * x;
  const float z = x * fmaf(x2, GELU_FIT_A3 * L, GELU_FIT_A1 * L);
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z));
}

// ---------------------------------------------------------------------------------------------
// Coalesced store of a 32 x 32 accumulator tile whose 32 columns are tokens (lane l % 32) and
// whose 32 rows are consecutive output features. In registers a lane holds 16 features of its
// own token spread over the row, so storing straight from registers scatters 4-16 byte pieces
// over 32 rows. Instead the wave writes the tile into its own LDS staging area and reads it back
// as row-major 16-byte pieces: store instruction k of lane l writes piece (l % PPR) of token
// k * TPI + l / PPR, so each instruction covers TPI complete 32-feature runs.
// ---------------------------------------------------------------------------------------------
template <typename T>
struct TileStage {
  static constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte piece
  static constexpr int PPR = 32 / EPC;               // pieces per token run of 32 features
  static constexpr int TPI = 64 / PPR;               // tokens per store instruction
  static constexpr int NI = 32 / TPI;                // store instructions per tile
  static constexpr int LD = 32 + EPC;                // staging row (elements), padded by 16 bytes
  static constexpr int SIZE = 32 * LD;               // staging elements per wave

  // Token (0..31) whose piece this lane stores in instruction k, and that piece's first feature.
  static __device__ __forceinline__ int token(int k, int lane) { return k * TPI + lane / PPR; }
  static __device__ __forceinline__ int feature(int lane) { return (lane % PPR) * EPC; }

  // acc element v of lane (lc, g) is feature acc_row(v, g) of token lc.
  static __device__ __forceinline__ void put(T *stg, const f32x16 &acc, int lc, int g) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      T *d = stg + lc * LD + 8 * j + 4 * g;
      if constexpr (sizeof(T) == 2) {
        *(bf16x4 *)d = bf16x4{(bf16)acc[4 * j], (bf16)acc[4 * j + 1], (bf16)acc[4 * j + 2], (bf16)acc[4 * j + 3]};
      } else {
        *(f32x4 *)d = f32x4{acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]};
      }
    }
  }
  static __device__ __forceinline__ u32x4 get(const T *stg, int k, int lane) {
    return *(const u32x4 *)(stg + token(k, lane) * LD + feature(lane));
  }
};

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
  int xh_g0;               // first 32-row group of this job's rows in `xh`
};

struct QkvArgs {
  int n_jobs;
  QkvJob job[2];
  int d_model, d_head;
  RowView x;               // block input rows (storage dtype in block 0, else fp32)
  const void *wq, *wk, *wv;   // [G][d][d] storage dtype
  const void *gamma, *beta;   // norm1 [d]
  RowView stats;           // per-row (mean, rstd) of x from the previous block's tail, fp32; base null if absent
  int tg;                  // token groups of 32 per wave (1, or 2 where the kernel supports it)
  int n_split;             // workgroups per token tile, each taking a contiguous range of the
                           // tile's weight chunks (1: one workgroup does all of them)
  int layer;
  float eps;
  float q_scale;           // queries are stored multiplied by this (log2(e) / sqrt(d_head))
  void *trash;             // 16 bytes that masked-off output pieces are written to
  const int *kv_shift;     // [n_seq] or null: K/V row t of sequence b is stored at row t + kv_shift[b]
  const void *xh;          // bf16: the normalised rows in fragment order (xh_piece), written by the
                           // previous block's post-attention kernel; null: norm 1 runs here
};

// ---------------------------------------------------------------------------------------------
// Fused post-attention launch (W^O + residual + norm2 + mixed FFN + residual) over the query rows
// of a block: job 0 = tail S rows (parameter set 0), job 1 = NS rows (sets 1..l_ns).
// ---------------------------------------------------------------------------------------------
struct PostJob {
  RowSet rs;
  int tile_start;          // first workgroup of this job
  int m_tiles;             // token tiles per group
  int xh_g0;               // first 32-row group of this job's rows in `xh`
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
  RowView stats;           // where to write per-row (mean, rstd) of X' for the next block's norm 1; base null: none
  int layer;
  float eps;
  int n_split;             // workgroups per token tile, each over a contiguous range of the FFN's
                           // hidden chunks (1: one workgroup does the whole FFN)
  RowView part;            // n_split > 1: partial X' rows of split s at part.base + s * part_split
  long long part_split;    // elements (fp32; compact rows by (sequence, position)); a reduce launch adds them
  void *xh;                // bf16, n_split == 1: where to write the next block's norm-1 output of X'
                           // in fragment order (xh_piece); null: none
  const void *xh_gamma, *xh_beta;   // the next block's norm-1 parameters [d]
  int out_from;            // X' rows at output positions (t - out.t_off) below this are not stored:
                           // the next block reads them only through `xh` (0: store every row)
};

// Normalised rows handed from a block's post-attention kernel to the next block's QKV kernel
// (bf16). Both launches enumerate a parameter group's rows in the same order r (a block's output
// rows are the next block's input rows); rows 32 G .. 32 G + 31 of group grp of a job form row
// group xh_g0 + grp * ceil(M / 32) + G, where M is the job's rows per group. A row group stores,
// for each 16-feature k-chunk kc, the 64 lanes' MFMA B fragments in lane order: lane (g, lc)
// holds features 16 kc + 8 g .. 16 kc + 8 g + 7 of row 32 G + lc. One wave reads a k-chunk of its
// 32 rows as one contiguous 1 KB load. Returns the index of the 16-byte piece.
__device__ __forceinline__ size_t xh_piece(int xh_g0, int grp, int m_rows, int G, int kcs, int kc, int lane) {
  const int per_grp = (m_rows + 31) >> 5;
  return ((size_t)(xh_g0 + grp * per_grp + G) * kcs + kc) * 64 + lane;
}

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
  const int *seq_shift;    // [n_seq_grp] or null: sequence z's query positions and prefix keys
                           // start seq_shift[z] rows later (ragged cached lengths)
  float *lse;              // or null: base-2 log-sum-exp of each query's scores (log2(e) S, the
                           // softmax's log normaliser), at lse[(z * n_heads + h) * R + i]
};

// ---------------------------------------------------------------------------------------------
// Grouped linear layer of the tokenizers: per group, y = act(x W^T + b) or x W^T + b + b_add over
// m rows.
// Input row r at x + r * x_ld elements; output row r at
//   y + (r / y_rps) * y_ss + (r % y_rps) * y_rs elements
// (y_rps rows per sample, so a group can write its rows straight into X(0)).
// Workgroups [tile0, tile0 + m_tiles * n / 64) belong to the group, output tile fastest.
// ---------------------------------------------------------------------------------------------
constexpr int LIN_MAX_GROUPS = 8;
struct LinGroup {
  const void *x; long long x_ld;
  const void *w, *b;       // W [n][k] (out, in), b [n]
  void *y; long long y_ss, y_rs; int y_rps;
  int m, n, k;
  int gelu;                // exact erf GELU after the bias
  int tile0;
  const int *y_row;        // or null: output row r goes to row y_row[r] (instead of r % y_rps) of its sample
  const void *b_add;       // or null: a second bias [n] added with b (groups without GELU only)
};
struct LinArgs {
  LinGroup g[LIN_MAX_GROUPS];
  int n_groups;
};

// Timestamp-aware merge: merged row of every event, per sample (one workgroup each). Event l of
// type i has key (t[i][b][l], i, l); its row is the number of the sample's events with a smaller key.
struct RankArgs {
  const long long *t[LIN_MAX_GROUPS];   // [batch][len[i]] timestamps of type i
  int *pos[LIN_MAX_GROUPS];             // [batch][len[i]] merged row of each event
  int len[LIN_MAX_GROUPS];
  int n_seq, total;                     // total = sum of len
};

// [SEP] rows: row j of sep [n_sep][d] to row sep_row[j] of each sample (sample_stride elements).
struct SepArgs {
  const void *sep;
  void *x0; long long sample_stride;
  int d, n_sep, batch;
  int sep_row[LIN_MAX_GROUPS];
};

}  // namespace ot
