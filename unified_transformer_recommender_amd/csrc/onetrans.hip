// C ABI and host planner of the OneTrans hot path.
//
// Every operation is the same per-block launch sequence over a different set of rows
// (fun-rec-mdbook 7.5.1-7.5.3):
//   norm1 -> mixed Q/K/V projection -> causal attention -> W^O + residual -> norm2
//   -> FFN up + GELU -> FFN down + bias + residual
// forward   : S and NS rows of each sample, K/V of all block rows, queries = tail S rows + NS rows
// prefill   : S rows only, K/V written into the user's cache (Stage I)
// score     : NS rows of each candidate, keys = user's cached S rows + own NS rows (Stage II)
// append    : the new rows only, K/V appended to the cache, keys = cached + new rows
//
// Rows are addressed by (sequence b, position t) where t is the row's position in the current
// block's input; the pyramid re-indexes the kept tail rows from 0 for the next block (the tail is
// contiguous per sequence, so no copy is made).

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "onetrans.h"
#include "common.hpp"
#include "launch.hpp"
#include "bwd.hpp"

using namespace ot;

namespace {

// ---- per-launch timing (off unless enabled) ---------------------------------------------------
struct TimedLaunch {
  int cls;
  hipEvent_t a, b;
};
bool g_timing = false;
std::vector<TimedLaunch> g_timed;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` (returning hipError_t); with timing on, brackets it with events on `s`.
// Set while an allocation-free call runs: no timing events are created or recorded for it.
thread_local bool t_untimed = false;

template <class F>
hipError_t timed(int cls, hipStream_t s, F &&launch) {
  if (!g_timing || t_untimed) return launch();
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) return hipErrorOutOfMemory;
  if (hipEventRecord(a, s) != hipSuccess) return hipErrorInvalidValue;
  const hipError_t e = launch();
  if (hipEventRecord(b, s) != hipSuccess) return hipErrorInvalidValue;
  g_timed.push_back(TimedLaunch{cls, a, b});
  return e;
}

struct Dims {
  int N, d, H, dh, dff, lns, dt;
  size_t esz;
  int layer;
  float eps;
};

inline bool misaligned(const void *p) { return ((uintptr_t)p & 15u) != 0; }

int check_cfg(const onetrans_config *c, Dims &D) {
  if (!c) return ONETRANS_ERR_INVALID_ARG;
  if (c->n_blocks < 1 || c->d_model < 1 || c->n_heads < 1 || c->d_ff < 1 || c->l_ns < 0)
    return ONETRANS_ERR_INVALID_ARG;
  if (c->norm != ONETRANS_RMSNORM && c->norm != ONETRANS_LAYERNORM) return ONETRANS_ERR_INVALID_ARG;
  if (c->dtype != ONETRANS_F32 && c->dtype != ONETRANS_BF16) return ONETRANS_ERR_INVALID_ARG;
  if (!(c->norm_eps >= 0.0f) || !(c->norm_eps < 1.0f)) return ONETRANS_ERR_INVALID_ARG;
  if (c->d_model % c->n_heads) return ONETRANS_ERR_SHAPE;
  D.N = c->n_blocks;
  D.d = c->d_model;
  D.H = c->n_heads;
  D.dh = c->d_model / c->n_heads;
  D.dff = c->d_ff;
  D.lns = c->l_ns;
  D.dt = c->dtype;
  D.esz = c->dtype == ONETRANS_BF16 ? 2 : 4;
  D.layer = c->norm == ONETRANS_LAYERNORM;
  D.eps = c->norm_eps;
  if (D.dh != 16 && D.dh != 32) return ONETRANS_ERR_UNSUPPORTED;
  if ((D.d != 64 && D.d != 128 && D.d != 256 && D.d != 512) || D.dff % 64 || D.dff > POST_MAX_DFF)
    return ONETRANS_ERR_UNSUPPORTED;
  if (D.lns > 32) return ONETRANS_ERR_UNSUPPORTED;
  return ONETRANS_OK;
}

int check_schedule(const onetrans_config *c, int l_s) {
  if (!c->s_queries) return ONETRANS_ERR_INVALID_ARG;
  int s = l_s;
  for (int n = 0; n < c->n_blocks; ++n) {
    const int q = c->s_queries[n];
    if (q < 1 || q > s) return ONETRANS_ERR_SHAPE;
    s = q;
  }
  return ONETRANS_OK;
}

// Launch sizes of a call over n_seq sequences of at most `rows` block rows each: every kernel's
// grid (QKV and post tiles: at most one per row; attention: query blocks x sequences x heads, at
// most rows x sequences x heads) must fit a 32-bit int. Checked before anything is enqueued, so a
// call that fails here has launched nothing.
int check_size(const Dims &D, long long n_seq, long long rows) {
  if (n_seq * rows * D.H > 0x7fffffffLL) return ONETRANS_ERR_SHAPE;
  return ONETRANS_OK;
}

int check_weights(const onetrans_block_weights *blk, const Dims &D) {
  if (!blk) return ONETRANS_ERR_INVALID_ARG;
  for (int n = 0; n < D.N; ++n) {
    const onetrans_block_weights &w = blk[n];
    const void *req[] = {w.norm1_g, w.norm2_g, w.wq, w.wk, w.wv, w.wo, w.w1, w.b1, w.w2, w.b2};
    for (const void *p : req) {
      if (!p) return ONETRANS_ERR_INVALID_ARG;
      if (misaligned(p)) return ONETRANS_ERR_ALIGNMENT;
    }
    if (D.layer) {
      if (!w.norm1_b || !w.norm2_b) return ONETRANS_ERR_INVALID_ARG;
      if (misaligned(w.norm1_b) || misaligned(w.norm2_b)) return ONETRANS_ERR_ALIGNMENT;
    }
  }
  return ONETRANS_OK;
}

// ---- workspace -------------------------------------------------------------------------------
struct Ws {
  size_t x[2], st[2], q, k, v, o, trash, seq, part, total;
  size_t part_rows;   // rows per split of the partial-sum buffer (0: no split post launches)
  size_t xh;          // normalised rows handed from a post launch to the next block's QKV launch
  bool has_xh;
};

// Block chains that hand each block's normalised input from the previous block's post-attention
// kernel to its QKV kernel: bf16 storage (the single-wave post kernel at d <= 256, the wave-pair
// kernel at d = 512).
inline bool handoff_dims(const Dims &D) { return D.dt == ONETRANS_BF16; }

inline size_t al(size_t b) { return (b + 255) & ~(size_t)255; }

// Split post launches (the FFN's hidden chunks over several workgroups per token tile, partial sums
// reduced afterwards) are used by a whole call or not at all, so that a call's results do not depend
// on how it is split over streams: when the call's n_call sequences of rq query rows need at most
// POST_SPLIT_BYTES of partials.
inline bool post_split_call(const Dims &D, size_t n_call, size_t rq) {
  return n_call * rq * POST_MAX_SPLIT * D.d * 4 <= (size_t)POST_SPLIT_BYTES;
}

// n: sequences; tin: max block input rows; rq: max query rows; kv: K/V buffers needed;
// n_call: sequences of the whole call (n is one part of it); xh: room for the normalised-row handoff
Ws ws_layout(const Dims &D, size_t n, size_t tin, size_t rq, bool kv, size_t n_call, bool xh = false) {
  Ws w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += al(bytes);
    return o;
  };
  const size_t d = D.d, es = D.esz;
  // block outputs alternate between two buffers: the fused tail reads its block input as the
  // residual while writing the block output, so the two must not alias
  w.x[0] = take(n * rq * d * 4);
  w.x[1] = take(n * rq * d * 4);
  // per-row (mean, rstd) of the block output in x[i], written by the post-attention kernel for the
  // next block's norm 1
  w.st[0] = take(n * rq * 8);
  w.st[1] = take(n * rq * 8);
  w.q = take(n * rq * d * es);
  w.k = kv ? take(n * tin * d * es) : 0;
  w.v = kv ? take(n * tin * d * es) : 0;
  w.o = take(n * rq * d * es);
  // 16 bytes that the QKV kernel's masked-off lanes store to (its store count stays fixed)
  w.trash = take(16);
  // per-sequence row offsets of ragged cached users (int32)
  w.seq = take(n * 4);
  // partial sums of post launches split over the FFN's hidden chunks (small launches only)
  w.part_rows = post_split_call(D, n_call, rq) ? n * rq : 0;
  w.part = take(w.part_rows * POST_MAX_SPLIT * d * 4);
  // a block's n * rq query rows in 32-row groups per parameter group: the S rows' groups plus at
  // most one partial group for each of the l_ns NS groups and the S group; bf16
  w.has_xh = xh && handoff_dims(D);
  w.xh = w.has_xh ? take((n * rq + 32 * (size_t)(D.lns + 1)) * d * 2) : 0;
  w.total = off;
  return w;
}

bool ws_dims(const onetrans_config *c, const Dims &D, int op, int n_seq, int l_s, int n_cand, int d_l, size_t &n,
             size_t &tin, size_t &rq, bool &kv) {
  switch (op) {
    case ONETRANS_OP_FORWARD:
      if (n_seq < 1 || l_s < 1 || !c->s_queries) return false;
      n = n_seq; tin = (size_t)l_s + D.lns; rq = (size_t)c->s_queries[0] + D.lns; kv = true;
      return true;
    case ONETRANS_OP_PREFILL:
      if (n_seq < 1 || l_s < 1 || !c->s_queries) return false;
      n = n_seq; tin = l_s; rq = c->s_queries[0]; kv = false;
      return true;
    case ONETRANS_OP_SCORE:
      if (n_seq < 1 || n_cand < 1 || D.lns < 1) return false;
      n = (size_t)n_seq * n_cand; tin = rq = D.lns; kv = true;
      return true;
    case ONETRANS_OP_APPEND:
      // l_s > 0: the recomputed window of a pyramided cache (Stage I over l_s rows per user)
      if (n_seq < 1 || d_l < 1 || l_s < 0) return false;
      n = n_seq; tin = rq = std::max(d_l, l_s); kv = false;
      return true;
    default:
      return false;
  }
}

// ---- launches ------------------------------------------------------------------------------
// One block over one operation's rows.
struct Step {
  int n_seq;
  int s, q;            // S rows in the key range (positions 0..s-1); S query rows (tail)
  int kv_t0, kv_n;     // S rows whose K/V are computed here
  int ns;              // NS rows (positions s..s+ns-1), 0 if none
  int in_t0, in_n;     // input rows present (positions)
  RowView x;           // block input by position
  int x_f32;
  HeadView kS, vS, kN, vN;
  int stage2, n_grp, n_cand, n_pre;
  const void *kp, *vp;
  long long pre_sb, pre_sh;
  long long own_sb, own_sh;
  RowView out;         // X' (fp32), t_off = first query position
  bool need_out;
  void *stats_in;      // (mean, rstd) per row of x, laid out like x; null: norm 1 computes them
  void *stats_out;     // where the post kernel writes (mean, rstd) per row of out; null: none
  const int *kv_shift; // device [n_seq] or null: K/V rows of sequence b go kv_shift[b] rows later
  const int *seq_shift;   // device [n_grp] or null: attention positions / prefix keys of sequence
                          // (or user) z start seq_shift[z] rows later
  float *lse;             // or null: per-query base-2 log-sum-exp of the attention scores
  bool no_post;           // stop after the attention (the training step's recomputation)
  int only;               // 0: every phase; else the phases to run (STEP_QKV | STEP_ATTN | STEP_POST)
  const void *xh_in;      // or null: the block input's normalised rows, handed over by the previous post launch
  void *xh_out;           // or null: where the post launch may hand over the next block's normalised rows
  const void *xh_gamma, *xh_beta;   // the next block's norm-1 parameters
  int xh_keep;            // with xh_out: the first output row the next block reads as a residual
                          // (its first query row); the rows before it are read only through xh_out
  bool *xh_written;       // set when the post launch wrote xh_out
};
constexpr int STEP_QKV = 1, STEP_ATTN = 2, STEP_POST = 4;

// The attention arguments of a step (its Q and O in the step's workspace).
AttnArgs step_attn_args(const Dims &D, const Step &st, char *ws, const Ws &L) {
  const int d = D.d, H = D.H, dh = D.dh;
  const int p0 = st.s - st.q, R = st.q + st.ns;
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.n_heads = H;
  a.d_model = d;
  a.R = R;
  a.p0 = p0;
  a.n_pre = st.n_pre;
  a.q = ws + L.q;
  a.q_sb = (long long)H * R * dh;
  a.q_sh = (long long)R * dh;
  a.k_pre = st.kp;
  a.v_pre = st.vp;
  a.pre_sb = st.pre_sb;
  a.pre_sh = st.pre_sh;
  a.o = ws + L.o;
  a.o_sb = (long long)R * d;
  a.seq_shift = st.seq_shift;
  a.lse = st.lse;
  if (st.stage2) {
    a.n_seq_grp = st.n_grp;
    a.n_cand = st.n_cand;
    a.k_own = st.kN.base;
    a.v_own = st.vN.base;
    a.own_sb = st.own_sb;
    a.own_sh = st.own_sh;
    const int cpw = 32 / st.ns;
    a.n_qblocks = (st.n_cand + ATTN_WAVES * cpw - 1) / (ATTN_WAVES * cpw);
  } else {
    a.n_seq_grp = st.n_seq;
    a.n_qblocks = (R + ATTN_QBLOCK - 1) / ATTN_QBLOCK;
  }
  return a;
}

int run_step(const Dims &D, const onetrans_block_weights &w, const Step &st, char *ws, const Ws &L,
             hipStream_t stream) {
  const int d = D.d, H = D.H, dh = D.dh;
  const int p0 = st.s - st.q;
  const int R = st.q + st.ns;
  char *qb = ws + L.q, *ob = ws + L.o;
  int rc;

  const HeadView q_v{qb, (long long)H * R * dh, (long long)R * dh, p0};
  const int only = st.only ? st.only : STEP_QKV | STEP_ATTN | STEP_POST;

  // pre-norm 1 + mixed Q/K/V: K/V for the S rows [kv_t0, kv_t0 + kv_n) and the NS rows, Q for the
  // rows at positions >= p0 (tail S rows and NS rows)
  if (only & STEP_QKV) {
    QkvArgs qa;
    memset(&qa, 0, sizeof(qa));
    const int no_q = 0x7fffffff;
    int nj = 0, bm = 0;
    long long tiles = 0, groups = 0;
    auto add_job = [&](RowSet rs, int q_from, HeadView k, HeadView v) {
      const long long m = (long long)rs.n_seq * rs.rows;
      if (m == 0 || rs.n_groups == 0) return;
      QkvJob &j = qa.job[nj++];
      j.rs = rs;
      j.q_from = q_from;
      j.k = k;
      j.v = v;
      j.q = q_v;
      j.m_tiles = (int)((m + bm - 1) / bm);
      j.tile_start = (int)tiles;
      tiles += (long long)j.m_tiles * rs.n_groups;
      j.xh_g0 = (int)groups;
      groups += (m + 31) / 32 * rs.n_groups;
    };
    auto add_jobs = [&](int tg) {
      nj = 0;
      tiles = 0;
      groups = 0;
      bm = qkv_tokens_per_tile(tg);
      qa.tg = tg;
      if (st.kv_n > 0) add_job(RowSet{st.n_seq, st.kv_n, 1, st.kv_t0, 0, 0}, st.need_out ? p0 : no_q, st.kS, st.vS);
      if (st.ns > 0) add_job(RowSet{st.n_seq, 1, st.ns, st.s, 1, 1}, st.need_out ? st.s : no_q, st.kN, st.vN);
    };
    // two token groups per wave, unless that leaves fewer workgroups than half the GPU's CUs; a
    // launch that still has few tiles splits each tile's weight chunks over several workgroups
    add_jobs(qkv_max_groups(D.dt, d));
    if (qa.tg == 2 && tiles < QKV_SMALL_LAUNCH) add_jobs(1);
    qa.n_split = 1;
    if (tiles > 0 && tiles < QKV_SPLIT_TARGET)
      qa.n_split = (int)std::min<long long>(qkv_max_split(d), (QKV_SPLIT_TARGET + tiles - 1) / tiles);
    qa.n_jobs = nj;
    qa.d_model = d;
    qa.d_head = dh;
    qa.x = st.x;
    qa.wq = w.wq;
    qa.wk = w.wk;
    qa.wv = w.wv;
    qa.gamma = w.norm1_g;
    qa.beta = w.norm1_b;
    // only the bf16 norm at d >= 256 consumes row statistics (the other shapes keep the whole row
    // in registers and take them in the kernel)
    const bool row_stats = D.dt == ONETRANS_BF16 && d >= 256;
    if (row_stats && st.stats_in) qa.stats = RowView{st.stats_in, st.x.sb / d * 2, st.x.t_off, 2};
    qa.layer = D.layer;
    qa.eps = D.eps;
    qa.q_scale = 1.4426950408889634f / sqrtf((float)dh);
    qa.trash = ws + L.trash;
    qa.kv_shift = st.kv_shift;
    qa.xh = st.xh_in;
    const hipError_t e = timed(ONETRANS_K_QKV, stream, [&] { return launch_qkv(D.dt, st.x_f32, qa, (int)tiles, stream); });
    if (e != hipSuccess) return ONETRANS_ERR_HIP;
  }
  if (!st.need_out) return ONETRANS_OK;

  // attention
  if (only & STEP_ATTN) {
    const AttnArgs a = step_attn_args(D, st, ws, L);
    if (timed(ONETRANS_K_ATTN, stream, [&] { return launch_attn(D.dt, dh, st.stage2, a, stream); }) != hipSuccess)
      return ONETRANS_ERR_HIP;
  }
  if (st.no_post || !(only & STEP_POST)) return ONETRANS_OK;

  // W^O + residual + norm2 + mixed FFN + residual, fused, over the query rows:
  // tail S rows use parameter set 0, NS token j uses set 1 + j
  {
    PostArgs pa;
    memset(&pa, 0, sizeof(pa));
    const int bm = post_tokens_per_tile(D.dt, d);
    int nj = 0;
    long long tiles = 0, groups = 0;
    auto add_job = [&](RowSet rs) {
      const long long m = (long long)rs.n_seq * rs.rows;
      if (m == 0 || rs.n_groups == 0) return;
      PostJob &j = pa.job[nj++];
      j.rs = rs;
      j.m_tiles = (int)((m + bm - 1) / bm);
      j.tile_start = (int)tiles;
      tiles += (long long)j.m_tiles * rs.n_groups;
      j.xh_g0 = (int)groups;
      groups += (m + 31) / 32 * rs.n_groups;
    };
    if (st.q > 0) add_job(RowSet{st.n_seq, st.q, 1, p0, 0, 0});
    if (st.ns > 0) add_job(RowSet{st.n_seq, 1, st.ns, st.s, 1, 1});
    pa.n_jobs = nj;
    pa.d_model = d;
    pa.d_ff = D.dff;
    pa.o = RowView{ob, (long long)R * d, p0, d};
    pa.resid = st.x;
    pa.out = st.out;
    pa.wo = w.wo;
    pa.w1 = w.w1;
    pa.b1 = w.b1;
    pa.w2 = w.w2;
    pa.b2 = w.b2;
    pa.gamma = w.norm2_g;
    pa.beta = w.norm2_b;
    if (D.dt == ONETRANS_BF16 && d >= 256 && st.stats_out) pa.stats = RowView{st.stats_out, st.out.sb / d * 2, st.out.t_off, 2};
    pa.layer = D.layer;
    pa.eps = D.eps;
    // a small call splits the FFN's hidden chunks over up to POST_MAX_SPLIT workgroups per tile (the
    // 32-token-tile kernels; partial sums in the workspace, then one reduce launch)
    pa.n_split = 1;
    const long long rows = (long long)st.n_seq * R;
    const bool splittable = (D.dt == ONETRANS_BF16 || d <= 256) && L.part_rows > 0 && rows <= (long long)L.part_rows;
    if (splittable) {
      const int nc = D.dff / 32;
      while (pa.n_split < POST_MAX_SPLIT && nc % (pa.n_split * 2) == 0) pa.n_split *= 2;
    }
    if (pa.n_split > 1) {
      // compact rows, whatever the layout of `out` (x_tail's rows are `capacity` apart): the launch's
      // R query rows per sequence from position p0, n_seq * R <= part_rows
      pa.part = RowView{ws + L.part, (long long)R * d, p0, d};
      pa.part_split = (long long)L.part_rows * d;
    }
    // hand the next block's normalised rows over (the whole-FFN launches of the single-wave kernel);
    // the next block's row groups are this launch's: its input rows are these query rows, in order
    if (st.xh_out && pa.n_split == 1 && handoff_dims(D)) {
      pa.xh = st.xh_out;
      pa.xh_gamma = st.xh_gamma;
      pa.xh_beta = st.xh_beta;
      pa.out_from = st.xh_keep;
    }
    hipError_t e = timed(ONETRANS_K_POST, stream, [&] { return launch_post(D.dt, st.x_f32, pa, (int)tiles, stream); });
    if (e == hipSuccess && pa.xh && st.xh_written) *st.xh_written = true;
    if (e == hipSuccess && pa.n_split > 1)
      e = timed(ONETRANS_K_POST, stream, [&] { return launch_post_reduce(pa, (int)rows, stream); });
    if (e != hipSuccess) return ONETRANS_ERR_HIP;
  }
  return ONETRANS_OK;
}

int check_ws(const Dims &D, const Ws &L, void *ws, size_t ws_bytes) {
  if (!ws) return ONETRANS_ERR_INVALID_ARG;
  if (misaligned(ws)) return ONETRANS_ERR_ALIGNMENT;
  if (ws_bytes < L.total) return ONETRANS_ERR_WORKSPACE;
  (void)D;
  return ONETRANS_OK;
}

int check_cache(const onetrans_kv_cache *c) {
  if (!c || !c->k || !c->v || !c->layer_len) return ONETRANS_ERR_INVALID_ARG;
  if (c->n_users < 1 || c->capacity < 1) return ONETRANS_ERR_INVALID_ARG;
  if (misaligned(c->k) || misaligned(c->v) || (c->x_tail && misaligned(c->x_tail))) return ONETRANS_ERR_ALIGNMENT;
  return ONETRANS_OK;
}

// Ragged users: every user_len within [0, limit].
int check_user_len(const onetrans_kv_cache *c, int n_users, int limit) {
  for (int u = 0; u < n_users; ++u)
    if (c->user_len[u] < 0 || c->user_len[u] > limit) return ONETRANS_ERR_SHAPE;
  return ONETRANS_OK;
}

// Copy the users' cached lengths into the workspace (read on the host at enqueue time).
int upload_user_len(const onetrans_kv_cache *c, int n_users, char *ws, const Ws &L, hipStream_t stream) {
  if (hipMemcpyAsync(ws + L.seq, c->user_len, (size_t)n_users * sizeof(int), hipMemcpyHostToDevice, stream) !=
      hipSuccess)
    return ONETRANS_ERR_HIP;
  return ONETRANS_OK;
}

// Cache views of block n: layout [user][block][head][capacity][d_head].
inline HeadView cache_view(const Dims &D, const onetrans_kv_cache *c, void *base, int n) {
  const long long per_head = (long long)c->capacity * D.dh;
  return HeadView{(char *)base + (size_t)n * D.H * per_head * D.esz, (long long)D.N * D.H * per_head, per_head, 0};
}

// Arguments of a Stage II call (everything but the workspace).
int check_score(const onetrans_config *cfg, const onetrans_block_weights *blk, const onetrans_kv_cache *cache,
                const void *x_ns, int n_users, int n_cand, const void *out_ns, Dims &D) {
  int rc;
  if ((rc = check_cfg(cfg, D))) return rc;
  if (n_users < 1 || n_cand < 1) return ONETRANS_ERR_SHAPE;
  if (D.lns < 1) return ONETRANS_ERR_SHAPE;
  if ((rc = check_weights(blk, D))) return rc;
  if (!x_ns || !out_ns) return ONETRANS_ERR_INVALID_ARG;
  if (misaligned(x_ns) || misaligned(out_ns)) return ONETRANS_ERR_ALIGNMENT;
  if ((rc = check_cache(cache))) return rc;
  if (n_users > cache->n_users) return ONETRANS_ERR_SHAPE;
  for (int n = 0; n < D.N; ++n)
    if (cache->layer_len[n] < 0 || cache->layer_len[n] > cache->capacity) return ONETRANS_ERR_SHAPE;
  if (cache->user_len && (rc = check_user_len(cache, n_users, cache->capacity))) return rc;
  return check_size(D, (long long)n_users * n_cand, D.lns);
}

// ---- allocation-free Stage II: a library-owned device scratch ----------------------------------
// Stage II's workspace (block outputs, row statistics, Q/K/V/O of the candidates' NS rows, the
// ragged users' lengths) lives in this array instead of a caller buffer. It is in every GPU's copy
// of the library's device code and stays until the process ends. Host code never uses the array's
// name as an address (on the host it only stands for the symbol): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and kernels receive it as
// their workspace pointer.
static __device__ __align__(256) unsigned char scratch[ONETRANS_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
void *g_scratch[MAX_DEVICES];   // device address of `scratch` per device (null until first use)

// The current device's scratch address, looked up on the first call on that device.
int scratch_ptr(int dev, void *&out) {
  if (dev < 0 || dev >= MAX_DEVICES) return ONETRANS_ERR_HIP;
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ONETRANS_ERR_HIP;
    g_scratch[dev] = p;
  }
  out = g_scratch[dev];
  return ONETRANS_OK;
}

// ---- tokenizers (section 7.5.0) ----------------------------------------------------------------
// Workspace: the hidden activations of every MLP, [batch * rows][hidden] each, storage dtype.
// With the timestamp-aware merge also the merged row of every event, int32 [batch * len] per type.
struct TokPlan {
  int l_s, T, events;
  bool by_time;
  size_t hid[LIN_MAX_GROUPS], pos[LIN_MAX_GROUPS];
  size_t total;
};

int check_tok(const onetrans_config *cfg, const onetrans_tokenizer_config *tc, int batch, Dims &D, TokPlan &P) {
  int rc;
  if ((rc = check_cfg(cfg, D))) return rc;
  if (!tc || !tc->seq_len || !tc->seq_dim || !tc->seq_hidden) return ONETRANS_ERR_INVALID_ARG;
  if (tc->merge != ONETRANS_MERGE_INTENT && tc->merge != ONETRANS_MERGE_TIME) return ONETRANS_ERR_INVALID_ARG;
  if (batch < 1 || tc->n_seq < 1) return ONETRANS_ERR_SHAPE;
  if (tc->n_seq > LIN_MAX_GROUPS - 1) return ONETRANS_ERR_UNSUPPORTED;
  P.by_time = tc->merge == ONETRANS_MERGE_TIME;
  auto width_ok = [](int w) { return w >= 64 && w % 64 == 0; };
  long long l_s = 0, tiles1 = 0, tiles2 = 0;
  const long long rt = lin_rows_per_tile(), nt = lin_features_per_tile();
  size_t off = 0;
  for (int i = 0; i < tc->n_seq; ++i) {
    const int L = tc->seq_len[i];
    if (L < 0) return ONETRANS_ERR_SHAPE;
    if (!width_ok(tc->seq_dim[i]) || !width_ok(tc->seq_hidden[i])) return ONETRANS_ERR_UNSUPPORTED;
    const long long m = (long long)batch * L;
    if (m > (1LL << 30)) return ONETRANS_ERR_SHAPE;
    l_s += L + (P.by_time ? 0 : 1);
    tiles1 += (m + rt - 1) / rt * (tc->seq_hidden[i] / nt);
    tiles2 += (m + rt - 1) / rt * (D.d / nt);
    P.hid[i] = off;
    off += al((size_t)m * tc->seq_hidden[i] * D.esz);
  }
  if (D.lns > 0) {
    if (!width_ok(tc->ns_dim) || !width_ok(tc->ns_hidden)) return ONETRANS_ERR_UNSUPPORTED;
    tiles1 += (batch + rt - 1) / rt * (tc->ns_hidden / nt);
    tiles2 += (batch + rt - 1) / rt * ((long long)D.lns * D.d / nt);
    P.hid[tc->n_seq] = off;
    off += al((size_t)batch * tc->ns_hidden * D.esz);
  }
  if (l_s < 1 || l_s + D.lns > (1 << 24) || tiles1 >= (1LL << 31) || tiles2 >= (1LL << 31)) return ONETRANS_ERR_SHAPE;
  if (P.by_time) {
    if (l_s > RANK_MAX_EVENTS) return ONETRANS_ERR_UNSUPPORTED;
    for (int i = 0; i < tc->n_seq; ++i) {
      P.pos[i] = off;
      off += al((size_t)batch * tc->seq_len[i] * 4);
    }
  }
  P.events = (int)(P.by_time ? l_s : l_s - tc->n_seq);
  P.l_s = (int)l_s;
  P.T = P.l_s + D.lns;
  P.total = off > 0 ? off : 256;
  return ONETRANS_OK;
}

int check_mlp(const onetrans_mlp_weights *m) {
  if (!m || !m->w1 || !m->b1 || !m->w2 || !m->b2) return ONETRANS_ERR_INVALID_ARG;
  if (misaligned(m->w1) || misaligned(m->b1) || misaligned(m->w2) || misaligned(m->b2)) return ONETRANS_ERR_ALIGNMENT;
  return ONETRANS_OK;
}

// ---- batches over several streams ---------------------------------------------------------------
// Samples (forward) and users (Stage I, Stage II, append) are independent, so a call can run as
// up to four contiguous parts, part 0 on the caller's stream and part i on a library-owned stream
// of the same device (default priority), forked from and joined back into the caller's stream with
// events. The late pyramid blocks and the append / Stage II launches are small, and every kernel
// ends in a partial wave; parts in flight together fill those tails and the launch gaps.
// The workspace is always sized for the largest split the call's size allows (WsParts parts), which
// also holds every smaller split (halving a part never needs more bytes).
constexpr int MAX_PARTS = 4;
constexpr int FORWARD_PART_MIN = 32;   // samples per part
constexpr int USER_PART_MIN = 8;       // users per part
int g_streams = 2;                     // 1, 2 or 4
inline int ws_parts_for(int n, int min_part) { return n >= 4 * min_part ? 4 : n >= 2 * min_part ? 2 : 1; }
inline int parts_for(int n, int min_part) { return std::min(g_streams, ws_parts_for(n, min_part)); }

struct Side {
  hipStream_t s[MAX_PARTS - 1] = {};
  hipEvent_t fork = nullptr;
  hipEvent_t join[MAX_PARTS - 1] = {};
};
Side g_side[64];

// The side streams of the current device, created on first use. Returns 1 on a HIP error, and -1
// when `stream` belongs to another device than the current one (the call then stays on one stream:
// the side streams and their events live on the current device).
int side_streams(hipStream_t stream, Side *&out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  if (stream) {
    hipDevice_t sdev = 0;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return 1;
    if ((int)sdev != dev) return -1;
  }
  Side &sd = g_side[dev];
  if (!sd.fork) {
    for (int i = 0; i < MAX_PARTS - 1; ++i) {
      if (hipStreamCreateWithFlags(&sd.s[i], hipStreamNonBlocking) != hipSuccess) return 1;
      if (hipEventCreateWithFlags(&sd.join[i], hipEventDisableTiming) != hipSuccess) return 1;
    }
    if (hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming) != hipSuccess) return 1;
  }
  out = &sd;
  return 0;
}

// Runs run(first, count, part, stream) over `parts` contiguous ranges of [0, n) (ceil(n / parts)
// each, the last one shorter), each on its own stream, and joins them back into `stream`.
template <class F>
int over_streams(int n, int parts, hipStream_t stream, F &&run) {
  Side *sd = nullptr;
  if (parts > 1) {
    const int side = side_streams(stream, sd);
    if (side > 0) return ONETRANS_ERR_HIP;
    if (side < 0) parts = 1;
  }
  if (parts == 1) return run(0, n, 0, stream);
  if (hipEventRecord(sd->fork, stream) != hipSuccess) return ONETRANS_ERR_HIP;
  for (int i = 1; i < parts; ++i)
    if (hipStreamWaitEvent(sd->s[i - 1], sd->fork, 0) != hipSuccess) return ONETRANS_ERR_HIP;
  const int per = (n + parts - 1) / parts;
  int rc;
  for (int i = 0; i < parts && i * per < n; ++i)
    if ((rc = run(i * per, std::min(per, n - i * per), i, i == 0 ? stream : sd->s[i - 1]))) return rc;
  for (int i = 1; i < parts; ++i)
    if (hipEventRecord(sd->join[i - 1], sd->s[i - 1]) != hipSuccess ||
        hipStreamWaitEvent(stream, sd->join[i - 1], 0) != hipSuccess)
      return ONETRANS_ERR_HIP;
  return ONETRANS_OK;
}

// The users [first, ...) of a cache: layout [user][block][head][capacity][d_head], so a pointer
// offset (and the matching slice of user_len); layer_len stays shared.
onetrans_kv_cache user_view(const Dims &D, const onetrans_kv_cache *c, int first) {
  onetrans_kv_cache v = *c;
  const size_t user_bytes = (size_t)D.N * D.H * c->capacity * D.dh * D.esz;
  v.k = (char *)c->k + first * user_bytes;
  v.v = (char *)c->v + first * user_bytes;
  v.n_users = c->n_users - first;
  v.user_len = c->user_len ? c->user_len + first : nullptr;
  v.x_tail = c->x_tail ? (char *)c->x_tail + first * (size_t)c->capacity * D.d * 4 : nullptr;
  return v;
}

int forward_run(const Dims &D, const onetrans_config *cfg, const onetrans_block_weights *blk, const void *x0,
                int batch, int l_s, void *out, char *w, const Ws &L, hipStream_t stream) {
  int rc;
  const int d = D.d, H = D.H, dh = D.dh;
  int s = l_s;
  RowView x{const_cast<void *>(x0), (long long)(l_s + D.lns) * d, 0, d};
  int x_f32 = D.dt == ONETRANS_F32;
  void *stats = nullptr;   // (mean, rstd) rows of x when the previous block wrote them
  bool handed = false;     // the previous block's post launch wrote x's normalised rows to L.xh
  for (int n = 0; n < D.N; ++n) {
    const int q = cfg->s_queries[n];
    const int T = s + D.lns, R = q + D.lns, p0 = s - q;
    Step st{};
    st.n_seq = batch;
    st.s = s;
    st.q = q;
    st.kv_t0 = 0;
    st.kv_n = s;
    st.ns = D.lns;
    st.in_t0 = 0;
    st.in_n = T;
    st.x = x;
    st.x_f32 = x_f32;
    st.kS = HeadView{w + L.k, (long long)H * T * dh, (long long)T * dh, 0};
    st.vS = HeadView{w + L.v, (long long)H * T * dh, (long long)T * dh, 0};
    st.kN = st.kS;
    st.vN = st.vS;
    st.stage2 = 0;
    st.n_pre = T;
    st.kp = w + L.k;
    st.vp = w + L.v;
    st.pre_sb = (long long)H * T * dh;
    st.pre_sh = (long long)T * dh;
    st.out = RowView{n + 1 == D.N ? out : (void *)(w + L.x[n & 1]), (long long)R * d, p0, d};
    st.need_out = true;
    st.stats_in = stats;
    st.stats_out = n + 1 == D.N ? nullptr : (void *)(w + L.st[n & 1]);
    // one handoff buffer: the next block's QKV launch reads it before its post launch rewrites it
    bool wrote = false;
    st.xh_in = handed ? w + L.xh : nullptr;
    if (L.has_xh && n + 1 < D.N) {
      st.xh_out = w + L.xh;
      st.xh_gamma = blk[n + 1].norm1_g;
      st.xh_beta = blk[n + 1].norm1_b;
      st.xh_keep = q - cfg->s_queries[n + 1];
      st.xh_written = &wrote;
    }
    if ((rc = run_step(D, blk[n], st, w, L, stream))) return rc;
    x = RowView{w + L.x[n & 1], (long long)R * d, 0, d};
    stats = st.stats_out;
    handed = wrote;
    x_f32 = 1;
    s = q;
  }
  return ONETRANS_OK;
}

// Rows of user-major [user][capacity][d] fp32 x_tail, addressed by position in the sequence.
inline RowView tail_rows(const Dims &D, const onetrans_kv_cache *c, int t_off) {
  return RowView{c->x_tail, (long long)c->capacity * D.d, t_off, D.d};
}

// The append launch sequence over blocks [0, n_head) for `n_users` users of `cache` (a view whose
// first user is the call's first user), with workspace `w` laid out as L. l_old: cached rows (0
// for ragged users, whose own lengths come from cache->user_len). Every block computes the d_l new
// rows; their K/V go to offset l_old. When n_head == N the last block keeps q_final of the new rows
// as queries (its last q_final rows; out_new [U][q_final][d]); otherwise the outputs of block
// n_head - 1 for the new rows go to x_tail at their positions (the recomputed blocks' input).
int append_run(const Dims &D, const onetrans_block_weights *blk, const onetrans_kv_cache *cache, const void *x_new,
               int n_users, int d_l, void *out_new, char *w, const Ws &L, int l_old, int n_head, int q_final,
               hipStream_t stream) {
  int rc;
  const bool ragged = cache->user_len != nullptr;
  if (ragged && (rc = upload_user_len(cache, n_users, w, L, stream))) return rc;
  // ragged users: positions are relative to each user's own cached length, which the QKV kernel
  // adds to the cache rows it writes and the attention to its query positions and key count
  const int *shift = ragged ? (const int *)(w + L.seq) : nullptr;
  const int d = D.d;
  RowView x{const_cast<void *>(x_new), (long long)d_l * d, l_old, d};
  int x_f32 = D.dt == ONETRANS_F32;
  void *stats = nullptr;   // (mean, rstd) rows of x when the previous block wrote them
  for (int n = 0; n < n_head; ++n) {
    const bool last = n + 1 == D.N;        // the stack's last block
    const bool to_tail = n + 1 == n_head && !last;
    const int q = last ? q_final : d_l;
    Step st{};
    st.n_seq = n_users;
    st.s = l_old + d_l;
    st.q = q;
    st.kv_t0 = l_old;
    st.kv_n = d_l;
    st.ns = 0;
    st.in_t0 = l_old;
    st.in_n = d_l;
    st.x = x;
    st.x_f32 = x_f32;
    st.kS = cache_view(D, cache, cache->k, n);
    st.vS = cache_view(D, cache, cache->v, n);
    st.kN = st.kS;
    st.vN = st.vS;
    st.stage2 = 0;
    st.n_pre = l_old + d_l;
    st.kp = st.kS.base;
    st.vp = st.vS.base;
    st.pre_sb = st.kS.sb;
    st.pre_sh = st.kS.sh;
    if (to_tail)
      st.out = tail_rows(D, cache, 0);
    else if (last)
      st.out = RowView{out_new, (long long)q * d, l_old + d_l - q, d};
    else
      st.out = RowView{w + L.x[n & 1], (long long)d_l * d, l_old, d};
    st.kv_shift = shift;
    st.seq_shift = shift;
    st.stats_in = stats;
    st.stats_out = last || to_tail ? nullptr : (void *)(w + L.st[n & 1]);
    st.need_out = !last || (out_new != nullptr && q > 0);
    if ((rc = run_step(D, blk[n], st, w, L, stream))) return rc;
    x = RowView{w + L.x[n & 1], (long long)d_l * d, l_old, d};
    stats = st.stats_out;
    x_f32 = 1;
  }
  return ONETRANS_OK;
}

// The Stage II launch sequence for `n_users` users of `cache` (a view whose first user is the
// call's first user), with workspace `w` laid out as L.
int score_run(const Dims &D, const onetrans_block_weights *blk, const onetrans_kv_cache *cache, const void *x_ns,
              int n_users, int n_cand, void *out_ns, char *w, const Ws &L, hipStream_t stream) {
  int rc;
  const bool ragged = cache->user_len != nullptr;
  if (ragged && (rc = upload_user_len(cache, n_users, w, L, stream))) return rc;
  const int d = D.d, H = D.H, dh = D.dh, ns = D.lns;
  const int nseq = n_users * n_cand;
  // ragged users: positions are relative to each user's own cached length (the attention adds it)
  RowView x{const_cast<void *>(x_ns), (long long)ns * d, ragged ? 0 : cache->layer_len[0], d};
  int x_f32 = D.dt == ONETRANS_F32;
  void *stats = nullptr;   // (mean, rstd) rows of x when the previous block wrote them
  bool handed = false;     // the previous block's post launch wrote x's normalised rows to L.xh
  for (int n = 0; n < D.N; ++n) {
    const int s = ragged ? 0 : cache->layer_len[n];
    Step st{};
    st.n_seq = nseq;
    st.s = s;
    st.q = 0;
    st.kv_t0 = 0;
    st.kv_n = 0;
    st.ns = ns;
    st.in_t0 = s;
    st.in_n = ns;
    x.t_off = s;
    st.x = x;
    st.x_f32 = x_f32;
    st.kN = HeadView{w + L.k, (long long)H * ns * dh, (long long)ns * dh, s};
    st.vN = HeadView{w + L.v, (long long)H * ns * dh, (long long)ns * dh, s};
    st.kS = st.kN;
    st.vS = st.vN;
    const HeadView cv = cache_view(D, cache, cache->k, n);
    st.stage2 = 1;
    st.n_grp = n_users;
    st.n_cand = n_cand;
    st.n_pre = s;
    st.kp = cv.base;
    st.vp = cache_view(D, cache, cache->v, n).base;
    st.pre_sb = cv.sb;
    st.pre_sh = cv.sh;
    st.own_sb = st.kN.sb;
    st.own_sh = st.kN.sh;
    st.seq_shift = ragged ? (const int *)(w + L.seq) : nullptr;
    st.out = RowView{n + 1 == D.N ? out_ns : (void *)(w + L.x[n & 1]), (long long)ns * d, s, d};
    st.need_out = true;
    st.stats_in = stats;
    st.stats_out = n + 1 == D.N ? nullptr : (void *)(w + L.st[n & 1]);
    // the NS rows are every row of the next block and all of its query rows: each is handed over
    // and kept as a residual
    bool wrote = false;
    st.xh_in = handed ? w + L.xh : nullptr;
    if (L.has_xh && n + 1 < D.N) {
      st.xh_out = w + L.xh;
      st.xh_gamma = blk[n + 1].norm1_g;
      st.xh_beta = blk[n + 1].norm1_b;
      st.xh_keep = 0;
      st.xh_written = &wrote;
    }
    if ((rc = run_step(D, blk[n], st, w, L, stream))) return rc;
    x = RowView{w + L.x[n & 1], (long long)ns * d, 0, d};
    stats = st.stats_out;
    handed = wrote;
    x_f32 = 1;
  }
  return ONETRANS_OK;
}

// A cross-request append followed by the scoring of the same users' candidates, block by block
// (unpyramided cache; d_l <= 32 appended rows and n_cand * l_ns <= 32 NS rows per user): per block
// the append's QKV (its K/V into the cache), Stage II's QKV, one attention pass over the user's keys
// for both (attn_pair_kernel: the cache is read once), then both post launches. Stage II of block
// n needs block n's appended K/V and block n - 1's Stage II output, both ready at that point, so
// the result equals append_run followed by score_run. Workspaces: wa laid out as La (append), wb as
// Lb (Stage II).
int append_score_run(const Dims &D, const onetrans_block_weights *blk, const onetrans_kv_cache *cache,
                     const void *x_new, int n_users, int d_l, void *out_new, const void *x_ns, int n_cand,
                     void *out_ns, char *wa, const Ws &La, char *wb, const Ws &Lb, int l_old, hipStream_t stream) {
  int rc;
  const bool ragged = cache->user_len != nullptr;
  if (ragged && (rc = upload_user_len(cache, n_users, wa, La, stream))) return rc;
  // ragged users: positions relative to each user's own (pre-append) cached length; Stage II's key
  // count is the same user's length after the append, which the pair kernel takes from the append
  const int *shift = ragged ? (const int *)(wa + La.seq) : nullptr;
  const int d = D.d, H = D.H, dh = D.dh, ns = D.lns;
  const int s_new = l_old + d_l;          // cached rows after the append (ragged: relative)
  RowView xa{const_cast<void *>(x_new), (long long)d_l * d, l_old, d};
  RowView xb{const_cast<void *>(x_ns), (long long)ns * d, s_new, d};
  int xa_f32 = D.dt == ONETRANS_F32, xb_f32 = xa_f32;
  void *sa = nullptr, *sb = nullptr;      // (mean, rstd) rows of the inputs when written
  for (int n = 0; n < D.N; ++n) {
    const bool last = n + 1 == D.N;
    Step A{};
    A.n_seq = n_users;
    A.s = s_new;
    A.q = d_l;
    A.kv_t0 = l_old;
    A.kv_n = d_l;
    A.in_t0 = l_old;
    A.in_n = d_l;
    A.x = xa;
    A.x_f32 = xa_f32;
    A.kS = cache_view(D, cache, cache->k, n);
    A.vS = cache_view(D, cache, cache->v, n);
    A.kN = A.kS;
    A.vN = A.vS;
    A.n_pre = s_new;
    A.kp = A.kS.base;
    A.vp = A.vS.base;
    A.pre_sb = A.kS.sb;
    A.pre_sh = A.kS.sh;
    A.out = last ? RowView{out_new, (long long)d_l * d, l_old, d} : RowView{wa + La.x[n & 1], (long long)d_l * d, l_old, d};
    A.kv_shift = shift;
    A.seq_shift = shift;
    A.stats_in = sa;
    A.stats_out = last ? nullptr : (void *)(wa + La.st[n & 1]);
    A.need_out = true;
    Step B{};
    B.n_seq = n_users * n_cand;
    B.s = s_new;
    B.ns = ns;
    B.in_t0 = s_new;
    B.in_n = ns;
    xb.t_off = s_new;
    B.x = xb;
    B.x_f32 = xb_f32;
    B.kN = HeadView{wb + Lb.k, (long long)H * ns * dh, (long long)ns * dh, s_new};
    B.vN = HeadView{wb + Lb.v, (long long)H * ns * dh, (long long)ns * dh, s_new};
    B.kS = B.kN;
    B.vS = B.vN;
    B.stage2 = 1;
    B.n_grp = n_users;
    B.n_cand = n_cand;
    B.n_pre = s_new;
    B.kp = A.kp;
    B.vp = A.vp;
    B.pre_sb = A.pre_sb;
    B.pre_sh = A.pre_sh;
    B.own_sb = B.kN.sb;
    B.own_sh = B.kN.sh;
    B.out = RowView{last ? out_ns : (void *)(wb + Lb.x[n & 1]), (long long)ns * d, s_new, d};
    B.stats_in = sb;
    B.stats_out = last ? nullptr : (void *)(wb + Lb.st[n & 1]);
    B.need_out = true;

    A.only = B.only = STEP_QKV;
    if ((rc = run_step(D, blk[n], A, wa, La, stream)) || (rc = run_step(D, blk[n], B, wb, Lb, stream))) return rc;
    {
      const AttnArgs aa = step_attn_args(D, A, wa, La), ab = step_attn_args(D, B, wb, Lb);
      if (timed(ONETRANS_K_ATTN, stream, [&] { return launch_attn_pair(D.dt, dh, aa, ab, stream); }) != hipSuccess)
        return ONETRANS_ERR_HIP;
    }
    A.only = B.only = STEP_POST;
    if ((rc = run_step(D, blk[n], A, wa, La, stream)) || (rc = run_step(D, blk[n], B, wb, Lb, stream))) return rc;
    xa = RowView{wa + La.x[n & 1], (long long)d_l * d, l_old, d};
    xb = RowView{wb + Lb.x[n & 1], (long long)ns * d, 0, d};
    sa = A.stats_out;
    sb = B.stats_out;
    xa_f32 = xb_f32 = 1;
  }
  return ONETRANS_OK;
}

// The Stage I launch sequence over blocks [n0, N) for `n_users` users of `cache` (a view whose
// first user is the call's first user), with workspace `w` laid out as L. Block n0's input rows are
// `x` (s rows per user at block positions 0..s-1; x_f32: fp32 rather than the storage dtype). Block
// n keeps q[n] tail rows as the next block's input and writes the K/V of all its rows into the
// cache; the last block keeps q_final rows and writes them to `out` ([U][q_final][d], or nothing
// if null). Block tail_block (-1: none; its positions must be the sequence's) also writes its kept
// rows to x_tail, from where the next block reads them. Writes no host state.
int stack_run(const Dims &D, const onetrans_block_weights *blk, RowView x, int x_f32, int s, int n_users,
              const onetrans_kv_cache *cache, int n0, const int *q_of, int q_final, int tail_block, void *out,
              char *w, const Ws &L, hipStream_t stream) {
  int rc;
  const int d = D.d;
  void *stats = nullptr;   // (mean, rstd) rows of x when the previous block wrote them
  bool handed = false;     // the previous block's post launch wrote x's normalised rows to L.xh
  for (int n = n0; n < D.N; ++n) {
    const bool last = n + 1 == D.N;
    const bool to_tail = n == tail_block && !last;
    const int q = last ? q_final : q_of[n];
    const int p0 = s - q;
    Step st{};
    st.n_seq = n_users;
    st.s = s;
    st.q = q;
    st.kv_t0 = 0;
    st.kv_n = s;
    st.ns = 0;
    st.in_t0 = 0;
    st.in_n = s;
    st.x = x;
    st.x_f32 = x_f32;
    st.kS = cache_view(D, cache, cache->k, n);
    st.vS = cache_view(D, cache, cache->v, n);
    st.kN = st.kS;
    st.vN = st.vS;
    st.stage2 = 0;
    st.n_pre = s;
    st.kp = st.kS.base;
    st.vp = st.vS.base;
    st.pre_sb = st.kS.sb;
    st.pre_sh = st.kS.sh;
    if (to_tail)
      st.out = tail_rows(D, cache, 0);
    else
      st.out = RowView{last ? out : (void *)(w + L.x[n & 1]), (long long)q * d, p0, d};
    st.need_out = !last || out != nullptr;
    st.stats_in = stats;
    st.stats_out = last || to_tail ? nullptr : (void *)(w + L.st[n & 1]);
    // normalised-row handoff to the next block; rows that go to x_tail are all kept (the caller's
    // buffer), otherwise the rows before the next block's first query row are not stored
    bool wrote = false;
    st.xh_in = handed ? w + L.xh : nullptr;
    if (L.has_xh && !last) {
      const int q_next = n + 2 == D.N ? q_final : q_of[n + 1];
      st.xh_out = w + L.xh;
      st.xh_gamma = blk[n + 1].norm1_g;
      st.xh_beta = blk[n + 1].norm1_b;
      st.xh_keep = to_tail ? 0 : q - q_next;
      st.xh_written = &wrote;
    }
    if ((rc = run_step(D, blk[n], st, w, L, stream))) return rc;
    // the next block's row t is this block's position p0 + t
    x = to_tail ? tail_rows(D, cache, -p0) : RowView{w + L.x[n & 1], (long long)q * d, 0, d};
    stats = st.stats_out;
    handed = wrote;
    x_f32 = 1;
    s = q;
  }
  return ONETRANS_OK;
}

// First block of a schedule that prunes (keeps fewer rows than its input has), or -1.
int first_pruning_block(const int *q, int N, int l_s) {
  int s = l_s;
  for (int n = 0; n < N; ++n) {
    if (q[n] < s) return n;
    s = q[n];
  }
  return -1;
}


// ---- training step (fun-rec-mdbook 7.5.3, closing paragraph: mixed precision with activation
// recomputation) ----------------------------------------------------------------------------------
//
// Forward over the batch keeping only each block's input rows (fp32 checkpoints), then per block,
// last to first, with s S rows in, q kept, T = s + l_ns rows, R = q + l_ns query rows, p0 = s - q:
//   recompute  xh^T = Norm1(X) (feature-major), Q/K/V and O with each query's log-sum-exp (the
//              forward's QKV and attention kernels), Y = X[tail] + O Wo^T, yh = Norm2(Y),
//              hid^T = GELU(hpre) with hpre = yh W1^T + b1 (hpre itself is not stored)
//   backward   dhpre = (dOut W2) * GELU'(hpre), hpre formed again in registers by the same kernel;
//              dW2 += dOut^T hid, db2 += dOut; dW1 += dhpre^T yh,
//              db1 += dhpre; dYh = dhpre W1; dY = Norm2'(dYh) + dOut; dO = dY Wo; dWo += dY^T O;
//              attention backward -> dK, dV, dQ; dWq/k/v += d{Q,K,V}^T Xh;
//              dXh = dK Wk + dV Wv + dQ Wq; dX = Norm1'(dXh) + dY on the tail rows
// Every mixed product runs as an S-rows job (set 0) and an NS job (set 1 + j for NS token j). Weight
// gradients are contractions over tokens of feature-major copies (tokens of a set contiguous).

inline long long pad64(long long n) { return (n + 63) / 64 * 64; }

// Element (b, t) of a row buffer at base + (b * sb + (t - t_off) * rs) * esz bytes.
struct RowBuf {
  char *base;
  size_t esz;
  long long sb;
  int rs, t_off;
};
inline Mat2 rows_S(const RowBuf &r, int t0, int cnt) {
  return Mat2{r.base + (long long)(t0 - r.t_off) * r.rs * (long long)r.esz, 0, r.sb, cnt, r.rs};
}
inline Mat2 rows_N(const RowBuf &r, int s) {
  return Mat2{r.base + (long long)(s - r.t_off) * r.rs * (long long)r.esz, r.rs, r.sb, 1, 0};
}
inline RowView view(const RowBuf &r) { return RowView{r.base, r.sb, r.t_off, r.rs}; }

// Row n of weight set w at base + (w * set + n * rs) * esz bytes.
struct WBuf {
  const char *base;
  size_t esz;
  long long set;
  int rs;
};
inline Mat2 w_set(const WBuf &w, int set0) { return Mat2{w.base + set0 * w.set * (long long)w.esz, w.set, 0, 0x7fffffff, w.rs}; }

// Feature-major copy of F features: S tokens at S + f * ldS + token, NS token j at N + (j F + f) ldN + b.
struct FeatBuf {
  char *S, *N;
  long long ldS, ldN;
  int F;
};
inline MatT featT_S(const FeatBuf &f) { return MatT{f.S, 0, f.ldS}; }
inline MatT featT_N(const FeatBuf &f) { return MatT{f.N, (long long)f.F * f.ldN, f.ldN}; }
inline Mat2 feat_S(const FeatBuf &f) { return Mat2{f.S, 0, 0, 0x7fffffff, (int)f.ldS}; }
inline Mat2 feat_N(const FeatBuf &f) { return Mat2{f.N, (long long)f.F * f.ldN, 0, 0x7fffffff, (int)f.ldN}; }

struct GemmPlan {
  GemmArgs a;
  long long tiles;
  long long part_elems;   // PARTIAL jobs: fp32 partial elements (splits included)
  long long rsum_elems;
};
inline void plan_init(GemmPlan &P) {
  memset(&P.a, 0, sizeof(P.a));
  P.tiles = P.part_elems = P.rsum_elems = 0;
}
inline void plan_add(GemmPlan &P, GemmJob j) {
  if (j.m <= 0 || j.n_groups <= 0) return;
  j.m_tiles = (j.m + gemm_tokens_per_tile() - 1) / gemm_tokens_per_tile();
  j.n_tiles = j.n_feat / gemm_features_per_tile();
  j.tile0 = (int)P.tiles;
  P.tiles += (long long)j.n_split * j.n_groups * j.m_tiles * j.n_tiles;
  P.a.job[P.a.n_jobs++] = j;
}

// Split of a weight-gradient contraction over `chunks` 128-byte chunks per row: enough workgroups
// for the GPU (about 1024 per job), at least 8 chunks per split.
inline int wgrad_split(long long chunks, long long tiles) {
  long long s = (1024 + tiles - 1) / tiles;
  s = std::min(s, chunks / 8);
  return (int)std::max(1LL, std::min(s, 256LL));
}

// dW[set][m][n] (+ row sums) = sum over the set's tokens of A^T B, for the S set (one group) and
// the NS sets (l_ns groups); partials and row-sum partials at running offsets of part / rsum.
struct WgradOut {
  float *w, *b;   // gradient destinations (set 0 first), b may be null
};
void wgrad_jobs(GemmPlan &P, RedArgs *R, const Dims &D, const FeatBuf &A, const FeatBuf &Bf, long long tokS,
                int B, WgradOut dst, float *part, float *rsum) {
  const int m = A.F, n = Bf.F;
  const int kc = (int)(128 / D.esz);
  for (int ns = 0; ns < 2; ++ns) {
    const int groups = ns ? D.lns : 1;
    if (groups == 0 || (ns ? B : tokS) == 0) continue;
    GemmJob j;
    memset(&j, 0, sizeof(j));
    j.a = ns ? feat_N(A) : feat_S(A);
    j.b = ns ? feat_N(Bf) : feat_S(Bf);
    j.m = m;
    j.n_feat = n;
    j.k_len = (int)(ns ? A.ldN : A.ldS);
    j.n_groups = groups;
    const long long base_tiles = (long long)groups * ((m + 127) / 128) * (n / 64);
    j.n_split = wgrad_split(j.k_len / kc, base_tiles);
    j.epi = EPI_PARTIAL;
    j.out = Mat2{part ? part + P.part_elems : nullptr, (long long)m * n, 0, 0x7fffffff, n};
    j.part_split = (long long)groups * m * n;
    if (dst.b) {
      j.rowsum = rsum ? rsum + P.rsum_elems : nullptr;
      j.rowsum_split = (long long)groups * m;
    }
    const long long pe = (long long)j.n_split * groups * m * n, re = dst.b ? (long long)j.n_split * groups * m : 0;
    if (R && part) {
      RedJob &r = R->job[R->n_jobs++];
      r.src = part + P.part_elems;
      r.split = j.part_split;
      r.n_split = j.n_split;
      r.dst = dst.w + (ns ? (long long)m * n : 0);
      r.count = (long long)groups * m * n;
      r.start = R->total;
      R->total += (r.count + 3) / 4 * 4;
      if (dst.b) {
        RedJob &rb = R->job[R->n_jobs++];
        rb.src = rsum + P.rsum_elems;
        rb.split = j.rowsum_split;
        rb.n_split = j.n_split;
        rb.dst = dst.b + (ns ? m : 0);
        rb.count = (long long)groups * m;
        rb.start = R->total;
        R->total += (rb.count + 3) / 4 * 4;
      }
    }
    P.part_elems += (pe + 63) / 64 * 64;
    P.rsum_elems += (re + 63) / 64 * 64;
    plan_add(P, j);
  }
}

struct TrainWs {
  Ws fw;                      // the forward kernels' buffers (q, k, v, o, trash)
  std::vector<size_t> ckpt;   // [N]: block n's input rows (n >= 1), fp32 [B][T_n][d]
  size_t lse, dvec, y, yh, dhpre, dyh, dy32, dyt, dout_t, d_o, dqkv, dxh, dx32;
  size_t xhT, dkT, dvT, dqT, oT, dyT, yhT, dhpreT, hidT, doutT;
  size_t woT, w1T, w2T, wcT;
  size_t part, rsum, colpart, colsum2;
  long long ldS_all, ldS_tail, ldN;   // block-0 (largest) feature-major row lengths
  size_t total;
};

// S rows of block n (s_n) and the schedule's kept rows.
inline int block_s(const onetrans_config *cfg, int l_s, int n) { return n == 0 ? l_s : cfg->s_queries[n - 1]; }

TrainWs train_layout(const Dims &D, const onetrans_config *cfg, int B, int l_s) {
  TrainWs w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += al(bytes);
    return o;
  };
  const size_t d = D.d, es = D.esz, L = D.lns, dff = D.dff, G = 1 + L;
  const size_t T0 = (size_t)l_s + L, R0 = (size_t)cfg->s_queries[0] + L;
  const size_t rowsT = (size_t)B * T0, rowsR = (size_t)B * R0;
  w.fw = Ws{};
  w.fw.q = take(rowsR * d * es);
  w.fw.k = take(rowsT * d * es);
  w.fw.v = take(rowsT * d * es);
  w.fw.o = take(rowsR * d * es);
  w.fw.trash = take(16);
  w.fw.part_rows = 0;
  w.ckpt.assign(D.N, 0);
  for (int n = 1; n < D.N; ++n) w.ckpt[n] = take((size_t)B * (block_s(cfg, l_s, n) + L) * d * 4);
  w.lse = take(rowsR * D.H * 4);
  w.dvec = take(rowsR * D.H * 4);
  w.y = take(rowsR * d * 4);
  w.yh = take(rowsR * d * es);
  w.dhpre = take(rowsR * dff * es);
  w.dyh = take(rowsR * d * 4);
  w.dy32 = take(rowsR * d * 4);
  w.dyt = take(rowsR * d * es);
  w.dout_t = take(rowsR * d * es);
  w.d_o = take(rowsR * d * es);
  w.dqkv = take(rowsT * 3 * d * es);
  w.dxh = take(rowsT * d * 4);
  w.dx32 = take((D.N > 1 ? rowsR : 0) * d * 4);
  w.ldS_all = pad64((long long)B * l_s);
  w.ldS_tail = pad64((long long)B * cfg->s_queries[0]);
  w.ldN = pad64(B);
  auto feat = [&](size_t F, long long ldS) { return take(F * (size_t)ldS * es + L * F * (size_t)w.ldN * es); };
  w.xhT = feat(d, w.ldS_all);
  w.dkT = feat(d, w.ldS_all);
  w.dvT = feat(d, w.ldS_all);
  w.dqT = feat(d, w.ldS_all);
  w.oT = feat(d, w.ldS_tail);
  w.dyT = feat(d, w.ldS_tail);
  w.yhT = feat(d, w.ldS_tail);
  w.doutT = feat(d, w.ldS_tail);
  w.dhpreT = feat(dff, w.ldS_tail);
  w.hidT = feat(dff, w.ldS_tail);
  w.woT = take(G * d * d * es);
  w.w1T = take(G * d * dff * es);
  w.w2T = take(G * dff * d * es);
  w.wcT = take(G * d * 3 * d * es);
  // the weight-gradient launches' partials and the norms' column partials: the largest block
  long long part = 0, rsum = 0, tiles32 = 0;
  for (int n = 0; n < D.N; ++n) {
    const int s = block_s(cfg, l_s, n), q = cfg->s_queries[n];
    const long long ldA = pad64((long long)B * s), ldQ = pad64((long long)B * q);
    FeatBuf fd{nullptr, nullptr, ldA, w.ldN, D.d}, fq{nullptr, nullptr, ldQ, w.ldN, D.d},
        ff{nullptr, nullptr, ldQ, w.ldN, D.dff};
    GemmPlan P1, P2;
    plan_init(P1);
    plan_init(P2);
    float dummy;
    wgrad_jobs(P1, nullptr, D, fq, ff, (long long)B * q, B, WgradOut{&dummy, &dummy}, nullptr, nullptr);   // dW2
    wgrad_jobs(P1, nullptr, D, ff, fq, (long long)B * q, B, WgradOut{&dummy, &dummy}, nullptr, nullptr);   // dW1
    for (int i = 0; i < 3; ++i)
      wgrad_jobs(P2, nullptr, D, fd, fd, (long long)B * s, B, WgradOut{&dummy, nullptr}, nullptr, nullptr);
    wgrad_jobs(P2, nullptr, D, fq, fq, (long long)B * q, B, WgradOut{&dummy, nullptr}, nullptr, nullptr);   // dWo
    part = std::max({part, P1.part_elems, P2.part_elems});
    rsum = std::max({rsum, P1.rsum_elems, P2.rsum_elems});
    const long long t32 = ((long long)B * s + 31) / 32 + (long long)L * ((B + 31) / 32);
    tiles32 = std::max(tiles32, t32);
  }
  w.part = take((size_t)part * 4);
  w.rsum = take((size_t)rsum * 4);
  w.colpart = take((size_t)tiles32 * 2 * d * 4);
  w.colsum2 = take((size_t)((tiles32 + COLSUM_PER - 1) / COLSUM_PER) * 2 * d * 4);
  w.total = off;
  return w;
}

int check_grads(const onetrans_block_grads *g, const Dims &D) {
  if (!g) return ONETRANS_ERR_INVALID_ARG;
  for (int n = 0; n < D.N; ++n) {
    const float *req[] = {g[n].norm1_g, g[n].norm2_g, g[n].wq, g[n].wk, g[n].wv, g[n].wo, g[n].w1, g[n].b1, g[n].w2, g[n].b2};
    for (const float *p : req) {
      if (!p) return ONETRANS_ERR_INVALID_ARG;
      if (misaligned(p)) return ONETRANS_ERR_ALIGNMENT;
    }
    if (misaligned(g[n].norm1_b) || misaligned(g[n].norm2_b)) return ONETRANS_ERR_ALIGNMENT;
  }
  return ONETRANS_OK;
}

int train_run(const Dims &D, const onetrans_config *cfg, const onetrans_block_weights *blk, const void *x0, int B,
              int l_s, const float *d_out, float *out, float *dx0, const onetrans_block_grads *grads, char *w,
              const TrainWs &W, hipStream_t stream) {
  int rc;
  const int d = D.d, H = D.H, dh = D.dh, L = D.lns, dff = D.dff, N = D.N;
  const size_t es = D.esz;
  const int dt = D.dt;
  auto hip_ok = [](hipError_t e) { return e == hipSuccess; };

  // ---- forward, keeping block inputs ------------------------------------------------------------
  auto input_of = [&](int n, RowView &x, int &x_f32) {
    const int T = block_s(cfg, l_s, n) + L;
    if (n == 0) {
      x = RowView{const_cast<void *>(x0), (long long)(l_s + L) * d, 0, d};
      x_f32 = dt == ONETRANS_F32;
    } else {
      x = RowView{w + W.ckpt[n], (long long)T * d, 0, d};
      x_f32 = 1;
    }
  };
  auto step_for = [&](int n, bool post) {
    const int s = block_s(cfg, l_s, n), q = cfg->s_queries[n];
    const int T = s + L, R = q + L, p0 = s - q;
    Step st{};
    st.n_seq = B;
    st.s = s;
    st.q = q;
    st.kv_t0 = 0;
    st.kv_n = s;
    st.ns = L;
    st.in_t0 = 0;
    st.in_n = T;
    input_of(n, st.x, st.x_f32);
    st.kS = HeadView{w + W.fw.k, (long long)H * T * dh, (long long)T * dh, 0};
    st.vS = HeadView{w + W.fw.v, (long long)H * T * dh, (long long)T * dh, 0};
    st.kN = st.kS;
    st.vN = st.vS;
    st.n_pre = T;
    st.kp = w + W.fw.k;
    st.vp = w + W.fw.v;
    st.pre_sb = (long long)H * T * dh;
    st.pre_sh = (long long)T * dh;
    st.need_out = true;
    st.no_post = !post;
    if (post) st.out = RowView{n + 1 == N ? (void *)out : (void *)(w + W.ckpt[n + 1]), (long long)R * d, p0, d};
    else st.lse = (float *)(w + W.lse);
    return st;
  };
  for (int n = 0; n < N; ++n) {
    if (n + 1 == N && !out) break;   // the last block's output is not needed for the gradients
    const Step st = step_for(n, true);
    if ((rc = run_step(D, blk[n], st, w, W.fw, stream))) return rc;
  }

  // ---- backward -----------------------------------------------------------------------------------
  auto tm = [&](int cls, auto &&launch) { return hip_ok(timed(cls, stream, launch)); };
  for (int n = N - 1; n >= 0; --n) {
    const onetrans_block_weights &wt = blk[n];
    const onetrans_block_grads &gr = grads[n];
    const int s = block_s(cfg, l_s, n), q = cfg->s_queries[n];
    const int T = s + L, R = q + L, p0 = s - q;
    const long long ldA = pad64((long long)B * s), ldQ = pad64((long long)B * q), ldN = W.ldN;
    RowView xv;
    int x_f32;
    input_of(n, xv, x_f32);
    const RowBuf X{(char *)xv.base, x_f32 ? 4u : es, xv.sb, d, 0};
    // block-local buffers: tail rows [B][R][*] at positions p0.., all rows [B][T][*]
    auto tail = [&](size_t off, size_t esz, int width) { return RowBuf{w + off, esz, (long long)R * width, width, p0}; };
    const RowBuf Ob = tail(W.fw.o, es, d), Yb = tail(W.y, 4, d), YHb = tail(W.yh, es, d),
                 DHPb = tail(W.dhpre, es, dff), DYHb = tail(W.dyh, 4, d), DY32 = tail(W.dy32, 4, d),
                 DYt = tail(W.dyt, es, d), DOt = tail(W.dout_t, es, d), DOb = tail(W.d_o, es, d);
    const RowBuf DOUT32 = n == N - 1 ? RowBuf{(char *)d_out, 4, (long long)R * d, d, p0} : tail(W.dx32, 4, d);
    const RowBuf DQKV{w + W.dqkv, es, (long long)T * 3 * d, 3 * d, 0}, DXH{w + W.dxh, 4, (long long)T * d, d, 0};
    auto fb = [&](size_t off, int F, long long ldS_max, long long ldS) {
      return FeatBuf{w + off, w + off + (size_t)F * ldS_max * es, ldS, ldN, F};
    };
    const FeatBuf xhT = fb(W.xhT, d, W.ldS_all, ldA), dkT = fb(W.dkT, d, W.ldS_all, ldA),
                  dvT = fb(W.dvT, d, W.ldS_all, ldA), dqT = fb(W.dqT, d, W.ldS_all, ldA),
                  oT = fb(W.oT, d, W.ldS_tail, ldQ), dyT = fb(W.dyT, d, W.ldS_tail, ldQ),
                  yhT = fb(W.yhT, d, W.ldS_tail, ldQ), doutT = fb(W.doutT, d, W.ldS_tail, ldQ),
                  dhpT = fb(W.dhpreT, dff, W.ldS_tail, ldQ), hidT = fb(W.hidT, dff, W.ldS_tail, ldQ);
    // the next lower block's d_out^T: this block's all-rows layout
    const FeatBuf doutT_next = fb(W.doutT, d, W.ldS_tail, ldA);

    // zero the padding columns of this block's feature-major buffers, and dQ of the rows before p0
    {
      FillArgs fa;
      memset(&fa, 0, sizeof(fa));
      bool full = false;
      auto add = [&](void *base, long long g, long long ld, int groups, int rows, long long c0, long long c1) {
        if (c1 <= c0 || rows == 0 || groups == 0) return;
        if (fa.n_jobs == FILL_MAX_JOBS) {
          full = true;
          return;
        }
        FillJob &j = fa.job[fa.n_jobs++];
        j = FillJob{base, g, ld, groups, rows, (int)c0, (int)c1, (int)es, fa.total};
        fa.total += (long long)groups * rows;
      };
      auto pads = [&](const FeatBuf &f, long long tok) {
        add(f.S, 0, f.ldS, 1, f.F, tok, f.ldS);
        add(f.N, (long long)f.F * f.ldN, f.ldN, L, f.F, B, f.ldN);
      };
      pads(xhT, (long long)B * s);
      pads(dkT, (long long)B * s);
      pads(dvT, (long long)B * s);
      pads(dqT, (long long)B * s);
      for (const FeatBuf *f : {&oT, &dyT, &yhT, &doutT, &dhpT, &hidT}) pads(*f, (long long)B * q);
      if (full) return ONETRANS_ERR_SHAPE;   // (not reached: 20 regions at most)
      if (!tm(ONETRANS_K_BWD_ROWS, [&] { return launch_fill(fa, stream); })) return ONETRANS_ERR_HIP;
    }
    // transposed weights: Wo^T, W1^T, W2^T and [Wk^T | Wv^T | Wq^T]
    {
      TrArgs ta;
      memset(&ta, 0, sizeof(ta));
      int tiles = 0;
      const int G = 1 + L;
      auto add = [&](const void *src, size_t dst_off, int rows, int cols, int dst_ld, int dst_off_col) {
        TrJob &j = ta.job[ta.n_jobs++];
        j = TrJob{src, w + dst_off, rows, cols, G, (long long)rows * cols, (long long)cols * dst_ld, dst_ld, dst_off_col, tiles};
        tiles += G * ((rows + 31) / 32) * ((cols + 31) / 32);
      };
      add(wt.wo, W.woT, d, d, d, 0);
      add(wt.w1, W.w1T, dff, d, dff, 0);
      add(wt.w2, W.w2T, d, dff, d, 0);
      add(wt.wk, W.wcT, d, d, 3 * d, 0);
      add(wt.wv, W.wcT, d, d, 3 * d, d);
      add(wt.wq, W.wcT, d, d, 3 * d, 2 * d);
      if (!tm(ONETRANS_K_BWD_ROWS, [&] { return launch_transpose(dt, ta, tiles, stream); })) return ONETRANS_ERR_HIP;
    }
    const WBuf Wo{(const char *)wt.wo, es, (long long)d * d, d}, W1{(const char *)wt.w1, es, (long long)dff * d, d},
        WoT{w + W.woT, es, (long long)d * d, d}, W1T{w + W.w1T, es, (long long)d * dff, dff},
        W2T{w + W.w2T, es, (long long)dff * d, d}, WcT{w + W.wcT, es, (long long)d * 3 * d, 3 * d};

    // rows launch over the S rows [t0, t0 + cnt) and the NS rows of every sample
    auto rows_launch = [&](RowsArgs ra, int t0, int cnt, const FeatBuf *outT) {
      long long tiles = 0;
      ra.n_jobs = 0;
      auto add = [&](RowSet rs, void *ot, long long g, long long ld) {
        const long long m = (long long)rs.n_seq * rs.rows;
        if (m == 0 || rs.n_groups == 0) return;
        RowsJob &j = ra.job[ra.n_jobs++];
        j.rs = rs;
        j.m_tiles = (int)((m + 31) / 32);
        j.tile0 = (int)tiles;
        j.outT = ot;
        j.tr_g = g;
        j.tr_ld = ld;
        tiles += (long long)j.m_tiles * rs.n_groups;
      };
      add(RowSet{B, cnt, 1, t0, 0, 0}, outT ? outT->S : nullptr, 0, outT ? outT->ldS : 0);
      add(RowSet{B, 1, L, s, 1, 1}, outT ? outT->N : nullptr, outT ? (long long)outT->F * outT->ldN : 0, outT ? outT->ldN : 0);
      ra.d = d;
      ra.layer = D.layer;
      ra.eps = D.eps;
      ra.n_heads = H;
      if (!tm(ONETRANS_K_BWD_ROWS, [&] { return launch_rows(dt, ra, (int)tiles, stream); })) return -1LL;
      return tiles;
    };
    // mixed product over the S rows [t0, t0 + cnt) (set 0) and the NS rows (sets 1..l_ns)
    // pre (EPI_DGELU): the pre-activation's operands, rows of pre->first times pre->second (k = d)
    auto act_gemm = [&](const RowBuf &A, const WBuf &Wb, int n_feat, int k_len, int t0, int cnt, int epi,
                        const void *bias, const RowBuf *resid, const std::pair<const RowBuf *, const WBuf *> *pre,
                        const RowBuf *outb, bool out_f32, const FeatBuf *outT) {
      GemmPlan P;
      plan_init(P);
      for (int ns = 0; ns < 2; ++ns) {
        GemmJob j;
        memset(&j, 0, sizeof(j));
        j.a = ns ? rows_N(A, s) : rows_S(A, t0, cnt);
        j.b = w_set(Wb, ns);
        j.m = ns ? B : B * cnt;
        j.n_feat = n_feat;
        j.k_len = k_len;
        j.n_groups = ns ? L : 1;
        j.n_split = 1;
        j.epi = epi;
        if (bias) {
          j.bias = (const char *)bias + (ns ? (long long)n_feat * es : 0);
          j.bias_g = n_feat;
        }
        if (resid) {
          j.resid = ns ? rows_N(*resid, s) : rows_S(*resid, t0, cnt);
          j.resid_f32 = resid->esz == 4;
        }
        if (pre) {
          j.a2 = ns ? rows_N(*pre->first, s) : rows_S(*pre->first, t0, cnt);
          j.b2 = w_set(*pre->second, ns);
          j.k_len2 = d;
        }
        if (outb) {
          j.out = ns ? rows_N(*outb, s) : rows_S(*outb, t0, cnt);
          j.out_f32 = out_f32;
        }
        if (outT) j.outT = ns ? featT_N(*outT) : featT_S(*outT);
        plan_add(P, j);
      }
      return tm(ONETRANS_K_BWD_GEMM, [&] { return launch_gemm(dt, P.a, (int)P.tiles, stream); });
    };

    // ---- recompute ----
    {   // xh^T = Norm1(X) over all rows
      RowsArgs ra;
      memset(&ra, 0, sizeof(ra));
      ra.mode = ROWS_NORM_FWD;
      ra.x = view(X);
      ra.x_f32 = x_f32;
      ra.gamma = wt.norm1_g;
      ra.beta = wt.norm1_b;
      if (rows_launch(ra, 0, s, &xhT) < 0) return ONETRANS_ERR_HIP;
    }
    {   // Q/K/V and O (with the log-sum-exp) by the forward's kernels
      const Step st = step_for(n, false);
      if ((rc = run_step(D, wt, st, w, W.fw, stream))) return rc;
    }
    // Y = X[tail] + O Wo^T (fp32)
    if (!act_gemm(Ob, Wo, d, d, p0, q, EPI_STORE, nullptr, &X, nullptr, &Yb, true, nullptr)) return ONETRANS_ERR_HIP;
    {   // yh = Norm2(Y): rows and feature-major
      RowsArgs ra;
      memset(&ra, 0, sizeof(ra));
      ra.mode = ROWS_NORM_FWD;
      ra.x = view(Yb);
      ra.x_f32 = 1;
      ra.gamma = wt.norm2_g;
      ra.beta = wt.norm2_b;
      ra.out_t = view(YHb);
      if (rows_launch(ra, p0, q, &yhT) < 0) return ONETRANS_ERR_HIP;
    }
    // hid^T = GELU(yh W1^T + b1) (feature-major only: the backward forms the pre-activation again)
    if (!act_gemm(YHb, W1, dff, d, p0, q, EPI_GELU, wt.b1, nullptr, nullptr, nullptr, false, &hidT)) return ONETRANS_ERR_HIP;

    // ---- backward ----
    if (n == N - 1) {   // the caller's d_out: storage-dtype rows and feature-major copy
      RowsArgs ra;
      memset(&ra, 0, sizeof(ra));
      ra.mode = ROWS_CONVERT;
      ra.x = view(DOUT32);
      ra.x_f32 = 1;
      ra.out_t = view(DOt);
      if (rows_launch(ra, p0, q, &doutT) < 0) return ONETRANS_ERR_HIP;
    }
    // dhpre = (dOut W2) * GELU'(yh W1^T + b1), the pre-activation formed in registers: rows and
    // feature-major
    {
      const std::pair<const RowBuf *, const WBuf *> pre{&YHb, &W1};
      if (!act_gemm(DOt, W2T, dff, d, p0, q, EPI_DGELU, wt.b1, nullptr, &pre, &DHPb, false, &dhpT)) return ONETRANS_ERR_HIP;
    }
    {   // dW2, db2, dW1, db1
      GemmPlan P;
      plan_init(P);
      RedArgs ra;
      memset(&ra, 0, sizeof(ra));
      float *part = (float *)(w + W.part), *rsum = (float *)(w + W.rsum);
      wgrad_jobs(P, &ra, D, doutT, hidT, (long long)B * q, B, WgradOut{gr.w2, gr.b2}, part, rsum);
      wgrad_jobs(P, &ra, D, dhpT, yhT, (long long)B * q, B, WgradOut{gr.w1, gr.b1}, part, rsum);
      if (!tm(ONETRANS_K_BWD_GEMM, [&] { return launch_gemm(dt, P.a, (int)P.tiles, stream); })) return ONETRANS_ERR_HIP;
      if (!tm(ONETRANS_K_BWD_GEMM, [&] { return launch_reduce(ra, stream); })) return ONETRANS_ERR_HIP;
    }
    // dYh = dhpre W1 (fp32)
    if (!act_gemm(DHPb, W1T, d, dff, p0, q, EPI_STORE, nullptr, nullptr, nullptr, &DYHb, true, nullptr)) return ONETRANS_ERR_HIP;
    {   // dY = Norm2'(dYh) + dOut: fp32 rows, storage rows, feature-major; dg2 / db2 column partials
      RowsArgs ra;
      memset(&ra, 0, sizeof(ra));
      ra.mode = ROWS_NORM_BWD;
      ra.x = view(Yb);
      ra.x_f32 = 1;
      ra.dy = view(DYHb);
      ra.res = view(DOUT32);
      ra.res_from = 0;
      ra.gamma = wt.norm2_g;
      ra.beta = wt.norm2_b;
      ra.out_f32 = view(DY32);
      ra.out_t = view(DYt);
      ra.colpart = (float *)(w + W.colpart);
      const long long tiles = rows_launch(ra, p0, q, &dyT);
      if (tiles < 0) return ONETRANS_ERR_HIP;
      if (!tm(ONETRANS_K_BWD_ROWS, [&] {
            return launch_colsum(ra.colpart, (int)tiles, d, gr.norm2_g, D.layer ? gr.norm2_b : nullptr,
                                 (float *)(w + W.colsum2), stream);
          }))
        return ONETRANS_ERR_HIP;
    }
    // dO = dY Wo (storage rows)
    if (!act_gemm(DYt, WoT, d, d, p0, q, EPI_STORE, nullptr, nullptr, nullptr, &DOb, false, nullptr)) return ONETRANS_ERR_HIP;
    {   // D = rowsum(dO * O) per head, and O^T
      RowsArgs ra;
      memset(&ra, 0, sizeof(ra));
      ra.mode = ROWS_DOT;
      ra.x = view(Ob);
      ra.x_f32 = 0;
      ra.dy = view(DOb);
      ra.dvec = (float *)(w + W.dvec);
      ra.d_sb = (long long)H * R;
      ra.d_R = R;
      ra.d_p0 = p0;
      if (dt == ONETRANS_F32) ra.x_f32 = 1;
      if (rows_launch(ra, p0, q, &oT) < 0) return ONETRANS_ERR_HIP;
    }
    {   // attention backward
      AttnBwdArgs a;
      memset(&a, 0, sizeof(a));
      a.n_seq = B;
      a.n_heads = H;
      a.d_model = d;
      a.T = T;
      a.s = s;
      a.R = R;
      a.p0 = p0;
      a.q = w + W.fw.q;
      a.q_sb = (long long)H * R * dh;
      a.k = w + W.fw.k;
      a.v = w + W.fw.v;
      a.kv_sb = (long long)H * T * dh;
      a.dout = w + W.d_o;
      a.lse = (const float *)(w + W.lse);
      a.dvec = (const float *)(w + W.dvec);
      a.dqkv = w + W.dqkv;
      const FeatBuf *tf[3] = {&dkT, &dvT, &dqT};
      for (int i = 0; i < 3; ++i) {
        a.tS[i] = tf[i]->S;
        a.tN[i] = tf[i]->N;
      }
      a.tS_ld = ldA;
      a.tN_g = (long long)d * ldN;
      a.tN_ld = ldN;
      a.n_kblocks = (T + 32 * ATTB_WAVES - 1) / (32 * ATTB_WAVES);
      a.n_qblocks = (R + 32 * ATTB_WAVES - 1) / (32 * ATTB_WAVES);
      if (!tm(ONETRANS_K_BWD_ATTN, [&] { return launch_attn_bwd(dt, dh, a, stream); })) return ONETRANS_ERR_HIP;
    }
    {   // dWq, dWk, dWv (over every S row; dQ is zero before p0) and dWo
      GemmPlan P;
      plan_init(P);
      RedArgs ra;
      memset(&ra, 0, sizeof(ra));
      float *part = (float *)(w + W.part);
      wgrad_jobs(P, &ra, D, dqT, xhT, (long long)B * s, B, WgradOut{gr.wq, nullptr}, part, nullptr);
      wgrad_jobs(P, &ra, D, dkT, xhT, (long long)B * s, B, WgradOut{gr.wk, nullptr}, part, nullptr);
      wgrad_jobs(P, &ra, D, dvT, xhT, (long long)B * s, B, WgradOut{gr.wv, nullptr}, part, nullptr);
      wgrad_jobs(P, &ra, D, dyT, oT, (long long)B * q, B, WgradOut{gr.wo, nullptr}, part, nullptr);
      if (!tm(ONETRANS_K_BWD_GEMM, [&] { return launch_gemm(dt, P.a, (int)P.tiles, stream); })) return ONETRANS_ERR_HIP;
      if (!tm(ONETRANS_K_BWD_GEMM, [&] { return launch_reduce(ra, stream); })) return ONETRANS_ERR_HIP;
    }
    // dXh = [dK | dV | dQ] [Wk; Wv; Wq] over all rows (fp32); the S rows before p0 issue no query,
    // so their contraction stops after [dK | dV] (their dQ columns are never written)
    {
      GemmPlan P;
      plan_init(P);
      for (int part = 0; part < 3; ++part) {
        GemmJob j;
        memset(&j, 0, sizeof(j));
        const bool ns = part == 2;
        const int t0 = part == 0 ? 0 : p0, cnt = part == 0 ? p0 : q;
        j.a = ns ? rows_N(DQKV, s) : rows_S(DQKV, t0, cnt);
        j.b = w_set(WcT, ns);
        j.m = ns ? B : B * cnt;
        j.n_feat = d;
        j.k_len = part == 0 ? 2 * d : 3 * d;
        j.n_groups = ns ? L : 1;
        j.n_split = 1;
        j.epi = EPI_STORE;
        j.out = ns ? rows_N(DXH, s) : rows_S(DXH, t0, cnt);
        j.out_f32 = 1;
        plan_add(P, j);
      }
      if (!tm(ONETRANS_K_BWD_GEMM, [&] { return launch_gemm(dt, P.a, (int)P.tiles, stream); })) return ONETRANS_ERR_HIP;
    }
    {   // dX = Norm1'(dXh) + dY on the tail rows: the lower block's d_out (fp32 rows, storage rows,
        // feature-major), or dX(0); dg1 / db1 column partials
      RowsArgs ra;
      memset(&ra, 0, sizeof(ra));
      ra.mode = ROWS_NORM_BWD;
      ra.x = view(X);
      ra.x_f32 = x_f32;
      ra.dy = view(DXH);
      ra.res = view(DY32);
      ra.res_from = p0;
      ra.gamma = wt.norm1_g;
      ra.beta = wt.norm1_b;
      ra.colpart = (float *)(w + W.colpart);
      const FeatBuf *ot = nullptr;
      if (n > 0) {
        ra.out_f32 = RowView{w + W.dx32, (long long)T * d, 0, d};
        ra.out_t = RowView{w + W.dout_t, (long long)T * d, 0, d};
        ot = &doutT_next;
      } else if (dx0) {
        ra.out_f32 = RowView{dx0, (long long)T * d, 0, d};
      }
      const long long tiles = rows_launch(ra, 0, s, ot);
      if (tiles < 0) return ONETRANS_ERR_HIP;
      if (!tm(ONETRANS_K_BWD_ROWS, [&] {
            return launch_colsum(ra.colpart, (int)tiles, d, gr.norm1_g, D.layer ? gr.norm1_b : nullptr,
                                 (float *)(w + W.colsum2), stream);
          }))
        return ONETRANS_ERR_HIP;
    }
    if (!D.layer) {   // RMSNorm has no shift: its gradient slots, when given, are zero
      FillArgs fa;
      memset(&fa, 0, sizeof(fa));
      for (float *p : {gr.norm1_b, gr.norm2_b})
        if (p) {
          FillJob &j = fa.job[fa.n_jobs++];
          j = FillJob{p, 0, d, 1, 1, 0, d, 4, fa.total};
          fa.total += 1;
        }
      if (fa.n_jobs && !tm(ONETRANS_K_BWD_ROWS, [&] { return launch_fill(fa, stream); })) return ONETRANS_ERR_HIP;
    }
  }
  return ONETRANS_OK;
}

}  // namespace

extern "C" {

size_t onetrans_workspace_bytes(const onetrans_config *cfg, int op, int n_seq, int l_s, int n_cand, int d_l) {
  Dims D;
  if (check_cfg(cfg, D)) return 0;
  if (op == ONETRANS_OP_APPEND_SCORE) {   // the append's workspace, then Stage II's
    const size_t wa = onetrans_workspace_bytes(cfg, ONETRANS_OP_APPEND, n_seq, 0, 0, d_l);
    const size_t wb = onetrans_workspace_bytes(cfg, ONETRANS_OP_SCORE, n_seq, 0, n_cand, 0);
    return wa && wb ? al(wa) + wb : 0;
  }
  size_t n, tin, rq;
  bool kv;
  if (!ws_dims(cfg, D, op, n_seq, l_s, n_cand, d_l, n, tin, rq, kv)) return 0;
  if ((op == ONETRANS_OP_FORWARD || op == ONETRANS_OP_PREFILL) && check_schedule(cfg, l_s)) return 0;
  const int parts = ws_parts_for(n_seq, op == ONETRANS_OP_FORWARD ? FORWARD_PART_MIN : USER_PART_MIN);
  const size_t per = op == ONETRANS_OP_SCORE ? (size_t)n_cand : 1;   // sequences per user
  return ws_layout(D, (size_t)((n_seq + parts - 1) / parts) * per, tin, rq, kv, (size_t)n_seq * per, true).total *
         parts;
}

size_t onetrans_backward_workspace_bytes(const onetrans_config *cfg, int batch, int l_s) {
  Dims D;
  if (check_cfg(cfg, D) || batch < 1 || l_s < 1 || check_schedule(cfg, l_s)) return 0;
  return train_layout(D, cfg, batch, l_s).total;
}

int onetrans_backward(const onetrans_config *cfg, const onetrans_block_weights *blk, const void *x0, int batch,
                      int l_s, const float *d_out, float *out, float *dx0, const onetrans_block_grads *grads,
                      void *ws, size_t ws_bytes, hipStream_t stream) {
  Dims D;
  int rc;
  if ((rc = check_cfg(cfg, D))) return rc;
  if (batch < 1 || l_s < 1) return ONETRANS_ERR_SHAPE;
  if ((rc = check_schedule(cfg, l_s))) return rc;
  if ((rc = check_weights(blk, D))) return rc;
  if ((rc = check_grads(grads, D))) return rc;
  if (!x0 || !d_out || !ws) return ONETRANS_ERR_INVALID_ARG;
  if (misaligned(x0) || misaligned(d_out) || misaligned(out) || misaligned(dx0) || misaligned(ws))
    return ONETRANS_ERR_ALIGNMENT;
  if ((rc = check_size(D, batch, (long long)l_s + D.lns))) return rc;
  // a weight-gradient tile spans 128 feature-major rows of every token of a set: byte offsets
  // within it are 32-bit
  if (128LL * pad64((long long)batch * l_s) * 4 >= (1LL << 32)) return ONETRANS_ERR_SHAPE;
  const TrainWs W = train_layout(D, cfg, batch, l_s);
  if (ws_bytes < W.total) return ONETRANS_ERR_WORKSPACE;
  return train_run(D, cfg, blk, x0, batch, l_s, d_out, out, dx0, grads, (char *)ws, W, stream);
}

size_t onetrans_kv_cache_bytes(const onetrans_config *cfg, int n_users, int capacity) {
  Dims D;
  if (check_cfg(cfg, D) || n_users < 1 || capacity < 1) return 0;
  return (size_t)n_users * D.N * D.H * (size_t)capacity * D.dh * D.esz;
}

int onetrans_forward(const onetrans_config *cfg, const onetrans_block_weights *blk, const void *x0, int batch,
                     int l_s, void *out, void *ws, size_t ws_bytes, hipStream_t stream) {
  Dims D;
  int rc;
  if ((rc = check_cfg(cfg, D))) return rc;
  if (batch < 1 || l_s < 1) return ONETRANS_ERR_SHAPE;
  if ((rc = check_schedule(cfg, l_s))) return rc;
  if ((rc = check_weights(blk, D))) return rc;
  if (!x0 || !out) return ONETRANS_ERR_INVALID_ARG;
  if (misaligned(x0) || misaligned(out)) return ONETRANS_ERR_ALIGNMENT;
  if ((rc = check_size(D, batch, (long long)l_s + D.lns))) return rc;
  size_t n, tin, rq;
  bool kv;
  ws_dims(cfg, D, ONETRANS_OP_FORWARD, batch, l_s, 0, 0, n, tin, rq, kv);
  const int wp = ws_parts_for(batch, FORWARD_PART_MIN), parts = parts_for(batch, FORWARD_PART_MIN);
  if (misaligned(ws)) return ONETRANS_ERR_ALIGNMENT;
  if (!ws) return ONETRANS_ERR_INVALID_ARG;
  if (ws_bytes < ws_layout(D, (batch + wp - 1) / wp, tin, rq, kv, batch, true).total * wp) return ONETRANS_ERR_WORKSPACE;
  const size_t part_bytes = ws_layout(D, (batch + parts - 1) / parts, tin, rq, kv, batch, true).total;
  const size_t in_row = (size_t)(l_s + D.lns) * D.d * D.esz;
  const size_t out_row = (size_t)(cfg->s_queries[D.N - 1] + D.lns) * D.d * 4;
  return over_streams(batch, parts, stream, [&](int first, int count, int part, hipStream_t st) {
    return forward_run(D, cfg, blk, (const char *)x0 + first * in_row, count, l_s, (char *)out + first * out_row,
                       (char *)ws + part * part_bytes, ws_layout(D, count, tin, rq, kv, batch, true), st);
  });
}

int onetrans_prefill_user(const onetrans_config *cfg, const onetrans_block_weights *blk, const void *x_s,
                          int n_users, int l_s, onetrans_kv_cache *cache, void *out_s, void *ws, size_t ws_bytes,
                          hipStream_t stream) {
  Dims D;
  int rc;
  if ((rc = check_cfg(cfg, D))) return rc;
  if (n_users < 1 || l_s < 1) return ONETRANS_ERR_SHAPE;
  if ((rc = check_schedule(cfg, l_s))) return rc;
  if ((rc = check_weights(blk, D))) return rc;
  if (!x_s) return ONETRANS_ERR_INVALID_ARG;
  if (misaligned(x_s) || (out_s && misaligned(out_s))) return ONETRANS_ERR_ALIGNMENT;
  if ((rc = check_cache(cache))) return rc;
  if (n_users > cache->n_users || l_s > cache->capacity) return ONETRANS_ERR_CACHE_CAPACITY;
  if ((rc = check_size(D, n_users, l_s))) return rc;
  if (cache->user_len) {
    // ragged users: padding rows behind each user's sequence are only harmless without pruning
    for (int n = 0; n < D.N; ++n)
      if (cfg->s_queries[n] != l_s) return ONETRANS_ERR_UNSUPPORTED;
    if ((rc = check_user_len(cache, n_users, l_s))) return rc;
  }
  size_t n, tin, rq;
  bool kv;
  ws_dims(cfg, D, ONETRANS_OP_PREFILL, n_users, l_s, 0, 0, n, tin, rq, kv);
  const int wp = ws_parts_for(n_users, USER_PART_MIN), parts = parts_for(n_users, USER_PART_MIN);
  if (misaligned(ws)) return ONETRANS_ERR_ALIGNMENT;
  if (!ws) return ONETRANS_ERR_INVALID_ARG;
  if (ws_bytes < ws_layout(D, (n_users + wp - 1) / wp, tin, rq, kv, n_users, true).total * wp)
    return ONETRANS_ERR_WORKSPACE;
  const size_t part_bytes = ws_layout(D, (n_users + parts - 1) / parts, tin, rq, kv, n_users, true).total;
  const size_t in_user = (size_t)l_s * D.d * D.esz, out_user = (size_t)cfg->s_queries[D.N - 1] * D.d * 4;
  // the first pruning block's kept rows go to x_tail too (when a later block exists to read them)
  const int n_star = first_pruning_block(cfg->s_queries, D.N, l_s);
  const int tail_block = cache->x_tail && n_star >= 0 && n_star < D.N - 1 ? n_star : -1;
  rc = over_streams(n_users, parts, stream, [&](int first, int count, int part, hipStream_t st) {
    const onetrans_kv_cache view = user_view(D, cache, first);
    RowView x{const_cast<char *>((const char *)x_s + first * in_user), (long long)l_s * D.d, 0, D.d};
    return stack_run(D, blk, x, D.dt == ONETRANS_F32, l_s, count, &view, 0, cfg->s_queries, cfg->s_queries[D.N - 1],
                     tail_block, out_s ? (char *)out_s + first * out_user : nullptr, (char *)ws + part * part_bytes,
                     ws_layout(D, count, tin, rq, kv, n_users, true), st);
  });
  if (rc) return rc;
  int s = l_s;
  for (int n = 0; n < D.N; ++n) {
    cache->layer_len[n] = s;
    s = cfg->s_queries[n];
  }
  cache->q_last = cfg->s_queries[D.N - 1];
  return ONETRANS_OK;
}

int onetrans_score_candidates(const onetrans_config *cfg, const onetrans_block_weights *blk,
                              const onetrans_kv_cache *cache, const void *x_ns, int n_users, int n_cand,
                              void *out_ns, void *ws, size_t ws_bytes, hipStream_t stream) {
  Dims D;
  int rc;
  if ((rc = check_score(cfg, blk, cache, x_ns, n_users, n_cand, out_ns, D))) return rc;
  size_t n, tin, rq;
  bool kv;
  ws_dims(cfg, D, ONETRANS_OP_SCORE, n_users, 0, n_cand, 0, n, tin, rq, kv);
  const int wp = ws_parts_for(n_users, USER_PART_MIN), parts = parts_for(n_users, USER_PART_MIN);
  if (misaligned(ws)) return ONETRANS_ERR_ALIGNMENT;
  if (!ws) return ONETRANS_ERR_INVALID_ARG;
  const size_t n_call = (size_t)n_users * n_cand;
  if (ws_bytes < ws_layout(D, (size_t)((n_users + wp - 1) / wp) * n_cand, tin, rq, kv, n_call, true).total * wp)
    return ONETRANS_ERR_WORKSPACE;
  const size_t part_bytes =
      ws_layout(D, (size_t)((n_users + parts - 1) / parts) * n_cand, tin, rq, kv, n_call, true).total;
  const size_t in_user = (size_t)n_cand * D.lns * D.d * D.esz, out_user = (size_t)n_cand * D.lns * D.d * 4;
  return over_streams(n_users, parts, stream, [&](int first, int count, int part, hipStream_t st) {
    const onetrans_kv_cache view = user_view(D, cache, first);
    return score_run(D, blk, &view, (const char *)x_ns + first * in_user, count, n_cand,
                     (char *)out_ns + first * out_user, (char *)ws + part * part_bytes,
                     ws_layout(D, (size_t)count * n_cand, tin, rq, kv, n_call, true), st);
  });
}

int onetrans_score_candidates_noalloc(const onetrans_config *cfg, const onetrans_block_weights *blk,
                                      const onetrans_kv_cache *cache, const void *x_ns, int n_users, int n_cand,
                                      void *out_ns, hipStream_t stream) {
  Dims D;
  int rc;
  if ((rc = check_score(cfg, blk, cache, x_ns, n_users, n_cand, out_ns, D))) return rc;
  // one part on the caller's stream: the whole call's workspace in the scratch
  size_t n, tin, rq;
  bool kv;
  ws_dims(cfg, D, ONETRANS_OP_SCORE, n_users, 0, n_cand, 0, n, tin, rq, kv);
  const Ws L = ws_layout(D, n, tin, rq, kv, n, true);
  if (L.total > (size_t)ONETRANS_SCRATCH_BYTES) return ONETRANS_ERR_SCRATCH;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ONETRANS_ERR_HIP;
  if (stream) {
    hipDevice_t sdev = 0;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return ONETRANS_ERR_HIP;
    if ((int)sdev != dev) return ONETRANS_ERR_INVALID_ARG;   // the scratch address is per device
  }
  void *w = nullptr;
  if ((rc = scratch_ptr(dev, w))) return rc;
  t_untimed = true;
  rc = score_run(D, blk, cache, x_ns, n_users, n_cand, out_ns, (char *)w, L, stream);
  t_untimed = false;
  return rc;
}

int onetrans_append_events(const onetrans_config *cfg, const onetrans_block_weights *blk, onetrans_kv_cache *cache,
                           const void *x_new, int n_users, int d_l, void *out_new, void *ws, size_t ws_bytes,
                           hipStream_t stream) {
  Dims D;
  int rc;
  if ((rc = check_cfg(cfg, D))) return rc;
  if (n_users < 1 || d_l < 1) return ONETRANS_ERR_SHAPE;
  if ((rc = check_weights(blk, D))) return rc;
  if (!x_new) return ONETRANS_ERR_INVALID_ARG;
  if (misaligned(x_new) || (out_new && misaligned(out_new))) return ONETRANS_ERR_ALIGNMENT;
  if ((rc = check_cache(cache))) return rc;
  if (n_users > cache->n_users) return ONETRANS_ERR_SHAPE;
  for (int n = 0; n < D.N; ++n)
    if (cache->layer_len[n] < 0 || cache->layer_len[n] > cache->capacity) return ONETRANS_ERR_SHAPE;
  // the cache's pyramid: block n has s_n = layer_len[n] rows and keeps q_n = layer_len[n + 1]
  // (the last block: q_last); n_star = the first block that prunes
  const int q_last = cache->q_last > 0 ? cache->q_last : cache->layer_len[D.N - 1];
  int n_star = -1;
  for (int n = 0; n < D.N; ++n) {
    const int qn = n + 1 < D.N ? cache->layer_len[n + 1] : q_last;
    if (qn > cache->layer_len[n]) return ONETRANS_ERR_SHAPE;   // no pyramid grows
    if (qn < cache->layer_len[n] && n_star < 0) n_star = n;
  }
  const bool ragged = cache->user_len != nullptr;
  const bool recompute = n_star >= 0 && n_star < D.N - 1;   // blocks n_star + 1 .. run again
  if (ragged && n_star >= 0) return ONETRANS_ERR_UNSUPPORTED;
  if (recompute && !cache->x_tail) return ONETRANS_ERR_INVALID_ARG;
  if (ragged) {
    if ((rc = check_user_len(cache, n_users, cache->capacity))) return rc;
    for (int u = 0; u < n_users; ++u)
      if ((long long)cache->user_len[u] + d_l > cache->capacity) return ONETRANS_ERR_CACHE_CAPACITY;
  } else if ((long long)cache->layer_len[0] + d_l > cache->capacity) {
    return ONETRANS_ERR_CACHE_CAPACITY;
  }
  const int window = recompute ? cache->layer_len[n_star + 1] : 0;   // rows of block n_star + 1
  if ((rc = check_size(D, n_users, std::max(d_l, window)))) return rc;
  size_t n, tin, rq;
  bool kv;
  ws_dims(cfg, D, ONETRANS_OP_APPEND, n_users, window, 0, d_l, n, tin, rq, kv);
  const int wp = ws_parts_for(n_users, USER_PART_MIN), parts = parts_for(n_users, USER_PART_MIN);
  if (misaligned(ws)) return ONETRANS_ERR_ALIGNMENT;
  if (!ws) return ONETRANS_ERR_INVALID_ARG;
  if (ws_bytes < ws_layout(D, (n_users + wp - 1) / wp, tin, rq, kv, n_users, true).total * wp)
    return ONETRANS_ERR_WORKSPACE;
  const int l_old = ragged ? 0 : cache->layer_len[0];
  const int l_new = l_old + d_l;
  // the last block's kept rows after the append: it grows with the sequence unless it prunes
  const bool last_prunes = n_star >= 0;    // n_star <= N - 1: the last block keeps a fixed count
  const int q_last_new = last_prunes ? q_last : q_last + d_l;
  const int q_final = std::min(d_l, q_last_new);   // final rows of the new events
  const int n_head = recompute ? n_star + 1 : D.N;
  // the recomputed blocks' schedule: block n keeps layer_len[n + 1] rows
  std::vector<int> q_of(D.N);
  for (int b = 0; b + 1 < D.N; ++b) q_of[b] = cache->layer_len[b + 1];
  q_of[D.N - 1] = q_last;
  const size_t part_bytes = ws_layout(D, (n_users + parts - 1) / parts, tin, rq, kv, n_users, true).total;
  const size_t in_user = (size_t)d_l * D.d * D.esz, out_user = (size_t)q_final * D.d * 4;
  rc = over_streams(n_users, parts, stream, [&](int first, int count, int part, hipStream_t st) {
    const onetrans_kv_cache view = user_view(D, cache, first);
    char *w = (char *)ws + part * part_bytes;
    const Ws Lp = ws_layout(D, count, tin, rq, kv, n_users, true);
    void *out = out_new ? (char *)out_new + first * out_user : nullptr;
    int r = append_run(D, blk, &view, (const char *)x_new + first * in_user, count, d_l, out, w, Lp, l_old, n_head,
                       q_final, st);
    if (r || !recompute) return r;
    // blocks n_star + 1 .. over their slid windows: block n_star + 1 reads the last `window` rows of
    // the sequence from x_tail (the old rows written by prefill, the new ones by the blocks above)
    return stack_run(D, blk, tail_rows(D, &view, -(l_new - window)), 1, window, count, &view, n_star + 1, q_of.data(),
                     q_final, -1, out, w, Lp, st);
  });
  if (rc) return rc;
  if (ragged) {
    int longest = 0;
    for (int u = 0; u < n_users; ++u) longest = max(longest, cache->user_len[u] += d_l);
    for (int b = 0; b < D.N; ++b) cache->layer_len[b] = max(cache->layer_len[b], longest);
    cache->q_last = cache->layer_len[D.N - 1];
  } else {
    for (int b = 0; b < n_head; ++b) cache->layer_len[b] = l_new;
    cache->q_last = q_last_new;
  }
  return ONETRANS_OK;
}

int onetrans_append_score(const onetrans_config *cfg, const onetrans_block_weights *blk, onetrans_kv_cache *cache,
                          const void *x_new, int n_users, int d_l, void *out_new, const void *x_ns, int n_cand,
                          void *out_ns, void *ws, size_t ws_bytes, hipStream_t stream) {
  Dims D;
  int rc;
  if ((rc = check_score(cfg, blk, cache, x_ns, n_users, n_cand, out_ns, D))) return rc;
  if (d_l < 1) return ONETRANS_ERR_SHAPE;
  if (!x_new || !out_new) return ONETRANS_ERR_INVALID_ARG;
  if (misaligned(x_new) || misaligned(out_new)) return ONETRANS_ERR_ALIGNMENT;
  // one pass over a user's keys for both query sets: at most 32 appended rows and 32 NS rows per
  // user, and an unpyramided cache (every block holds the whole sequence)
  if (d_l > 32 || (long long)n_cand * D.lns > 32) return ONETRANS_ERR_UNSUPPORTED;
  const int q_last = cache->q_last > 0 ? cache->q_last : cache->layer_len[D.N - 1];
  for (int n = 0; n < D.N; ++n) {
    const int qn = n + 1 < D.N ? cache->layer_len[n + 1] : q_last;
    if (qn != cache->layer_len[n]) return ONETRANS_ERR_UNSUPPORTED;
  }
  const bool ragged = cache->user_len != nullptr;
  if (ragged) {
    for (int u = 0; u < n_users; ++u)
      if ((long long)cache->user_len[u] + d_l > cache->capacity) return ONETRANS_ERR_CACHE_CAPACITY;
  } else if ((long long)cache->layer_len[0] + d_l > cache->capacity) {
    return ONETRANS_ERR_CACHE_CAPACITY;
  }
  if ((rc = check_size(D, n_users, d_l))) return rc;
  if (!ws) return ONETRANS_ERR_INVALID_ARG;
  if (misaligned(ws)) return ONETRANS_ERR_ALIGNMENT;
  const size_t wa_bytes = onetrans_workspace_bytes(cfg, ONETRANS_OP_APPEND, n_users, 0, 0, d_l);
  if (ws_bytes < onetrans_workspace_bytes(cfg, ONETRANS_OP_APPEND_SCORE, n_users, 0, n_cand, d_l))
    return ONETRANS_ERR_WORKSPACE;
  size_t n, tin_a, rq_a, tin_b, rq_b;
  bool kv_a, kv_b;
  ws_dims(cfg, D, ONETRANS_OP_APPEND, n_users, 0, 0, d_l, n, tin_a, rq_a, kv_a);
  ws_dims(cfg, D, ONETRANS_OP_SCORE, n_users, 0, n_cand, 0, n, tin_b, rq_b, kv_b);
  const int parts = parts_for(n_users, USER_PART_MIN);
  const size_t n_call_b = (size_t)n_users * n_cand;
  const size_t pa = ws_layout(D, (n_users + parts - 1) / parts, tin_a, rq_a, kv_a, n_users).total;
  const size_t pb = ws_layout(D, (size_t)((n_users + parts - 1) / parts) * n_cand, tin_b, rq_b, kv_b, n_call_b).total;
  char *wb0 = (char *)ws + al(wa_bytes);
  const int l_old = ragged ? 0 : cache->layer_len[0];
  const size_t in_a = (size_t)d_l * D.d * D.esz, out_a = (size_t)d_l * D.d * 4;
  const size_t in_b = (size_t)n_cand * D.lns * D.d * D.esz, out_b = (size_t)n_cand * D.lns * D.d * 4;
  rc = over_streams(n_users, parts, stream, [&](int first, int count, int part, hipStream_t st) {
    const onetrans_kv_cache view = user_view(D, cache, first);
    return append_score_run(D, blk, &view, (const char *)x_new + first * in_a, count, d_l, (char *)out_new + first * out_a,
                            (const char *)x_ns + first * in_b, n_cand, (char *)out_ns + first * out_b,
                            (char *)ws + part * pa, ws_layout(D, count, tin_a, rq_a, kv_a, n_users), wb0 + part * pb,
                            ws_layout(D, (size_t)count * n_cand, tin_b, rq_b, kv_b, n_call_b), l_old, st);
  });
  if (rc) return rc;
  if (ragged) {
    int longest = 0;
    for (int u = 0; u < n_users; ++u) longest = max(longest, cache->user_len[u] += d_l);
    for (int b = 0; b < D.N; ++b) cache->layer_len[b] = max(cache->layer_len[b], longest);
    cache->q_last = cache->layer_len[D.N - 1];
  } else {
    for (int b = 0; b < D.N; ++b) cache->layer_len[b] = l_old + d_l;
    cache->q_last = l_old + d_l;
  }
  return ONETRANS_OK;
}

size_t onetrans_tokenize_workspace_bytes(const onetrans_config *cfg, const onetrans_tokenizer_config *tc,
                                         int batch) {
  Dims D;
  TokPlan P;
  if (check_tok(cfg, tc, batch, D, P)) return 0;
  return P.total;
}

int onetrans_tokenize(const onetrans_config *cfg, const onetrans_tokenizer_config *tc,
                      const onetrans_mlp_weights *seq_mlp, const void *seq_vec, const onetrans_mlp_weights *ns_mlp,
                      const void *const *events, const void *const *times, const void *ns_feat, int batch,
                      void *x0, void *ws, size_t ws_bytes, hipStream_t stream) {
  Dims D;
  TokPlan P;
  int rc;
  if ((rc = check_tok(cfg, tc, batch, D, P))) return rc;
  if (!seq_mlp || !seq_vec || !events || !x0 || !ws || (P.by_time && !times)) return ONETRANS_ERR_INVALID_ARG;
  if (misaligned(seq_vec) || misaligned(x0) || misaligned(ws)) return ONETRANS_ERR_ALIGNMENT;
  const int n_seq = tc->n_seq;
  for (int i = 0; i < n_seq; ++i) {
    if ((rc = check_mlp(&seq_mlp[i]))) return rc;
    if (tc->seq_len[i] > 0 && (!events[i] || (P.by_time && !times[i]))) return ONETRANS_ERR_INVALID_ARG;
    if (misaligned(events[i]) || (P.by_time && ((uintptr_t)times[i] & 7u))) return ONETRANS_ERR_ALIGNMENT;
  }
  if (D.lns > 0) {
    if ((rc = check_mlp(ns_mlp))) return rc;
    if (!ns_feat) return ONETRANS_ERR_INVALID_ARG;
    if (misaligned(ns_feat)) return ONETRANS_ERR_ALIGNMENT;
  }
  if (ws_bytes < P.total) return ONETRANS_ERR_WORKSPACE;

  const int rt = lin_rows_per_tile(), nt = lin_features_per_tile();
  const long long d = D.d, sample = (long long)P.T * d;
  // The launches for samples [b0, b0 + nb) on stream st. Every buffer is sample-major, so a range of
  // samples is a pointer offset into each (hidden activations and row indices included).
  auto run = [&](int b0, int nb, hipStream_t st) -> int {
    auto at = [](const void *p, size_t bytes) { return p ? (const char *)p + bytes : nullptr; };
    char *w = (char *)ws;
    char *x = (char *)x0 + (size_t)b0 * sample * D.esz;
    LinArgs l1{}, l2{};
    int tiles1 = 0, tiles2 = 0;
    auto add = [&](LinArgs &A, int &tiles, LinGroup g) {
      if (g.m == 0) return;
      g.tile0 = tiles;
      A.g[A.n_groups++] = g;
      tiles += (g.m + rt - 1) / rt * (g.n / nt);
    };
    SepArgs sa{};
    sa.sep = seq_vec;
    sa.x0 = x;
    sa.sample_stride = sample;
    sa.d = D.d;
    sa.n_sep = n_seq;
    sa.batch = nb;
    RankArgs ra{};
    ra.n_seq = n_seq;
    ra.total = P.l_s;
    int off = 0;   // first row of sequence i inside the S-tokens (intent order)
    for (int i = 0; i < n_seq; ++i) {
      const int L = tc->seq_len[i], h = tc->seq_hidden[i], m = nb * L;
      const size_t r0 = (size_t)b0 * L;   // first event row of the range
      const onetrans_mlp_weights &p = seq_mlp[i];
      char *hid = w + P.hid[i] + r0 * h * D.esz;
      // MLP_i, layer 1: events -> hidden (GELU); layer 2: hidden -> rows off..off+L-1 of each
      // sample, or, merged by time, to each event's ranked row plus the type embedding
      add(l1, tiles1, LinGroup{at(events[i], r0 * tc->seq_dim[i] * D.esz), tc->seq_dim[i], p.w1, p.b1, hid, h, 0, 1, m,
                               h, tc->seq_dim[i], 1, 0});
      if (P.by_time) {
        int *pos = (int *)(w + P.pos[i]) + r0;
        ra.t[i] = (const long long *)at(times[i], r0 * sizeof(long long));
        ra.pos[i] = pos;
        ra.len[i] = L;
        add(l2, tiles2, LinGroup{hid, h, p.w2, p.b2, x, sample, d, L, m, D.d, h, 0, 0, pos,
                                 (const char *)seq_vec + (size_t)i * d * D.esz});
      } else {
        add(l2, tiles2, LinGroup{hid, h, p.w2, p.b2, x + (size_t)off * d * D.esz, sample, d, L, m, D.d, h, 0, 0});
        sa.sep_row[i] = off + L;
        off += L + 1;
      }
    }
    if (D.lns > 0) {
      // Auto-Split: one row per sample, its l_ns * d outputs are the sample's NS rows in order
      const int h = tc->ns_hidden;
      char *hid = w + P.hid[n_seq] + (size_t)b0 * h * D.esz;
      add(l1, tiles1, LinGroup{at(ns_feat, (size_t)b0 * tc->ns_dim * D.esz), tc->ns_dim, ns_mlp->w1, ns_mlp->b1, hid, h,
                               0, 1, nb, h, tc->ns_dim, 1, 0});
      add(l2, tiles2, LinGroup{hid, h, ns_mlp->w2, ns_mlp->b2, x + (size_t)P.l_s * d * D.esz, sample, 0, 1, nb,
                               D.lns * D.d, h, 0, 0});
    }
    if (P.by_time && timed(ONETRANS_K_MERGE, st, [&] { return launch_rank(ra, nb, st); }) != hipSuccess)
      return ONETRANS_ERR_HIP;
    if (tiles1 > 0 && timed(ONETRANS_K_LIN, st, [&] { return launch_lin(D.dt, l1, tiles1, st); }) != hipSuccess)
      return ONETRANS_ERR_HIP;
    if (tiles2 > 0 && timed(ONETRANS_K_LIN, st, [&] { return launch_lin(D.dt, l2, tiles2, st); }) != hipSuccess)
      return ONETRANS_ERR_HIP;
    if (!P.by_time && timed(ONETRANS_K_MERGE, st, [&] { return launch_sep(D.dt, sa, st); }) != hipSuccess)
      return ONETRANS_ERR_HIP;
    return ONETRANS_OK;
  };
  // One stream: each launch already has thousands of workgroups, and two concurrent half-batches
  // measured 7 % slower (they only contend for HBM).
  return run(0, batch, stream);
}

const char *onetrans_status_string(int status) {
  switch (status) {
    case ONETRANS_OK: return "ok";
    case ONETRANS_ERR_INVALID_ARG: return "invalid argument";
    case ONETRANS_ERR_SHAPE: return "inconsistent shape or pyramid schedule";
    case ONETRANS_ERR_UNSUPPORTED: return "unsupported configuration";
    case ONETRANS_ERR_WORKSPACE: return "workspace too small";
    case ONETRANS_ERR_CACHE_CAPACITY: return "kv cache capacity exceeded";
    case ONETRANS_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
    case ONETRANS_ERR_HIP: return "HIP runtime error";
    case ONETRANS_ERR_SCRATCH: return "call needs more than the library's static scratch (ONETRANS_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

const char *onetrans_version(void) { return "onetrans-gfx950 0.1"; }

int onetrans_set_streams(int n) {
  if (n != 1 && n != 2 && n != 4) return ONETRANS_ERR_INVALID_ARG;
  g_streams = n;
  return ONETRANS_OK;
}

int onetrans_timing_enable(int on) {
  g_timing = on != 0;
  return ONETRANS_OK;
}

int onetrans_timing_read(double *ms, long long *launches) {
  int rc = ONETRANS_OK;
  for (const TimedLaunch &t : g_timed) {
    float e = 0.0f;
    if (hipEventSynchronize(t.b) != hipSuccess || hipEventElapsedTime(&e, t.a, t.b) != hipSuccess) rc = ONETRANS_ERR_HIP;
    if (ms && t.cls >= 0 && t.cls < ONETRANS_K_COUNT) ms[t.cls] += e;
    if (launches && t.cls >= 0 && t.cls < ONETRANS_K_COUNT) launches[t.cls] += 1;
    g_event_pool.push_back(t.a);
    g_event_pool.push_back(t.b);
  }
  g_timed.clear();
  return rc;
}

}  // extern "C"
