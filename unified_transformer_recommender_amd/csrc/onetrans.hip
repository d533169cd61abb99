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
#include <vector>

#include "onetrans.h"
#include "common.hpp"
#include "launch.hpp"

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
template <class F>
hipError_t timed(int cls, hipStream_t s, F &&launch) {
  if (!g_timing) return launch();
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
  if (D.dt == ONETRANS_F32 && D.d > 256) return ONETRANS_ERR_UNSUPPORTED;
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
  size_t x[2], st[2], q, k, v, o, trash, seq, total;
};

inline size_t al(size_t b) { return (b + 255) & ~(size_t)255; }

// n: sequences; tin: max block input rows; rq: max query rows; kv: K/V buffers needed
Ws ws_layout(const Dims &D, size_t n, size_t tin, size_t rq, bool kv) {
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
      if (n_seq < 1 || d_l < 1) return false;
      n = n_seq; tin = rq = d_l; kv = false;
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
};

int run_step(const Dims &D, const onetrans_block_weights &w, const Step &st, char *ws, const Ws &L,
             hipStream_t stream) {
  const int d = D.d, H = D.H, dh = D.dh;
  const int p0 = st.s - st.q;
  const int R = st.q + st.ns;
  char *qb = ws + L.q, *ob = ws + L.o;
  int rc;

  const HeadView q_v{qb, (long long)H * R * dh, (long long)R * dh, p0};

  // pre-norm 1 + mixed Q/K/V: K/V for the S rows [kv_t0, kv_t0 + kv_n) and the NS rows, Q for the
  // rows at positions >= p0 (tail S rows and NS rows)
  {
    QkvArgs qa;
    memset(&qa, 0, sizeof(qa));
    const int no_q = 0x7fffffff;
    int nj = 0, bm = 0;
    long long tiles = 0;
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
    };
    auto add_jobs = [&](int tg) {
      nj = 0;
      tiles = 0;
      bm = qkv_tokens_per_tile(tg);
      qa.tg = tg;
      if (st.kv_n > 0) add_job(RowSet{st.n_seq, st.kv_n, 1, st.kv_t0, 0, 0}, st.need_out ? p0 : no_q, st.kS, st.vS);
      if (st.ns > 0) add_job(RowSet{st.n_seq, 1, st.ns, st.s, 1, 1}, st.need_out ? st.s : no_q, st.kN, st.vN);
    };
    // two token groups per wave, unless that leaves fewer workgroups than half the GPU's CUs
    add_jobs(qkv_max_groups(D.dt, d));
    if (qa.tg == 2 && tiles < QKV_SMALL_LAUNCH) add_jobs(1);
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
    if (tiles > 0x7fffffffLL) return ONETRANS_ERR_UNSUPPORTED;
    const hipError_t e = timed(ONETRANS_K_QKV, stream, [&] { return launch_qkv(D.dt, st.x_f32, qa, (int)tiles, stream); });
    if (e != hipSuccess) return ONETRANS_ERR_HIP;
  }
  if (!st.need_out) return ONETRANS_OK;

  // attention
  {
    AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.n_heads = H;
    a.d_model = d;
    a.R = R;
    a.p0 = p0;
    a.n_pre = st.n_pre;
    a.q = qb;
    a.q_sb = q_v.sb;
    a.q_sh = q_v.sh;
    a.k_pre = st.kp;
    a.v_pre = st.vp;
    a.pre_sb = st.pre_sb;
    a.pre_sh = st.pre_sh;
    a.o = ob;
    a.o_sb = (long long)R * d;
    a.seq_shift = st.seq_shift;
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
    if (timed(ONETRANS_K_ATTN, stream, [&] { return launch_attn(D.dt, dh, st.stage2, a, stream); }) != hipSuccess)
      return ONETRANS_ERR_HIP;
  }

  // W^O + residual + norm2 + mixed FFN + residual, fused, over the query rows:
  // tail S rows use parameter set 0, NS token j uses set 1 + j
  {
    PostArgs pa;
    memset(&pa, 0, sizeof(pa));
    const int bm = post_tokens_per_tile(D.dt, d);
    int nj = 0;
    long long tiles = 0;
    auto add_job = [&](RowSet rs) {
      const long long m = (long long)rs.n_seq * rs.rows;
      if (m == 0 || rs.n_groups == 0) return;
      PostJob &j = pa.job[nj++];
      j.rs = rs;
      j.m_tiles = (int)((m + bm - 1) / bm);
      j.tile_start = (int)tiles;
      tiles += (long long)j.m_tiles * rs.n_groups;
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
    if (tiles > 0x7fffffffLL) return ONETRANS_ERR_UNSUPPORTED;
    const hipError_t e = timed(ONETRANS_K_POST, stream, [&] { return launch_post(D.dt, st.x_f32, pa, (int)tiles, stream); });
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
  if (misaligned(c->k) || misaligned(c->v)) return ONETRANS_ERR_ALIGNMENT;
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
    if ((rc = run_step(D, blk[n], st, w, L, stream))) return rc;
    x = RowView{w + L.x[n & 1], (long long)R * d, 0, d};
    stats = st.stats_out;
    x_f32 = 1;
    s = q;
  }
  return ONETRANS_OK;
}

// The append launch sequence for `n_users` users of `cache` (a view whose first user is the call's
// first user), with workspace `w` laid out as L. l_old: cached rows (0 for ragged users, whose own
// lengths come from cache->user_len).
int append_run(const Dims &D, const onetrans_block_weights *blk, const onetrans_kv_cache *cache, const void *x_new,
               int n_users, int d_l, void *out_new, char *w, const Ws &L, int l_old, hipStream_t stream) {
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
  for (int n = 0; n < D.N; ++n) {
    const bool last = n + 1 == D.N;
    Step st{};
    st.n_seq = n_users;
    st.s = l_old + d_l;
    st.q = d_l;
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
    st.out = RowView{last && out_new ? out_new : (void *)(w + L.x[n & 1]), (long long)d_l * d, l_old, d};
    st.kv_shift = shift;
    st.seq_shift = shift;
    st.stats_in = stats;
    st.stats_out = last ? nullptr : (void *)(w + L.st[n & 1]);
    st.need_out = !last || out_new != nullptr;
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
    if ((rc = run_step(D, blk[n], st, w, L, stream))) return rc;
    x = RowView{w + L.x[n & 1], (long long)ns * d, 0, d};
    stats = st.stats_out;
    x_f32 = 1;
  }
  return ONETRANS_OK;
}

// The Stage I launch sequence for `n_users` users of `cache` (a view whose first user is the
// call's first user), with workspace `w` laid out as L. Writes no host state.
int prefill_run(const Dims &D, const onetrans_config *cfg, const onetrans_block_weights *blk, const void *x_s,
                int n_users, int l_s, const onetrans_kv_cache *cache, void *out_s, char *w, const Ws &L,
                hipStream_t stream) {
  int rc;
  const int d = D.d;
  int s = l_s;
  RowView x{const_cast<void *>(x_s), (long long)l_s * d, 0, d};
  int x_f32 = D.dt == ONETRANS_F32;
  void *stats = nullptr;   // (mean, rstd) rows of x when the previous block wrote them
  for (int n = 0; n < D.N; ++n) {
    const int q = cfg->s_queries[n];
    const int p0 = s - q;
    const bool last = n + 1 == D.N;
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
    st.out = RowView{last ? out_s : (void *)(w + L.x[n & 1]), (long long)q * d, p0, d};
    st.need_out = !last || out_s != nullptr;
    st.stats_in = stats;
    st.stats_out = last ? nullptr : (void *)(w + L.st[n & 1]);
    if ((rc = run_step(D, blk[n], st, w, L, stream))) return rc;
    x = RowView{w + L.x[n & 1], (long long)q * d, 0, d};
    stats = st.stats_out;
    x_f32 = 1;
    s = q;
  }
  return ONETRANS_OK;
}

}  // namespace

extern "C" {

size_t onetrans_workspace_bytes(const onetrans_config *cfg, int op, int n_seq, int l_s, int n_cand, int d_l) {
  Dims D;
  if (check_cfg(cfg, D)) return 0;
  size_t n, tin, rq;
  bool kv;
  if (!ws_dims(cfg, D, op, n_seq, l_s, n_cand, d_l, n, tin, rq, kv)) return 0;
  if ((op == ONETRANS_OP_FORWARD || op == ONETRANS_OP_PREFILL) && check_schedule(cfg, l_s)) return 0;
  const int parts = ws_parts_for(n_seq, op == ONETRANS_OP_FORWARD ? FORWARD_PART_MIN : USER_PART_MIN);
  const size_t per = op == ONETRANS_OP_SCORE ? (size_t)n_cand : 1;   // sequences per user
  return ws_layout(D, (size_t)((n_seq + parts - 1) / parts) * per, tin, rq, kv).total * parts;
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
  size_t n, tin, rq;
  bool kv;
  ws_dims(cfg, D, ONETRANS_OP_FORWARD, batch, l_s, 0, 0, n, tin, rq, kv);
  const int wp = ws_parts_for(batch, FORWARD_PART_MIN), parts = parts_for(batch, FORWARD_PART_MIN);
  if (misaligned(ws)) return ONETRANS_ERR_ALIGNMENT;
  if (!ws) return ONETRANS_ERR_INVALID_ARG;
  if (ws_bytes < ws_layout(D, (batch + wp - 1) / wp, tin, rq, kv).total * wp) return ONETRANS_ERR_WORKSPACE;
  const size_t part_bytes = ws_layout(D, (batch + parts - 1) / parts, tin, rq, kv).total;
  const size_t in_row = (size_t)(l_s + D.lns) * D.d * D.esz;
  const size_t out_row = (size_t)(cfg->s_queries[D.N - 1] + D.lns) * D.d * 4;
  return over_streams(batch, parts, stream, [&](int first, int count, int part, hipStream_t st) {
    return forward_run(D, cfg, blk, (const char *)x0 + first * in_row, count, l_s, (char *)out + first * out_row,
                       (char *)ws + part * part_bytes, ws_layout(D, count, tin, rq, kv), st);
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
  if (ws_bytes < ws_layout(D, (n_users + wp - 1) / wp, tin, rq, kv).total * wp) return ONETRANS_ERR_WORKSPACE;
  const size_t part_bytes = ws_layout(D, (n_users + parts - 1) / parts, tin, rq, kv).total;
  const size_t in_user = (size_t)l_s * D.d * D.esz, out_user = (size_t)cfg->s_queries[D.N - 1] * D.d * 4;
  rc = over_streams(n_users, parts, stream, [&](int first, int count, int part, hipStream_t st) {
    const onetrans_kv_cache view = user_view(D, cache, first);
    return prefill_run(D, cfg, blk, (const char *)x_s + first * in_user, count, l_s, &view,
                       out_s ? (char *)out_s + first * out_user : nullptr, (char *)ws + part * part_bytes,
                       ws_layout(D, count, tin, rq, kv), st);
  });
  if (rc) return rc;
  int s = l_s;
  for (int n = 0; n < D.N; ++n) {
    cache->layer_len[n] = s;
    s = cfg->s_queries[n];
  }
  return ONETRANS_OK;
}

int onetrans_score_candidates(const onetrans_config *cfg, const onetrans_block_weights *blk,
                              const onetrans_kv_cache *cache, const void *x_ns, int n_users, int n_cand,
                              void *out_ns, void *ws, size_t ws_bytes, hipStream_t stream) {
  Dims D;
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
  const bool ragged = cache->user_len != nullptr;
  if (ragged && (rc = check_user_len(cache, n_users, cache->capacity))) return rc;
  size_t n, tin, rq;
  bool kv;
  ws_dims(cfg, D, ONETRANS_OP_SCORE, n_users, 0, n_cand, 0, n, tin, rq, kv);
  const int wp = ws_parts_for(n_users, USER_PART_MIN), parts = parts_for(n_users, USER_PART_MIN);
  if (misaligned(ws)) return ONETRANS_ERR_ALIGNMENT;
  if (!ws) return ONETRANS_ERR_INVALID_ARG;
  if (ws_bytes < ws_layout(D, (size_t)((n_users + wp - 1) / wp) * n_cand, tin, rq, kv).total * wp)
    return ONETRANS_ERR_WORKSPACE;
  const size_t part_bytes = ws_layout(D, (size_t)((n_users + parts - 1) / parts) * n_cand, tin, rq, kv).total;
  const size_t in_user = (size_t)n_cand * D.lns * D.d * D.esz, out_user = (size_t)n_cand * D.lns * D.d * 4;
  return over_streams(n_users, parts, stream, [&](int first, int count, int part, hipStream_t st) {
    const onetrans_kv_cache view = user_view(D, cache, first);
    return score_run(D, blk, &view, (const char *)x_ns + first * in_user, count, n_cand,
                     (char *)out_ns + first * out_user, (char *)ws + part * part_bytes,
                     ws_layout(D, (size_t)count * n_cand, tin, rq, kv), st);
  });
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
  for (int n = 0; n < D.N; ++n) {
    if (cache->layer_len[n] < 0 || cache->layer_len[n] > cache->capacity) return ONETRANS_ERR_SHAPE;
    if (cache->layer_len[n] != cache->layer_len[0]) return ONETRANS_ERR_UNSUPPORTED;
  }
  const bool ragged = cache->user_len != nullptr;
  if (ragged) {
    if ((rc = check_user_len(cache, n_users, cache->capacity))) return rc;
    for (int u = 0; u < n_users; ++u)
      if ((long long)cache->user_len[u] + d_l > cache->capacity) return ONETRANS_ERR_CACHE_CAPACITY;
  } else if ((long long)cache->layer_len[0] + d_l > cache->capacity) {
    return ONETRANS_ERR_CACHE_CAPACITY;
  }
  size_t n, tin, rq;
  bool kv;
  ws_dims(cfg, D, ONETRANS_OP_APPEND, n_users, 0, 0, d_l, n, tin, rq, kv);
  const int wp = ws_parts_for(n_users, USER_PART_MIN), parts = parts_for(n_users, USER_PART_MIN);
  if (misaligned(ws)) return ONETRANS_ERR_ALIGNMENT;
  if (!ws) return ONETRANS_ERR_INVALID_ARG;
  if (ws_bytes < ws_layout(D, (n_users + wp - 1) / wp, tin, rq, kv).total * wp) return ONETRANS_ERR_WORKSPACE;
  const int l_old = ragged ? 0 : cache->layer_len[0];
  const size_t part_bytes = ws_layout(D, (n_users + parts - 1) / parts, tin, rq, kv).total;
  const size_t in_user = (size_t)d_l * D.d * D.esz, out_user = (size_t)d_l * D.d * 4;
  rc = over_streams(n_users, parts, stream, [&](int first, int count, int part, hipStream_t st) {
    const onetrans_kv_cache view = user_view(D, cache, first);
    return append_run(D, blk, &view, (const char *)x_new + first * in_user, count, d_l,
                      out_new ? (char *)out_new + first * out_user : nullptr, (char *)ws + part * part_bytes,
                      ws_layout(D, count, tin, rq, kv), l_old, st);
  });
  if (rc) return rc;
  if (ragged) {
    int longest = 0;
    for (int u = 0; u < n_users; ++u) longest = max(longest, cache->user_len[u] += d_l);
    for (int n = 0; n < D.N; ++n) cache->layer_len[n] = max(cache->layer_len[n], longest);
  } else {
    for (int n = 0; n < D.N; ++n) cache->layer_len[n] = l_old + d_l;
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
