/*
 * onetrans.h — C ABI of the MI355X (gfx950) OneTrans hot path.
 *
 * The method (fun-rec-mdbook, chapter 7.5 "OneTrans: Unifying Sequence Modeling and Feature
 * Interaction"; paper-daily deep reading of the OneTrans paper, section 2):
 *   X(0) = [S-tokens; NS-tokens], S rows first (section 7.5.0, equation for X(0));
 *   each block is a pre-norm causal Transformer block whose Q/K/V/O and FFN parameters are
 *   mixed: all S rows share one set, NS token j owns set 1 + j (section 7.5.1, conditional
 *   parameterization and Mixed FFN);
 *   the Pyramid Stack keeps only the tail S rows as queries (keys/values span all rows of the
 *   block) and the block output keeps only those rows (section 7.5.2);
 *   serving splits into Stage I (S side once per user, K/V cached per block) and Stage II
 *   (NS rows per candidate against the cache), and an append-only user sequence extends the
 *   cache by the new rows only (section 7.5.3).
 *
 * Conventions shared by every entry point
 *   - Every pointer is a DEVICE pointer unless marked "host". Device pointers must be 16-byte
 *     aligned. The caller owns all memory (inputs, outputs, weights, workspace, K/V cache); the
 *     library never allocates or frees device memory.
 *   - Calls are asynchronous on `stream` (NULL = the null stream). Buffers must stay alive until
 *     the stream has passed the call. Argument validation (shapes, launch sizes, workspace, cache
 *     capacity) happens on the host before anything is enqueued; a call that returns an error
 *     other than ONETRANS_ERR_HIP has enqueued nothing and changed no host state (layer_len,
 *     user_len). A call whose launch grids would not fit a 32-bit int returns SHAPE.
 *     Device faults surface at the caller's synchronisation or as ONETRANS_ERR_HIP of a later call.
 *   - Storage dtype (config.dtype) applies to X(0) / x_s / x_ns / x_new, all weights and norm
 *     parameters, and the K/V cache. Arithmetic accumulates in fp32; the residual stream between
 *     blocks is fp32; every output buffer (out, out_s, out_ns, out_new) is fp32.
 *   - Weight matrices are (out, in) row-major, like torch.nn.Linear: y = W x. Each matrix is
 *     stored as [1 + l_ns][rows][cols]: index 0 is the shared S set, 1 + j is NS token j.
 *   - No exceptions cross the boundary; every entry point returns an onetrans_status.
 *   - Supported shapes: d_head = d_model / n_heads in {16, 32}; d_model in {64, 128, 256, 512};
 *     d_ff a multiple of 64, at most 2048; 0 <= l_ns <= 32 (>= 1 for score_candidates).
 */
#ifndef ONETRANS_H_
#define ONETRANS_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ONETRANS_OK = 0,
  ONETRANS_ERR_INVALID_ARG = -1,    /* null pointer, bad enum, non-positive size */
  ONETRANS_ERR_SHAPE = -2,          /* inconsistent sizes or pyramid schedule */
  ONETRANS_ERR_UNSUPPORTED = -3,    /* valid but not implemented (d_head, dims, ragged + pyramid) */
  ONETRANS_ERR_WORKSPACE = -4,      /* ws_bytes smaller than onetrans_workspace_bytes() */
  ONETRANS_ERR_CACHE_CAPACITY = -5, /* cache too small for the rows to be written */
  ONETRANS_ERR_ALIGNMENT = -6,      /* a device pointer is not 16-byte aligned */
  ONETRANS_ERR_HIP = -7,            /* a HIP runtime call or kernel launch failed */
  ONETRANS_ERR_SCRATCH = -8         /* the call needs more than ONETRANS_SCRATCH_BYTES of scratch */
} onetrans_status;

typedef enum { ONETRANS_F32 = 0, ONETRANS_BF16 = 1 } onetrans_dtype;
typedef enum { ONETRANS_RMSNORM = 0, ONETRANS_LAYERNORM = 1 } onetrans_norm;
typedef enum {
  ONETRANS_OP_FORWARD = 0, ONETRANS_OP_PREFILL = 1, ONETRANS_OP_SCORE = 2, ONETRANS_OP_APPEND = 3,
  ONETRANS_OP_APPEND_SCORE = 4
} onetrans_op;

typedef struct {
  int n_blocks;           /* N */
  int d_model;            /* d */
  int n_heads;            /* H; head h owns columns [h*d_head, (h+1)*d_head) of q, k, v, o */
  int d_ff;               /* FFN width */
  int l_ns;               /* NS tokens per sample / candidate */
  int norm;               /* onetrans_norm. RMSNorm: x / sqrt(mean(x^2) + eps) * g.
                             LayerNorm: (x - mean) / sqrt(var + eps) * g + b (population var) */
  float norm_eps;
  int dtype;              /* onetrans_dtype (storage) */
  const int *s_queries;   /* host [n_blocks]: q_n, the S rows block n keeps as queries (pyramid,
                             section 7.5.2). Non-increasing, 1 <= q_n <= s_n where s_0 = l_s and
                             s_{n+1} = q_n. q_n = s_n for every block means no pyramid. */
} onetrans_config;

typedef struct {          /* one per block, storage dtype */
  const void *norm1_g, *norm1_b;   /* [d]; *_b is ignored by RMSNorm (may be NULL then) */
  const void *norm2_g, *norm2_b;   /* [d] */
  const void *wq, *wk, *wv, *wo;   /* [1+l_ns][d][d] */
  const void *w1, *b1;             /* [1+l_ns][d_ff][d], [1+l_ns][d_ff] */
  const void *w2, *b2;             /* [1+l_ns][d][d_ff], [1+l_ns][d] */
} onetrans_block_weights;

typedef struct {
  void *k, *v;            /* device, onetrans_kv_cache_bytes() bytes each, storage dtype,
                             layout [user][block][head][capacity][d_head] */
  int n_users;
  int capacity;           /* rows per (user, block) */
  int *layer_len;         /* host [n_blocks]: valid rows of block n (same for every user); written
                             by prefill_user (s_n) and advanced by append_events (+d_l) */
  int *user_len;          /* host [n_users] or NULL. Ragged users: when set, user u's valid rows are
                             the first user_len[u] rows of every block (an unpyramided cache) and
                             the calls below read and advance it per user. layer_len then bounds
                             them: prefill_user sets it to l_s (the padded length), append_events
                             raises it to the largest user_len if that is larger. NULL: every user
                             has layer_len[n] rows. */
  int q_last;             /* host: S rows the last block keeps (its output rows). prefill_user sets
                             it to s_queries[n_blocks - 1]; append_events advances it with the
                             sequence when the last block keeps every row (q_last equal to
                             layer_len[n_blocks - 1]). 0 is read as layer_len[n_blocks - 1]. */
  void *x_tail;           /* device or NULL: [n_users][capacity][d_model] fp32. For a pyramid that
                             prunes before its last block: the input rows of the block after the
                             first pruning block, each at its position in the user's sequence.
                             prefill_user writes them (when set), append_events reads and extends
                             them; an append to such a cache needs it. */
} onetrans_kv_cache;

/* Workspace bytes needed by one call of `op`.
 *   FORWARD: n_seq = batch, l_s = S rows per sample (n_cand, d_l ignored)
 *   PREFILL: n_seq = users, l_s = S rows per user
 *   SCORE:   n_seq = users, n_cand = candidates per user (l_s ignored)
 *   APPEND:  n_seq = users, d_l = appended rows per user; l_s = 0 for a cache whose pyramid
 *            prunes no block before the last, else the rows of the block after the first pruning
 *            block (layer_len[n* + 1]): that block onwards is recomputed over its window
 *   APPEND_SCORE: n_seq = users, d_l = appended rows per user, n_cand = candidates per user
 *            (l_s ignored): the APPEND workspace (l_s = 0) then the SCORE one
 * Returns 0 for an invalid configuration. */
size_t onetrans_workspace_bytes(const onetrans_config *cfg, int op, int n_seq, int l_s, int n_cand,
                                int d_l);

/* Bytes of ONE of the two cache arrays (K or V): n_users * n_blocks * n_heads * capacity * d_head
 * elements of the storage dtype. Returns 0 for an invalid configuration. */
size_t onetrans_kv_cache_bytes(const onetrans_config *cfg, int n_users, int capacity);

/* Monolithic forward of the block stack (sections 7.5.1-7.5.2) over `batch` independent samples.
 *   x0  [batch][l_s + l_ns][d] storage dtype: S rows then NS rows of each sample.
 *   out [batch][q_last + l_ns][d] fp32: final block rows (tail S rows then NS rows).
 * A batch of 64 or more samples runs as two halves (onetrans_set_streams), the second on a stream
 * the library creates once per device (default priority, kept until the process ends); it forks
 * from and joins back into `stream` with events, so the call is still ordered on `stream` alone.
 * When `stream` belongs to another device than the current one the call stays on `stream`.
 * Concurrent calls from several host threads on one device are not supported (they share those
 * streams' fork/join events).
 * Errors: INVALID_ARG, SHAPE, UNSUPPORTED, WORKSPACE, ALIGNMENT, HIP. */
int onetrans_forward(const onetrans_config *cfg, const onetrans_block_weights *blk /* host [n_blocks] */,
                     const void *x0, int batch, int l_s, void *out, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/* Stage I (section 7.5.3): run the S rows of `n_users` users through every block (pyramid
 * included, no NS rows: S rows never attend to NS rows) and write each block's K/V rows into the
 * cache: block n gets s_n rows at positions 0..s_n-1. Sets cache->layer_len[n] = s_n and
 * cache->q_last = s_queries[n_blocks - 1]. With cache->x_tail set and a schedule that prunes
 * before its last block, the outputs of the first pruning block (the next block's input rows) are
 * also written there, at their positions in the sequence, for a later append_events.
 *   x_s   [n_users][l_s][d] storage dtype.
 *   out_s [n_users][q_last][d] fp32 final S rows, or NULL.
 * Ragged users (cache->user_len set by the caller, 0 <= user_len[u] <= l_s): user u's sequence is
 * the first user_len[u] rows of x_s[u]; the rows after it are padding. Row t only attends to rows
 * <= t, so the first user_len[u] rows of every block, in the cache and in out_s, are exactly those
 * of user u's own sequence (the padding rows hold values no later call reads). Needs an
 * unpyramided schedule (every s_queries[n] = l_s), otherwise UNSUPPORTED.
 * 16 or more users run as two halves on two streams, forked from and joined back into `stream`
 * (see onetrans_forward).
 * Errors: as forward, plus CACHE_CAPACITY (capacity < l_s or n_users > cache->n_users), SHAPE (a
 * user_len outside [0, l_s]). */
int onetrans_prefill_user(const onetrans_config *cfg, const onetrans_block_weights *blk,
                          const void *x_s, int n_users, int l_s, onetrans_kv_cache *cache, void *out_s,
                          void *ws, size_t ws_bytes, hipStream_t stream);

/* Stage II (section 7.5.3): score `n_cand` candidates per user. At block n the NS rows of a
 * candidate sit behind the user's layer_len[n] (ragged: user_len[u]) cached S rows; NS query j
 * attends over those cached keys and its own NS keys 0..j in one softmax, then goes through its
 * token-specific FFN.
 *   x_ns   [n_users][n_cand][l_ns][d] storage dtype.
 *   out_ns [n_users][n_cand][l_ns][d] fp32 final NS rows.
 * The cache is read only. 16 or more users run as two halves on two streams, forked from and
 * joined back into `stream` (see onetrans_forward). Errors: as forward, plus SHAPE if
 * n_users > cache->n_users or a layer_len is out of range. */
int onetrans_score_candidates(const onetrans_config *cfg, const onetrans_block_weights *blk,
                              const onetrans_kv_cache *cache, const void *x_ns, int n_users,
                              int n_cand, void *out_ns, void *ws, size_t ws_bytes,
                              hipStream_t stream);

/* Allocation-free Stage II, for callers that cannot allocate device memory or create streams:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, validation, work and results as onetrans_score_candidates, minus the workspace: the
 * workspace lives in a static device array of the library, ONETRANS_SCRATCH_BYTES (64 MiB) per GPU,
 * which each GPU the library runs on holds until the process ends. Its device address is looked up
 * once per device (hipGetSymbolAddress, on the first call with that device current); after that the
 * call makes no allocation of any kind: no hipMalloc / hipFree, no stream or event creation (the
 * whole call runs on `stream`, never split over side streams, and the per-launch timing is not
 * recorded for it).
 *   Size limit: the call needs the workspace of one part, at most
 *   onetrans_workspace_bytes(cfg, ONETRANS_OP_SCORE, n_users, 0, n_cand, 0) bytes (about
 *   72 KiB per candidate at d = 256 with 16 NS tokens, 144 KiB at d = 512): up to 903 candidates
 *   per call at d = 256 with 16 NS tokens, 450 at d = 512. A larger call returns ONETRANS_ERR_SCRATCH before anything is enqueued.
 *   Sharing: every call on one GPU uses that GPU's one array. Each call writes every scratch byte
 *   it reads before reading it (nothing has to start at zero), but calls that overlap in time on
 *   one GPU (two streams, two host threads) race on the array; order them on one stream.
 *   `stream` must belong to the current device (NULL = its null stream), otherwise INVALID_ARG.
 * Errors: as onetrans_score_candidates (without WORKSPACE), plus SCRATCH. */
#define ONETRANS_SCRATCH_BYTES (64u << 20)
int onetrans_score_candidates_noalloc(const onetrans_config *cfg, const onetrans_block_weights *blk,
                                      const onetrans_kv_cache *cache, const void *x_ns, int n_users,
                                      int n_cand, void *out_ns, hipStream_t stream);

/* Cross-request append (section 7.5.3): `d_l` new S rows per user at positions L_old..L_old+d_l-1
 * behind the L_old cached rows. The result equals Stage I of the user's longer sequence under the
 * grown pyramid: a leading block that keeps every row keeps every row of the longer sequence too,
 * and from the first block that prunes on, each block keeps the same count of tail rows as before.
 *   Unpyramided cache (every layer_len equal, the last block keeps every row): only the new rows
 *   are computed (shared S parameters, keys = cached rows plus new rows up to themselves); their
 *   K/V go to offset L_old of every block and layer_len[n] becomes L_old + d_l.
 *   Pyramided cache: the blocks up to and including the first pruning block n* compute the new
 *   rows only, as above (the old rows' keys, values and outputs do not change: those blocks'
 *   windows start at the sequence's first row). The block after n* sees a window that slid by d_l
 *   rows, so blocks n* + 1 onwards are recomputed over their windows, reading their input rows
 *   from cache->x_tail (which prefill_user wrote and this call extends); their layer_len stay.
 *   When only the last block prunes, no block is recomputed.
 * cfg->s_queries is not read by this call: the pyramid comes from layer_len and q_last.
 * Ragged users (cache->user_len set; unpyramided caches only): L_old is user_len[u] for user u,
 * and user_len[u] advances by d_l (the lengths are read and advanced on the host at enqueue time).
 * 16 or more users run as two halves on two streams, forked from and joined back into `stream`
 * (see onetrans_forward for the stream's lifetime and thread-safety).
 *   x_new   [n_users][d_l][d] storage dtype.
 *   out_new [n_users][min(d_l, q_last')][d] fp32, or NULL: the final rows of the new events that
 *           the last block keeps (q_last' = q_last after the call; d_l rows without pyramid).
 * Errors: as forward, plus CACHE_CAPACITY (L_old + d_l > capacity for some user), WORKSPACE (ws
 * sized without the recomputed window, see onetrans_workspace_bytes), INVALID_ARG (a cache that
 * prunes before its last block without x_tail), UNSUPPORTED (ragged users on a pyramided cache),
 * SHAPE (a user_len outside [0, capacity], or layer_len / q_last that no pyramid produces). */
int onetrans_append_events(const onetrans_config *cfg, const onetrans_block_weights *blk,
                           onetrans_kv_cache *cache, const void *x_new, int n_users, int d_l,
                           void *out_new, void *ws, size_t ws_bytes, hipStream_t stream);

/* Cross-request append followed by Stage II scoring of the same users (section 7.5.3: the new
 * events extend the cached sequence, then each candidate's NS rows attend over the whole cached
 * sequence, the new rows included). Equal, bit for bit, to onetrans_append_events(cfg, blk, cache,
 * x_new, n_users, d_l, out_new, ...) followed by onetrans_score_candidates(cfg, blk, cache, x_ns,
 * n_users, n_cand, out_ns, ...), but each block's attention for both query sets runs as one pass
 * over the user's cached keys, so the cache is read once per block instead of twice.
 *   x_new   [n_users][d_l][d] storage dtype; out_new [n_users][d_l][d] fp32 (required).
 *   x_ns    [n_users][n_cand][l_ns][d] storage dtype; out_ns [n_users][n_cand][l_ns][d] fp32.
 *   ws      onetrans_workspace_bytes(cfg, ONETRANS_OP_APPEND_SCORE, n_users, 0, n_cand, d_l) bytes.
 * Supported: an unpyramided cache (every layer_len equal and q_last the same), d_l <= 32 and
 * n_cand * l_ns <= 32; otherwise UNSUPPORTED (call the two entry points instead). Ragged users as
 * in append_events: user u's Stage II keys are its user_len[u] + d_l rows. The cache lengths advance
 * as in append_events. 16 or more users run as two halves on two streams (see onetrans_forward).
 * Errors: those of the two calls it replaces, plus INVALID_ARG for a NULL out_new and UNSUPPORTED
 * as above. */
int onetrans_append_score(const onetrans_config *cfg, const onetrans_block_weights *blk,
                          onetrans_kv_cache *cache, const void *x_new, int n_users, int d_l,
                          void *out_new, const void *x_ns, int n_cand, void *out_ns, void *ws,
                          size_t ws_bytes, hipStream_t stream);

/* ---- Training step (section 7.5.3, closing paragraph: mixed-precision training with activation
 * recomputation; paper-daily deep reading, section 4.3, system-efficiency table) ---------------
 *
 * The gradients of one training step of the block stack over a batch, for a loss whose gradient
 * with respect to the stack's final rows (the last block's kept rows, q_last + l_ns per sample)
 * is d_out. The call runs the forward over the batch keeping only each block's input rows (fp32),
 * then walks the blocks backwards, recomputing each block's internals from its input (activation
 * recomputation) before its backward: the norms, the mixed Q/K/V/O and FFN products, and the
 * causal attention with the pyramid's tail queries, with its probabilities recomputed from the
 * kept per-query log-sum-exp (never stored). Products take storage-dtype operands and accumulate
 * in fp32; every gradient is accumulated and written in fp32.
 * Parameter gradients are sums over the batch, kept per weight set: index 0 of a [1 + l_ns][..]
 * gradient is the shared S set (every S row of every sample), 1 + j is NS token j's own set. */
typedef struct {          /* one per block, device, fp32, shapes as onetrans_block_weights */
  float *norm1_g, *norm1_b;        /* [d]; *_b may be NULL (RMSNorm: written as zeros when set) */
  float *norm2_g, *norm2_b;        /* [d] */
  float *wq, *wk, *wv, *wo;        /* [1+l_ns][d][d] */
  float *w1, *b1;                  /* [1+l_ns][d_ff][d], [1+l_ns][d_ff] */
  float *w2, *b2;                  /* [1+l_ns][d][d_ff], [1+l_ns][d] */
} onetrans_block_grads;

/* Workspace bytes of onetrans_backward for `batch` samples of l_s S rows (0: invalid config or
 * schedule). */
size_t onetrans_backward_workspace_bytes(const onetrans_config *cfg, int batch, int l_s);

/* One training step's gradients (see above).
 *   x0     [batch][l_s + l_ns][d] storage dtype: X(0)
 *   d_out  [batch][q_last + l_ns][d] fp32: dL/d(final rows), q_last = s_queries[n_blocks - 1]
 *   out    [batch][q_last + l_ns][d] fp32 or NULL: the forward's final rows
 *   dx0    [batch][l_s + l_ns][d] fp32 or NULL: dL/dX(0)
 *   grads  host [n_blocks]: every gradient buffer is overwritten (not accumulated into)
 * Runs on `stream` alone. Errors: as onetrans_forward (INVALID_ARG also for a null gradient
 * pointer other than *_b, ALIGNMENT for a misaligned one). */
int onetrans_backward(const onetrans_config *cfg, const onetrans_block_weights *blk, const void *x0, int batch,
                      int l_s, const float *d_out, float *out, float *dx0, const onetrans_block_grads *grads,
                      void *ws, size_t ws_bytes, hipStream_t stream);

/* ---- Tokenizers ahead of block 1 (section 7.5.0, "Unified Tokenization") -------------------
 *
 * S-tokens: n_seq behaviour sequences (types), given in intent order (highest intent first).
 * Event e of type i is a raw embedding of width seq_dim[i]; the behaviour-specific MLP_i maps it
 * to width d. Two merges:
 *   ONETRANS_MERGE_INTENT (timestamp-agnostic): the aligned sequences in the given order, each
 *     followed by its own learnable [SEP] row, so L_S = sum_i seq_len[i] + n_seq and sequence i
 *     starts at row off_i = sum_{j<i} (seq_len[j] + 1).
 *   ONETRANS_MERGE_TIME (timestamp-aware): every aligned event row plus the learnable embedding of
 *     its behaviour type, all events of a sample in ascending time; equal times keep the type
 *     order, then the order inside the sequence. No [SEP] rows: L_S = sum_i seq_len[i].
 * NS-tokens (Auto-Split tokenizer): one MLP maps a sample's concatenated non-sequential features
 * (width ns_dim) to l_ns * d values; NS token j is values [j d, (j + 1) d).
 * Every MLP here is MLP(x) = W2 GELU(W1 x + b1) + b2 with the exact erf GELU, weights (out, in)
 * row-major like the blocks' matrices.
 */
typedef enum { ONETRANS_MERGE_INTENT = 0, ONETRANS_MERGE_TIME = 1 } onetrans_merge;

typedef struct {
  int n_seq;              /* behaviour types, 1..7 */
  const int *seq_len;     /* host [n_seq]: events per sample of type i (>= 0) */
  const int *seq_dim;     /* host [n_seq]: raw event width, a multiple of 64 */
  const int *seq_hidden;  /* host [n_seq]: hidden width of MLP_i, a multiple of 64 */
  int ns_dim;             /* width of Concat(NS), a multiple of 64 (ignored when l_ns = 0) */
  int ns_hidden;          /* hidden width of the Auto-Split MLP, a multiple of 64 (same) */
  int merge;              /* onetrans_merge */
} onetrans_tokenizer_config;

typedef struct {          /* storage dtype */
  const void *w1, *b1;    /* [hidden][in], [hidden] */
  const void *w2, *b2;    /* [out][hidden], [out] */
} onetrans_mlp_weights;

/* Workspace bytes of onetrans_tokenize for `batch` samples (the hidden activations of every MLP,
 * in the storage dtype; with the timestamp-aware merge also one int32 row index per event).
 * Returns 0 for an invalid configuration. */
size_t onetrans_tokenize_workspace_bytes(const onetrans_config *cfg, const onetrans_tokenizer_config *tc,
                                         int batch);

/* Builds X(0) = [S-tokens; NS-tokens] for `batch` samples: the input of onetrans_forward.
 *   seq_mlp  host [n_seq]: MLP_i, in = seq_dim[i], hidden = seq_hidden[i], out = d.
 *   seq_vec  [n_seq][d]: INTENT: the [SEP] row written after sequence i; TIME: the embedding of
 *            behaviour type i, added to each of its event rows.
 *   ns_mlp   host pointer to the Auto-Split MLP (in = ns_dim, hidden = ns_hidden, out = l_ns * d);
 *            NULL when l_ns = 0.
 *   events   host [n_seq] of device pointers: events[i] is [batch][seq_len[i]][seq_dim[i]]
 *            (may be NULL when seq_len[i] = 0).
 *   times    TIME: host [n_seq] of device pointers, times[i] is int64 [batch][seq_len[i]] (may be
 *            NULL when seq_len[i] = 0). Any order is merged exactly; chronological sequences
 *            (non-decreasing per type) take the fast path (binary search instead of an all-pairs
 *            count per sample). INTENT: ignored (NULL).
 *   ns_feat  [batch][ns_dim] (NULL when l_ns = 0).
 *   x0       [batch][L_S + l_ns][d] storage dtype, written entirely.
 * Hidden activations are rounded to the storage dtype; accumulation is fp32.
 * Errors: INVALID_ARG (null pointer, bad dtype or merge), SHAPE (n_seq, a negative length,
 * L_S < 1), UNSUPPORTED (a width not a multiple of 64, n_seq > 7, TIME with more than 8192 events
 * per sample), WORKSPACE, ALIGNMENT, HIP. */
int onetrans_tokenize(const onetrans_config *cfg, const onetrans_tokenizer_config *tc,
                      const onetrans_mlp_weights *seq_mlp, const void *seq_vec,
                      const onetrans_mlp_weights *ns_mlp, const void *const *events,
                      const void *const *times, const void *ns_feat, int batch, void *x0, void *ws,
                      size_t ws_bytes, hipStream_t stream);

/* Streams of the batched calls. 2 (default): a forward of 64 or more samples, and a Stage I,
 * Stage II or append call over 16 or more users, run as two parts on two streams. 4: up to four
 * parts (from 128 samples or 32 users). 1: every call on the caller's stream alone (one kernel at a
 * time, as a per-kernel profile needs). Parts are contiguous ranges of samples or users; results
 * are identical in every setting and workspace sizes do not depend on it. Process-wide setting.
 * Returns INVALID_ARG for other values. */
int onetrans_set_streams(int n);

/* Kernel classes of the per-launch timing below. */
typedef enum {
  ONETRANS_K_QKV = 0,        /* fused pre-norm 1 + mixed Q/K/V projection */
  ONETRANS_K_ATTN = 1,       /* causal / Stage II attention */
  ONETRANS_K_POST = 2,       /* fused W^O + residual + pre-norm 2 + mixed FFN + residual */
  ONETRANS_K_LIN = 3,        /* tokenizer linear layers (grouped MLP layers) */
  ONETRANS_K_MERGE = 4,      /* tokenizer merge: [SEP] rows, or time-order ranks */
  ONETRANS_K_BWD_GEMM = 5,   /* training step: recomputed and backward products, weight gradients
                                (with their split-sum reductions) */
  ONETRANS_K_BWD_ATTN = 6,   /* training step: attention backward (dK/dV and dQ) */
  ONETRANS_K_BWD_ROWS = 7,   /* training step: norms and their backward, conversions, column sums,
                                weight transposes, zero fills */
  ONETRANS_K_COUNT = 8
} onetrans_kernel_class;

/* Per-launch device timing (tracing aid). While enabled, the library brackets every kernel launch
 * with a pair of hipEvents recorded on the call's stream. onetrans_timing_read() waits for the
 * recorded events, adds each pair's elapsed time to ms[class] and counts launches[class]
 * (arrays of ONETRANS_K_COUNT entries, host), then forgets the pairs. Off by default; not
 * thread-safe (one caller at a time). Returns ONETRANS_ERR_HIP if an event call fails. */
int onetrans_timing_enable(int on);
int onetrans_timing_read(double *ms, long long *launches);

/* Static text for a status code. */
const char *onetrans_status_string(int status);

/* Library version string, e.g. "onetrans-gfx950 0.1". */
const char *onetrans_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ONETRANS_H_ */
