"""Algorithmic work of the OneTrans hot path (host-side arithmetic only, no device code).

FLOPs count 2 per useful multiply-add of the projections and the FFN, and 4 * d
per *visible* (query, key) pair of the causal attention (2 * d_head for Q.K and
2 * d_head for P.V, summed over the heads). Masked pairs, exponentials and norms
are not counted.

The complexity statements follow fun-rec-mdbook (English) chapter 7.5:
section 7.5.2 (the Pyramid Stack takes attention from O(L^2 d) to O(L L' d) and the
FFN from O(L d^2) to O(L' d^2)) and section 7.5.3 (KV caching takes per-request
sequence work from O(C L_S) to O(L_S + C L_NS), and cross-request append from
O(L_S) to O(dL_S)). The worked problems 7.5.3 and 7.5.4 of the Chinese edition
print numeric answers for two of these estimates; ``pyramid_attention_ratio``
and ``kv_cache_saving`` reproduce them.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Sequence, Tuple


@dataclass
class Work:
    gemm: float = 0.0        # projection + FFN flops
    attn: float = 0.0        # attention flops (visible pairs only)

    @property
    def total(self) -> float:
        return self.gemm + self.attn

    def __add__(self, o: "Work") -> "Work":
        return Work(self.gemm + o.gemm, self.attn + o.attn)

    def scale(self, k: float) -> "Work":
        return Work(self.gemm * k, self.attn * k)


def visible_pairs(first_query_pos: int, n_queries: int) -> int:
    """Visible (query, key) pairs when queries sit at consecutive positions p0..p0+R-1 and
    each sees keys 0..p (key position <= query position)."""
    p0, r = first_query_pos, n_queries
    return r * (p0 + 1) + r * (r - 1) // 2


def block_work(d: int, d_ff: int, kv_rows: int, q_rows: int, first_query_pos: int) -> Work:
    """One block: K/V for ``kv_rows`` rows, Q / W^O / FFN for ``q_rows`` tail rows."""
    gemm = 2.0 * d * d * (2 * kv_rows + 2 * q_rows) + 2.0 * 2 * d * d_ff * q_rows
    attn = 4.0 * d * visible_pairs(first_query_pos, q_rows)
    return Work(gemm, attn)


def forward_work(d: int, d_ff: int, l_ns: int, l_s: int, s_queries: Sequence[int]) -> Work:
    """Per candidate (one sample) of the monolithic forward over [S; NS]."""
    w, s = Work(), l_s
    for q in s_queries:
        w = w + block_work(d, d_ff, s + l_ns, q + l_ns, s - q)
        s = q
    return w


def prefill_work(d: int, d_ff: int, l_s: int, s_queries: Sequence[int]) -> Work:
    """Stage I per user: S rows only."""
    w, s = Work(), l_s
    for q in s_queries:
        w = w + block_work(d, d_ff, s, q, s - q)
        s = q
    return w


def score_work(d: int, d_ff: int, l_ns: int, l_s: int, s_queries: Sequence[int]) -> Work:
    """Stage II per candidate: NS rows against the cached S keys of every block."""
    w, s = Work(), l_s
    for q in s_queries:
        w = w + block_work(d, d_ff, l_ns, l_ns, s)
        s = q
    return w


def append_work(d: int, d_ff: int, n_blocks: int, l_old: int, d_l: int) -> Work:
    """Cross-request append per user (unpyramided): only the d_l new rows per block."""
    return block_work(d, d_ff, d_l, d_l, l_old).scale(n_blocks)


# --- the pages' order-of-magnitude estimates -------------------------------------------------

def pyramid_attention_ratio(query_fractions: Sequence[float]) -> float:
    """Worked problem 7.5.3: attention of a pyramid whose layer k keeps L * f_k queries
    against a fixed full-length K/V, relative to the same number of full layers.

    Cost of layer k ~ L * (L f_k); standard ~ L * L per layer."""
    return sum(query_fractions) / len(query_fractions)


def kv_cache_saving(n_cand: int, l_s: int, l_ns: int) -> Tuple[int, int, float]:
    """Worked problem 7.5.4: (per-candidate sequence work C*L_S, cached work L_S + C*L_NS, ratio)."""
    plain = n_cand * l_s
    cached = l_s + n_cand * l_ns
    return plain, cached, plain / cached


def mixed_param_count(d: int, d_ff: int, l_ns: int, with_wo: bool = True) -> int:
    """Parameters of one block under mixed parameterization: one S set plus one set per NS token,
    O(L_NS d^2 + d^2) ([en] 7.5.1, comparison with a per-token FFN)."""
    per_set = (4 if with_wo else 3) * d * d + 2 * d * d_ff + d_ff + d
    return (1 + l_ns) * per_set


# --- per kernel class (the launch sequence of one block) --------------------------------------

KERNEL_CLASSES = ("qkv", "attn", "post")


def _block_classes(d, d_ff, kv_rows, q_rows, first_query_pos, in_rows, in_bytes, store_bytes):
    """Algorithmic flops of one block for one sequence, by kernel class.

    "qkv" is the fused pre-norm 1 + Q/K/V projection, "post" the fused tail of the block
    (W^O projection plus both FFN projections)."""
    return {
        "qkv": 2.0 * d * d * (2 * kv_rows + q_rows),
        "attn": 4.0 * d * visible_pairs(first_query_pos, q_rows),
        "post": 2.0 * d * d * q_rows + 2.0 * 2 * d * d_ff * q_rows,
    }


def forward_classes(d, d_ff, l_ns, l_s, s_queries, store_bytes):
    """Per-candidate work of the monolithic forward split by kernel class."""
    tot, s = {}, l_s
    for n, q in enumerate(s_queries):
        in_bytes = store_bytes if n == 0 else 4
        c = _block_classes(d, d_ff, s + l_ns, q + l_ns, s - q, s + l_ns, in_bytes, store_bytes)
        for k, v in c.items():
            tot[k] = tot.get(k, 0.0) + v
        s = q
    return tot


def prefill_classes(d, d_ff, l_s, s_queries, store_bytes):
    tot, s = {}, l_s
    for n, q in enumerate(s_queries):
        c = _block_classes(d, d_ff, s, q, s - q, s, store_bytes if n == 0 else 4, store_bytes)
        for k, v in c.items():
            tot[k] = tot.get(k, 0.0) + v
        s = q
    return tot


def score_classes(d, d_ff, l_ns, l_s, s_queries, store_bytes):
    tot, s = {}, l_s
    for n, q in enumerate(s_queries):
        c = _block_classes(d, d_ff, l_ns, l_ns, s, l_ns, store_bytes if n == 0 else 4, store_bytes)
        for k, v in c.items():
            tot[k] = tot.get(k, 0.0) + v
        s = q
    return tot


def append_classes(d, d_ff, n_blocks, l_old, d_l, store_bytes):
    tot = {}
    for n in range(n_blocks):
        c = _block_classes(d, d_ff, d_l, d_l, l_old, d_l, store_bytes if n == 0 else 4, store_bytes)
        for k, v in c.items():
            tot[k] = tot.get(k, 0.0) + v
    return tot


def grown_schedule(l_s: int, s_queries: Sequence[int], d_l: int) -> Tuple[int, ...]:
    """Pyramid of a cached sequence of l_s rows after d_l rows are appended: leading blocks that
    keep every row keep every row of the longer sequence; from the first pruning block on the kept
    counts stay (the library derives the same from a cache's lengths)."""
    out, s, pruned = [], l_s, False
    for q in s_queries:
        pruned = pruned or q < s
        out.append(q if pruned else q + d_l)
        s = q
    return tuple(out)


def pyramid_append_classes(d, d_ff, l_old, d_l, s_queries, store_bytes, out_rows=None):
    """Per-user append to a cache prefilled with s_queries over l_old rows: the new rows through
    the blocks up to the first pruning block n*, then Stage I of blocks n* + 1 .. over their windows
    (which slid by d_l rows). out_rows: queries of the last recomputed block (its kept rows, or
    fewer when only the final rows of the new events are wanted). Without pruning before the last
    block this is the plain append."""
    s, n_star = l_old, None
    for n, q in enumerate(s_queries):
        if q < s:
            n_star = n
            break
        s = q
    n_blocks = len(s_queries)
    head = n_blocks if n_star is None or n_star == n_blocks - 1 else n_star + 1
    tot = append_classes(d, d_ff, head, l_old, d_l, store_bytes)
    if head < n_blocks:
        win = s_queries[n_star]
        tail = list(s_queries[head:])
        if out_rows is not None:
            tail[-1] = min(tail[-1], out_rows)
        for k, v in prefill_classes(d, d_ff, win, tail, 4).items():
            tot[k] = tot.get(k, 0.0) + v
    return tot


def append_cache_bytes(d, n_blocks, l_old, d_l, store_bytes):
    """K/V cache bytes one user's append must read (every cached row of every block, K and V)
    plus the new rows it writes: the HBM floor of the append path."""
    return float(n_blocks * 2 * d * store_bytes * (l_old + d_l) + n_blocks * 2 * d * store_bytes * d_l)


# --- tokenizers ahead of block 1 ([en] 7.5.0) ---------------------------------------------------

def tokenize_work(d, l_ns, seq_lens, seq_dims, seq_hidden, ns_dim, ns_hidden, store_bytes, merge="intent"):
    """Per-sample algorithmic flops and HBM bytes of the two grouped linear launches.

    flops: 2 m n k over every layer of every MLP. bytes: what each launch must read and write
    once: launch 1 reads the raw events / NS features and the first-layer weights and writes the
    hidden activations; launch 2 reads those and the second-layer weights and writes the non-[SEP]
    rows of X(0) (with the timestamp-aware merge also each event's int32 row index). Weights are
    counted once per launch, so per sample they are divided by the batch by the caller (returned
    separately)."""
    flops = 0.0
    act = 0.0        # per-sample activation bytes over both launches
    wts = 0.0        # weight bytes over both launches (once per launch, not per sample)
    for L, D, H in zip(seq_lens, seq_dims, seq_hidden):
        flops += 2.0 * L * (D * H + H * d)
        act += store_bytes * L * (D + H + H + d) + (4 * L if merge == "time" else 0)
        wts += store_bytes * (H * D + H + d * H + d) + (store_bytes * d if merge == "time" else 0)
    if l_ns > 0:
        flops += 2.0 * (ns_dim * ns_hidden + ns_hidden * l_ns * d)
        act += store_bytes * (ns_dim + 2 * ns_hidden + l_ns * d)
        wts += store_bytes * (ns_hidden * ns_dim + ns_hidden + l_ns * d * ns_hidden + l_ns * d)
    return flops, act, wts


# --- training step (forward keeping block inputs + backward with activation recomputation) ------

TRAIN_CLASSES = ("qkv", "attn", "post", "bwd_gemm", "bwd_attn", "bwd_rows")


def train_classes(d, d_ff, l_ns, l_s, s_queries):
    """Per-sample algorithmic flops of one training step by kernel class.

    The forward runs every block once (qkv, attn, post); the backward recomputes each block's Q/K/V
    and attention (qkv, attn again), then W^O and the FFN's first product (bwd_gemm), and runs the
    backward products: for q query rows and t block rows, the FFN's dHidden, dW2, dW1, dYh
    (4 x 2 q d d_ff), W^O's dO and dWo (2 x 2 q d^2), dWq (2 q d^2), dWk and dWv (2 x 2 t d^2) and
    dXh (2 t d 2d + 2 q d^2). Attention backward: dV, dP, dQ, dK (4 x 2 d per visible pair) plus
    the recomputed scores (2 d per pair); the dQ kernel's second pass over the scores and dP is
    implementation overhead and not counted. Row kernels (norms, conversions, sums) count no flops."""
    tot = {k: 0.0 for k in TRAIN_CLASSES}
    s = l_s
    for q in s_queries:
        t, r = s + l_ns, q + l_ns
        pairs = visible_pairs(s - q, r)
        fq = 2.0 * d * d * (2 * t + r)
        fa = 4.0 * d * pairs
        tot["qkv"] += 2 * fq
        tot["attn"] += 2 * fa
        tot["post"] += 2.0 * d * d * r + 4.0 * d * d_ff * r
        tot["bwd_gemm"] += (2.0 * d * d * r + 2.0 * d * d_ff * r          # recomputed W^O and W1
                            + 8.0 * r * d * d_ff + 4.0 * r * d * d        # FFN and W^O backward
                            + 2.0 * r * d * d + 4.0 * t * d * d           # dWq, dWk, dWv
                            + 4.0 * t * d * d + 2.0 * r * d * d)          # dXh
        tot["bwd_attn"] += 10.0 * d * pairs
        s = q
    return tot
