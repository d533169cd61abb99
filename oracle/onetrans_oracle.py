"""Plain, slow fp64 CPU oracle of the OneTrans block stack and its two-stage serving.

TEST INFRASTRUCTURE. Only tests, the smoke check and the benchmark's CPU-baseline
leg use this module; the HIP product path shares no code with it.

Sources (the pages this project implements):
  [zh]  fun-rec-mdbook (Chinese), chapter 7.5 "OneTrans"
  [en]  fun-rec-mdbook (English), chapter 7.5 "OneTrans: Unifying Sequence Modeling and
        Feature Interaction"
  [pdr] paper-daily deep reading of "OneTrans: Unified Feature Interaction and Sequence
        Modeling with One Transformer in Industrial Recommender"
  [lpl] listeners-pseudolab review notes "OneTrans 정리"

What is computed, per sample and independently (everything in float64 on the
given input values; in bf16 mode the caller passes bf16-rounded inputs):

  X = [S rows (s of them); NS rows (l_ns)]                  [en] 7.5.0, eq. for X(0)
  w(t) = 0 for S row t (< s), 1 + (t - s) for NS row t      [en] 7.5.1, conditional
                                                             parameterization of W_i
  Xh   = Norm1(X)                                           [en] 7.5.1 last paragraph (pre-norm)
  K_t  = Wk[w(t)] Xh_t, V_t = Wv[w(t)] Xh_t  for all rows   [en] 7.5.2 (K/V from all L tokens)
  Q_t  = Wq[w(t)] Xh_t for the tail rows only               [en] 7.5.2 (queries from the tail set)
  O_t  = concat_h softmax_{u <= t}(Q_t^h . K_u^h / sqrt(dh)) V_u^h    causal mask [en] 7.5.1
  Y_t  = X_t + Wo[w(t)] O_t                                  (multi-head output projection)
  X'_t = Y_t + W2[w(t)] phi(W1[w(t)] Norm2(Y_t) + b1[w(t)]) + b2[w(t)]   [en] 7.5.1 Mixed FFN
  next block input = X' over the tail rows, re-indexed from 0 [en] 7.5.2

Readings of points the pages leave open (each listed in the design notes):
  * the attention output projection W^O exists and is mixed like Q/K/V, with no bias;
  * norm gains/shifts are shared by all rows of a block (one set per sub-layer);
  * RMSNorm: x / sqrt(mean(x^2) + eps) * g;  LayerNorm: (x - mean) / sqrt(var + eps) * g + b
    with the population variance;
  * phi is the exact erf GELU 0.5 x (1 + erf(x / sqrt 2));
  * attention scale 1/sqrt(d_head), heads are contiguous column slices, no positional term;
  * a query sees itself (key position <= query position);
  * the pyramid count q_n counts S rows only; every NS row is always a query;
  * K/V of block n span that block's own input rows (s_n + l_ns), not the original L_S;
  * Stage II attends, per NS query j, over [cached S keys of that block; own NS keys <= j]
    in ONE softmax (the pages' "cross-attention then self-attention" is the two key
    segments of the same causal row);
  * cross-request append on a pyramided stack is recomputation of the longer sequence: the
    leading blocks that keep every row grow with the sequence, and from the first block that
    prunes on, each block keeps the same number of tail rows as before (see grown_schedule).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf

F64 = np.float64


# ----------------------------------------------------------------------------------------------
# elementary pieces
# ----------------------------------------------------------------------------------------------

def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm per row: x / sqrt(mean(x^2) + eps) * g   ([en] 7.5.1: pre-norm + RMSNorm)."""
    x = np.asarray(x, F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, F64)


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float) -> np.ndarray:
    """LayerNorm per row with population variance: (x - mu) / sqrt(var + eps) * g + b."""
    x = np.asarray(x, F64)
    mu = np.mean(x, axis=-1, keepdims=True)
    var = np.mean((x - mu) ** 2, axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(g, F64) + np.asarray(b, F64)


def norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, kind: str, eps: float) -> np.ndarray:
    if kind == "rms":
        return rms_norm(x, g, eps)
    if kind == "layer":
        return layer_norm(x, g, b, eps)
    raise ValueError(f"unknown norm {kind!r}")


def gelu(x: np.ndarray) -> np.ndarray:
    """phi of the Mixed FFN ([en] 7.5.1), read as the exact GELU: 0.5 x (1 + erf(x / sqrt(2)))."""
    x = np.asarray(x, F64)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def weight_group(t: int, s: int) -> int:
    """Index of the parameter set used by row t of a block whose first s rows are S-tokens.

    [en] 7.5.1: W_i = W_S for S-tokens, W_NS,i for NS-tokens; NS token j (row s + j)
    owns set 1 + j, the shared S set is index 0.
    """
    return 0 if t < s else 1 + (t - s)


def mixed_linear(x: np.ndarray, w: np.ndarray, rows: Sequence[int], s: int,
                 b: Optional[np.ndarray] = None) -> np.ndarray:
    """y_t = W[w(t)] x_t (+ b[w(t)]) for each row position t in ``rows`` (x holds those rows in order).

    Rows sharing a parameter set are multiplied together; this is the definition
    applied row by row, grouped only so that numpy does the loop.
    """
    x = np.asarray(x, F64)
    out = np.empty((x.shape[0], w.shape[1]), F64)
    groups: Dict[int, List[int]] = {}
    for i, t in enumerate(rows):
        groups.setdefault(weight_group(t, s), []).append(i)
    for g, idx in groups.items():
        y = x[idx] @ np.asarray(w[g], F64).T
        if b is not None:
            y = y + np.asarray(b[g], F64)
        out[idx] = y
    return out


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: Sequence[int],
                     k_pos: Sequence[int], n_heads: int) -> np.ndarray:
    """Multi-head attention with the causal rule key position <= query position ([en] 7.5.1).

    q: [R][d] at positions q_pos; k, v: [T][d] at positions k_pos. Head h is the
    column slice [h*dh, (h+1)*dh); scores are scaled by 1/sqrt(dh).
    """
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    d = q.shape[1]
    dh = d // n_heads
    visible = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]     # [R][T]
    out = np.empty((q.shape[0], d), F64)
    for h in range(n_heads):
        sl = slice(h * dh, (h + 1) * dh)
        scores = (q[:, sl] @ k[:, sl].T) / math.sqrt(dh)
        scores = np.where(visible, scores, -np.inf)
        scores = scores - scores.max(axis=1, keepdims=True)
        p = np.exp(scores)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, sl] = p @ v[:, sl]
    return out


# ----------------------------------------------------------------------------------------------
# one block
# ----------------------------------------------------------------------------------------------

@dataclass
class BlockTrace:
    """Intermediates of one block for one sample (row order = the block's own rows)."""
    xh: np.ndarray = None    # [T][d]   Norm1 of all input rows
    q: np.ndarray = None     # [R][d]   queries of the tail rows
    k: np.ndarray = None     # [T][d]
    v: np.ndarray = None     # [T][d]
    o: np.ndarray = None     # [R][d]   attention output before W^O
    y: np.ndarray = None     # [R][d]   after the attention residual
    h: np.ndarray = None     # [R][d_ff] FFN hidden after phi
    out: np.ndarray = None   # [R][d]   block output (tail rows)


def block_forward(x: np.ndarray, s: int, q_keep: int, p, m, trace: Optional[BlockTrace] = None
                  ) -> np.ndarray:
    """One OneTrans block over x = [s S rows; l_ns NS rows]; returns the tail q_keep S rows + NS rows.

    [en] 7.5.1 (mixed parameterization, causal mask, Mixed FFN, pre-norm) and
    [en] 7.5.2 (queries only from the tail set Q = {T - R + 1 .. T}, keys/values
    from all T rows, output keeps the rows of Q).
    """
    x = np.asarray(x, F64)
    T = x.shape[0]
    rows = list(range(T))
    tail = list(range(s - q_keep, T))
    xh = norm(x, p.norm1_g, p.norm1_b, m.norm, m.norm_eps)
    k = mixed_linear(xh, p.wk, rows, s)
    v = mixed_linear(xh, p.wv, rows, s)
    q = mixed_linear(xh[tail], p.wq, tail, s)
    o = causal_attention(q, k, v, tail, rows, m.n_heads)
    y = x[tail] + mixed_linear(o, p.wo, tail, s)
    yh = norm(y, p.norm2_g, p.norm2_b, m.norm, m.norm_eps)
    hid = gelu(mixed_linear(yh, p.w1, tail, s, p.b1))
    out = y + mixed_linear(hid, p.w2, tail, s, p.b2)
    if trace is not None:
        trace.xh, trace.q, trace.k, trace.v, trace.o, trace.y, trace.h, trace.out = \
            xh, q, k, v, o, y, hid, out
    return out


# ----------------------------------------------------------------------------------------------
# the four operations
# ----------------------------------------------------------------------------------------------

def forward(x0: np.ndarray, weights, m, s_queries: Sequence[int],
            traces: Optional[List[BlockTrace]] = None) -> np.ndarray:
    """Stack of OneTrans blocks over one sample X(0) = [L_S S rows; l_ns NS rows].

    Returns the final block's rows: [q_last + l_ns][d]. s_queries[n] is the number
    of S rows block n keeps as queries (the pyramid, [en] 7.5.2); block n + 1 sees
    exactly those rows plus the NS rows.
    """
    x = np.asarray(x0, F64)
    s = x.shape[0] - m.l_ns
    for n, p in enumerate(weights):
        tr = BlockTrace() if traces is not None else None
        x = block_forward(x, s, s_queries[n], p, m, tr)
        if traces is not None:
            traces.append(tr)
        s = s_queries[n]
    return x


def forward_batch(x0: np.ndarray, weights, m, s_queries: Sequence[int]) -> np.ndarray:
    """forward() applied to each sample of x0 [B][L_S + l_ns][d] independently."""
    return np.stack([forward(x, weights, m, s_queries) for x in x0])


def prefill_user(x_s: np.ndarray, weights, m, s_queries: Sequence[int]
                 ) -> Tuple[List[Dict[str, np.ndarray]], np.ndarray]:
    """Stage I ([en] 7.5.3): run the S rows alone through every block, caching each block's K/V.

    S rows never attend to NS rows (causal mask, NS rows come last), so the S side
    is computed once per user. Returns (cache, final S rows) where cache[n] holds
    'k' and 'v' of the s_n S rows of block n: [s_n][d] each.
    """
    x = np.asarray(x_s, F64)
    s = x.shape[0]
    cache = []
    for n, p in enumerate(weights):
        q_keep = s_queries[n]
        rows = list(range(s))
        tail = list(range(s - q_keep, s))
        xh = norm(x, p.norm1_g, p.norm1_b, m.norm, m.norm_eps)
        k = mixed_linear(xh, p.wk, rows, s)
        v = mixed_linear(xh, p.wv, rows, s)
        cache.append({"k": k, "v": v})
        q = mixed_linear(xh[tail], p.wq, tail, s)
        o = causal_attention(q, k, v, tail, rows, m.n_heads)
        y = x[tail] + mixed_linear(o, p.wo, tail, s)
        yh = norm(y, p.norm2_g, p.norm2_b, m.norm, m.norm_eps)
        x = y + mixed_linear(gelu(mixed_linear(yh, p.w1, tail, s, p.b1)), p.w2, tail, s, p.b2)
        s = q_keep
    return cache, x


def score_candidate(cache: List[Dict[str, np.ndarray]], x_ns: np.ndarray, weights, m) -> np.ndarray:
    """Stage II ([en] 7.5.3) for one candidate: NS rows only, against the user's cached S K/V.

    At block n the NS rows sit at positions s_n .. s_n + l_ns - 1 behind the s_n
    cached S rows; NS query j attends over the cached S keys and its own NS keys
    0..j (one softmax), then goes through its token-specific FFN. Returns the
    final NS rows [l_ns][d].
    """
    x = np.asarray(x_ns, F64)
    for n, p in enumerate(weights):
        s = cache[n]["k"].shape[0]
        rows = [s + j for j in range(m.l_ns)]
        xh = norm(x, p.norm1_g, p.norm1_b, m.norm, m.norm_eps)
        q = mixed_linear(xh, p.wq, rows, s)
        k = np.concatenate([cache[n]["k"], mixed_linear(xh, p.wk, rows, s)])
        v = np.concatenate([cache[n]["v"], mixed_linear(xh, p.wv, rows, s)])
        o = causal_attention(q, k, v, rows, list(range(s + m.l_ns)), m.n_heads)
        y = x + mixed_linear(o, p.wo, rows, s)
        yh = norm(y, p.norm2_g, p.norm2_b, m.norm, m.norm_eps)
        x = y + mixed_linear(gelu(mixed_linear(yh, p.w1, rows, s, p.b1)), p.w2, rows, s, p.b2)
    return x


def append_events(cache: List[Dict[str, np.ndarray]], x_new: np.ndarray, weights, m
                  ) -> Tuple[List[Dict[str, np.ndarray]], np.ndarray]:
    """Cross-request append ([en] 7.5.3): compute only the new rows and extend the cache.

    The cache must be unpyramided (every block holds the same L_old rows). At
    block n the new rows sit at positions L_old .. L_old + dL - 1, use the shared
    S parameters, attend over the cached rows plus the new rows up to themselves,
    and their K/V are appended to that block's cache. Returns (new cache, final
    new rows [dL][d]).
    """
    lens = {c["k"].shape[0] for c in cache}
    if len(lens) != 1:
        raise ValueError("append needs an unpyramided cache (equal rows in every block)")
    l_old = lens.pop()
    x = np.asarray(x_new, F64)
    dl = x.shape[0]
    s = l_old + dl                       # every appended row is an S row
    rows = list(range(l_old, l_old + dl))
    new_cache = []
    for n, p in enumerate(weights):
        xh = norm(x, p.norm1_g, p.norm1_b, m.norm, m.norm_eps)
        k = np.concatenate([cache[n]["k"], mixed_linear(xh, p.wk, rows, s)])
        v = np.concatenate([cache[n]["v"], mixed_linear(xh, p.wv, rows, s)])
        new_cache.append({"k": k, "v": v})
        q = mixed_linear(xh, p.wq, rows, s)
        o = causal_attention(q, k, v, rows, list(range(l_old + dl)), m.n_heads)
        y = x + mixed_linear(o, p.wo, rows, s)
        yh = norm(y, p.norm2_g, p.norm2_b, m.norm, m.norm_eps)
        x = y + mixed_linear(gelu(mixed_linear(yh, p.w1, rows, s, p.b1)), p.w2, rows, s, p.b2)
    return new_cache, x


def grown_schedule(l_s: int, s_queries: Sequence[int], d_l: int) -> Tuple[int, ...]:
    """Pyramid of a user sequence of l_s rows after d_l more rows are appended ([en] 7.5.2 keeps a
    fixed number of tail rows per block; [en] 7.5.3 appends events at the end).

    Reading: a leading block that keeps every row of its input (q_n = s_n) keeps every row of the
    longer sequence too; from the first block that prunes (q_n < s_n) on, every block keeps the
    same count of tail rows as before.
    """
    out, s, pruned = [], l_s, False
    for q in s_queries:
        pruned = pruned or q < s
        out.append(q if pruned else q + d_l)
        s = q
    return tuple(out)


def append_recompute(x_s_old: np.ndarray, x_new: np.ndarray, weights, m, s_queries: Sequence[int]
                     ) -> Tuple[List[Dict[str, np.ndarray]], np.ndarray]:
    """Cross-request append on any cache, pyramided or not: the cache and final rows that Stage I of
    the concatenated sequence produces ([en] 7.5.3: appending equals recomputing), under the grown
    pyramid. x_s_old: the user's l_s earlier rows (prefilled with s_queries). Returns (cache, final
    rows of the new events that the last block keeps: the last min(d_l, q_last) rows)."""
    x_old = np.asarray(x_s_old, F64)
    x_new = np.asarray(x_new, F64)
    d_l = x_new.shape[0]
    sched = grown_schedule(x_old.shape[0], s_queries, d_l)
    cache, final = prefill_user(np.concatenate([x_old, x_new]), weights, m, sched)
    return cache, final[final.shape[0] - min(d_l, sched[-1]):]
