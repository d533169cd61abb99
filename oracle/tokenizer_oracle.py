"""Plain, slow fp64 CPU oracle of the tokenizers that build the first block's input X(0).

TEST INFRASTRUCTURE. Only tests, the smoke check and the benchmark's CPU-baseline leg use this
module; the HIP product path shares no code with it.

Source: fun-rec-mdbook (English), chapter 7.5 "OneTrans", section 7.5.0 "Unified Tokenization"
(the equations for the aligned sequences, S-tokens, NS-tokens and X(0)); the paper-daily deep
reading of the OneTrans paper, section 2.1 "Unified Tokenization", recommends the Auto-Split
tokenizer because one MLP instead of one per feature group saves kernel launches.

What is computed, per sample and independently:

  S~_i      = [MLP_i(e_i1), ..., MLP_i(e_iL_i)]       one behaviour-specific MLP per sequence type,
                                                      applied to every event of that sequence
  S-tokens  = Merge(S~_1, ..., S~_n)                  timestamp-agnostic merge: the sequences in the
                                                      given (intent) order, each followed by its own
                                                      learnable [SEP] row; L_S = sum L_i + n
                                                      timestamp-aware merge: every event row plus its
                                                      behaviour type's embedding, all events in time
                                                      order; L_S = sum L_i
  NS-tokens = Split(MLP(Concat(NS)), L_NS)            one MLP over the concatenated non-sequential
                                                      features, its output cut into L_NS rows of d
  X(0)      = [S-tokens; NS-tokens]

Readings of points the section leaves open (each listed in the design notes):
  * an MLP is two linear layers with biases and the exact erf GELU between them:
    MLP(x) = W2 GELU(W1 x + b1) + b2, weights stored (out, in) like nn.Linear;
  * the hidden width of each MLP is a free parameter of the model;
  * the merge puts one [SEP] row after every sequence (so L_SEP = n), sequences in the order the
    caller gives them (highest intent first);
  * Split cuts the MLP output into consecutive pieces of width d: NS token j is output elements
    [j d, (j + 1) d);
  * timestamp-aware merge: the behaviour-type identifier is a learnable vector per type added to
    each of its event rows; events go in ascending time (oldest first, so the newest events are
    the tail the pyramid keeps); equal times keep the intent order of the types, then the order
    within the sequence; no [SEP] rows.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

from .onetrans_oracle import gelu

F64 = np.float64


def mlp(x: np.ndarray, w1: np.ndarray, b1: np.ndarray, w2: np.ndarray, b2: np.ndarray) -> np.ndarray:
    """Two-layer MLP on the last axis: W2 GELU(W1 x + b1) + b2 (weights (out, in))."""
    x = np.asarray(x, F64)
    h = gelu(x @ np.asarray(w1, F64).T + np.asarray(b1, F64))
    return h @ np.asarray(w2, F64).T + np.asarray(b2, F64)


def s_tokens(events: Sequence[np.ndarray], seq_mlps: Sequence[dict], sep: np.ndarray) -> np.ndarray:
    """Aligned and merged behaviour sequences of one sample: [S~_1; SEP_1; S~_2; SEP_2; ...]."""
    rows = []
    for i, (e, p) in enumerate(zip(events, seq_mlps)):
        rows.append(mlp(e, p["w1"], p["b1"], p["w2"], p["b2"]))
        rows.append(np.asarray(sep[i], F64)[None, :])
    return np.concatenate(rows, axis=0)


def s_tokens_by_time(events: Sequence[np.ndarray], times: Sequence[np.ndarray], seq_mlps: Sequence[dict],
                     type_emb: np.ndarray) -> np.ndarray:
    """Timestamp-aware merge of one sample: aligned event rows plus their type's embedding, sorted by
    (time, type index, position in the sequence)."""
    rows, keys = [], []
    for i, (e, t, p) in enumerate(zip(events, times, seq_mlps)):
        rows.append(mlp(e, p["w1"], p["b1"], p["w2"], p["b2"]) + np.asarray(type_emb[i], F64))
        keys += [(int(t[l]), i, l) for l in range(len(t))]
    order = sorted(range(len(keys)), key=lambda r: keys[r])
    return np.concatenate(rows, axis=0)[order]


def ns_tokens(ns_feat: np.ndarray, ns_mlp: dict, l_ns: int) -> np.ndarray:
    """Auto-Split tokenizer of one sample: Split(MLP(Concat(NS)), l_ns) -> [l_ns][d]."""
    y = mlp(ns_feat, ns_mlp["w1"], ns_mlp["b1"], ns_mlp["w2"], ns_mlp["b2"])
    assert y.shape[-1] % l_ns == 0
    return y.reshape(l_ns, y.shape[-1] // l_ns)


def tokenize(events: Sequence[np.ndarray], ns_feat: np.ndarray, tw: dict, l_ns: int, times=None) -> np.ndarray:
    """X(0) = [S-tokens; NS-tokens] of one sample.

    events[i]: [L_i][D_i] raw event embeddings of behaviour type i; ns_feat: [F] concatenated
    non-sequential features; tw: {"seq": [ {w1, b1, w2, b2} per type ], "sep": [n][d],
    "ns": {w1, b1, w2, b2}}. With times (times[i]: [L_i] integer timestamps) the merge is the
    timestamp-aware one and tw["sep"] holds the behaviour-type embeddings.
    """
    if times is None:
        s = s_tokens(events, tw["seq"], tw["sep"])
    else:
        s = s_tokens_by_time(events, times, tw["seq"], tw["sep"])
    if l_ns == 0:
        return s
    return np.concatenate([s, ns_tokens(ns_feat, tw["ns"], l_ns)], axis=0)


def tokenize_batch(events: Sequence[np.ndarray], ns_feat: np.ndarray, tw: dict, l_ns: int, times=None) -> np.ndarray:
    """Batched form: events[i] is [B][L_i][D_i], ns_feat [B][F] (times[i] [B][L_i]); returns X(0)
    [B][L_S + l_ns][d]."""
    B = ns_feat.shape[0]
    return np.stack([tokenize([e[b] for e in events], ns_feat[b], tw, l_ns,
                              None if times is None else [t[b] for t in times]) for b in range(B)])
