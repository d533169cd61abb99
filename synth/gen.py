"""Seeded generators for weights and inputs.

All arrays are float32. When the model's storage dtype is bf16 the generated
values are rounded to the nearest bf16 value (ties to even) before they are
returned, so the oracle and the device path see the very same numbers: the
oracle computes on these values, the device path uploads their bf16 bits.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

from .shapes import ModelShape, Workload

_STD = 0.02


# ----------------------------------------------------------------------------------------------
# bf16 rounding (input preparation only)
# ----------------------------------------------------------------------------------------------

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values after round-to-nearest-even to bf16 (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float32 array of the bf16 values nearest to ``a`` (ties to even)."""
    bits = bf16_bits(a).astype(np.uint32) << 16
    return bits.view(np.float32).reshape(np.shape(a))


def _maybe_round(a: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(a) if dtype == "bf16" else a


def _normal(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


# ----------------------------------------------------------------------------------------------
# weights
# ----------------------------------------------------------------------------------------------

@dataclass
class BlockWeights:
    """Parameters of one block. Leading index of every matrix/bias: 0 = shared S set, 1+j = NS token j.

    Matrices are (out, in) row-major, i.e. y = W @ x for a column vector x.
    """
    norm1_g: np.ndarray  # [d]
    norm1_b: np.ndarray  # [d] (unused by RMSNorm)
    norm2_g: np.ndarray  # [d]
    norm2_b: np.ndarray  # [d]
    wq: np.ndarray       # [G][d][d]
    wk: np.ndarray       # [G][d][d]
    wv: np.ndarray       # [G][d][d]
    wo: np.ndarray       # [G][d][d]
    w1: np.ndarray       # [G][d_ff][d]
    b1: np.ndarray       # [G][d_ff]
    w2: np.ndarray       # [G][d][d_ff]
    b2: np.ndarray       # [G][d]

    FIELDS = ("norm1_g", "norm1_b", "norm2_g", "norm2_b", "wq", "wk", "wv", "wo", "w1", "b1", "w2", "b2")

    def copy(self) -> "BlockWeights":
        return BlockWeights(**{f: getattr(self, f).copy() for f in self.FIELDS})


def make_weights(m: ModelShape) -> List[BlockWeights]:
    """Seeded per-block parameters (block n uses child stream n of the model's weight seed)."""
    d, f, g = m.d_model, m.d_ff, m.n_groups
    out = []
    for n in range(m.n_blocks):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(m.weight_seed, spawn_key=(n,))))
        p = dict(
            norm1_g=1.0 + _normal(rng, (d,), _STD),
            norm1_b=_normal(rng, (d,), _STD),
            norm2_g=1.0 + _normal(rng, (d,), _STD),
            norm2_b=_normal(rng, (d,), _STD),
            wq=_normal(rng, (g, d, d), _STD),
            wk=_normal(rng, (g, d, d), _STD),
            wv=_normal(rng, (g, d, d), _STD),
            wo=_normal(rng, (g, d, d), _STD),
            w1=_normal(rng, (g, f, d), _STD),
            b1=_normal(rng, (g, f), _STD),
            w2=_normal(rng, (g, d, f), _STD),
            b2=_normal(rng, (g, d), _STD),
        )
        out.append(BlockWeights(**{k: _maybe_round(v.astype(np.float32), m.dtype) for k, v in p.items()}))
    return out


def sep_vectors(m: ModelShape, n_sep: int) -> np.ndarray:
    """[SEP] stand-in rows, drawn once per model and shared by all samples: [n_sep][d]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(m.sep_seed)))
    return _normal(rng, (n_sep, m.d_model))


# ----------------------------------------------------------------------------------------------
# inputs
# ----------------------------------------------------------------------------------------------

def _rng(seed: int, key: Sequence[int]) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def _s_rows(w: Workload, rng: np.random.Generator, n_rows: int) -> np.ndarray:
    x = _normal(rng, (n_rows, w.model.d_model))
    if w.seq_lens:
        seps = sep_vectors(w.model, len(w.seq_lens))
        for i, r in enumerate(w.sep_rows):
            if r < n_rows:
                x[r] = seps[i]
    return x


def forward_sample(w: Workload, b: int) -> np.ndarray:
    """X(0) of sample b: [L_S + L_NS][d] (S rows with [SEP] rows in place, then NS rows)."""
    rng = _rng(w.input_seed, (b,))
    s = _s_rows(w, rng, w.l_s)
    ns = _normal(rng, (w.model.l_ns, w.model.d_model))
    return _maybe_round(np.concatenate([s, ns], axis=0), w.model.dtype)


def forward_batch(w: Workload, samples: Optional[Sequence[int]] = None) -> np.ndarray:
    idx = range(w.batch) if samples is None else samples
    return np.stack([forward_sample(w, b) for b in idx])


def user_sequence(w: Workload, u: int) -> np.ndarray:
    """S rows of user u: [L_S][d] (two-stage: with [SEP] rows; append: old + new rows in time order)."""
    rng = _rng(w.input_seed, (0, u))
    return _maybe_round(_s_rows(w, rng, w.l_s if w.kind != "append" else w.l_old + w.d_l), w.model.dtype)


def user_sequences(w: Workload, users: Optional[Sequence[int]] = None) -> np.ndarray:
    idx = range(w.n_users) if users is None else users
    return np.stack([user_sequence(w, u) for u in idx])


def candidate_tokens(w: Workload, u: int, c: int) -> np.ndarray:
    """NS tokens of candidate c of user u: [L_NS][d] ~ N(0, 1)."""
    rng = _rng(w.input_seed, (1, u * max(w.n_cand, 1) + c))
    return _maybe_round(_normal(rng, (w.model.l_ns, w.model.d_model)), w.model.dtype)


def candidate_batch(w: Workload, users: Optional[Sequence[int]] = None,
                    cands: Optional[Sequence[int]] = None) -> np.ndarray:
    """[U][C][L_NS][d]."""
    us = range(w.n_users) if users is None else users
    cs = range(w.n_cand) if cands is None else cands
    return np.stack([np.stack([candidate_tokens(w, u, c) for c in cs]) for u in us])


def append_rows(w: Workload, u: int):
    """(old rows [l_old][d], new rows [d_l][d]) of user u for the append workload."""
    s = user_sequence(w, u)
    return s[: w.l_old], s[w.l_old:]


def user_cached_lengths(w: Workload) -> list:
    """Ragged append: each user's cached rows before the append, uniform in [l_old_min, l_old]
    (every user has l_old when l_old_min is 0)."""
    if not w.l_old_min:
        return [w.l_old] * w.n_users
    rng = _rng(w.input_seed, (2,))
    return [int(x) for x in rng.integers(w.l_old_min, w.l_old + 1, size=w.n_users)]


def append_batch(w: Workload, users: Optional[Sequence[int]] = None):
    us = range(w.n_users) if users is None else users
    s = np.stack([user_sequence(w, u) for u in us])
    return s[:, : w.l_old], s[:, w.l_old:]


def grad_out_sample(w: Workload, b: int) -> np.ndarray:
    """Training step: the loss gradient of sample b's final rows, [q_last + L_NS][d] fp32, N(0,1)."""
    rng = _rng(w.input_seed, (3, b))
    return _normal(rng, (w.s_queries[-1] + w.model.l_ns, w.model.d_model))


def grad_out_batch(w: Workload, samples: Optional[Sequence[int]] = None) -> np.ndarray:
    idx = range(w.batch) if samples is None else samples
    return np.stack([grad_out_sample(w, b) for b in idx])
