"""Shapes and seeded inputs of the tokenizers ahead of block 1 (sizes and random numbers only).

fun-rec-mdbook "OneTrans", section 7.5.0 "Unified Tokenization": every behaviour sequence type i
has events of its own raw width D_i that a behaviour-specific MLP maps to d; the non-sequential
features are concatenated (width F) and one MLP maps them to L_NS * d values. The pages give no
raw widths or hidden widths, so the workloads below choose them (multiples of 64, in the range of
item-ID plus side-information embeddings); the behaviour sequence lengths and L_NS are those of
the block workloads.

Timestamps (timestamp-aware merge): each behaviour type logs events at its own rate; a sample's
sequence of type i starts at a uniform offset in [0, 1000) s and advances by geometric gaps of mean
about (i + 1) * 20 s, clipped at 0 so that some events share a time (ties across and within types).

Value distributions: raw event embeddings and NS features ~ N(0, 1); MLP matrices
~ N(0, 1 / fan_in) so that pre-activations are O(1) and the GELU works in its curved range;
biases ~ N(0, 0.1^2); the [SEP] rows are the model's seeded [SEP] vectors (one per sequence); in the
timestamp-aware merge the same vectors serve as the behaviour-type embeddings.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Sequence, Tuple

import numpy as np

from .gen import _maybe_round, _normal, sep_vectors
from .shapes import WORKLOADS, ModelShape, TEST_SHAPES


@dataclass(frozen=True)
class TokWorkload:
    key: str
    description: str
    model: ModelShape
    seq_lens: Tuple[int, ...]      # events per sample of each behaviour type, merge order
    seq_dims: Tuple[int, ...]      # raw event width D_i
    seq_hidden: Tuple[int, ...]    # hidden width of MLP_i
    ns_dim: int                    # width of Concat(NS)
    ns_hidden: int                 # hidden width of the Auto-Split MLP
    batch: int
    input_seed: int
    weight_seed: int
    parity_subset: Tuple[int, ...] = field(default_factory=tuple)
    merge: str = "intent"          # "intent": [SEP] after each sequence; "time": interleaved by time

    @property
    def l_s(self) -> int:
        return sum(self.seq_lens) + (len(self.seq_lens) if self.merge == "intent" else 0)

    @property
    def n_seq(self) -> int:
        return len(self.seq_lens)

    def with_dtype(self, dtype: str) -> "TokWorkload":
        return replace(self, model=replace(self.model, dtype=dtype))

    def with_model(self, **kw) -> "TokWorkload":
        return replace(self, model=replace(self.model, **kw))


_MID = ModelShape(name="tok_mid", n_blocks=1, d_model=128, n_heads=4, d_ff=256, l_ns=3, norm="rms",
                  norm_eps=1e-6, dtype="f32", weight_seed=1200, sep_seed=3200)

TOK_WORKLOADS = {
    "tok_tiny": TokWorkload(
        key="tok_tiny", description="tiny model (d=64, L_NS=4): sequences 15 + 15 events of widths 64 / 128",
        model=TEST_SHAPES["tiny3_fwd"].model, seq_lens=(15, 15), seq_dims=(64, 128), seq_hidden=(128, 64),
        ns_dim=192, ns_hidden=128, batch=8, input_seed=2200, weight_seed=1300),
    "tok_mid": TokWorkload(
        key="tok_mid", description="d=128, L_NS=3: four sequences of 37, 0, 100 and 5 events (one empty), "
                                   "ragged row tiles; NS features 320 wide",
        model=_MID, seq_lens=(37, 0, 100, 5), seq_dims=(128, 64, 192, 64), seq_hidden=(192, 64, 128, 256),
        ns_dim=320, ns_hidden=192, batch=5, input_seed=2201, weight_seed=1301),
    "tokenize_s": TokWorkload(
        key="tokenize_s",
        description="Tokenizers of the OneTransS-shaped model: batch 256; behaviour sequences order 187, "
                    "cart 200, click 800 events of raw widths 128 / 128 / 64, MLP_i hidden 256 -> d=256; "
                    "Auto-Split MLP 1024 -> 1024 -> 16 x 256; bf16 storage, fp32 accumulation",
        model=WORKLOADS["onetrans_s"].model, seq_lens=(187, 200, 800), seq_dims=(128, 128, 64),
        seq_hidden=(256, 256, 256), ns_dim=1024, ns_hidden=1024, batch=256, input_seed=2202,
        weight_seed=1302, parity_subset=(0, 77, 255)),
}
TOK_WORKLOADS["tok_mid_time"] = replace(TOK_WORKLOADS["tok_mid"], key="tok_mid_time", merge="time",
                                        description="tok_mid with the timestamp-aware merge")
TOK_WORKLOADS["tokenize_s_time"] = replace(
    TOK_WORKLOADS["tokenize_s"], key="tokenize_s_time", merge="time",
    description=TOK_WORKLOADS["tokenize_s"].description + "; timestamp-aware merge (events interleaved by "
                                                          "time, type embeddings added, no [SEP])")


def tok_workload(key: str, dtype: Optional[str] = None) -> TokWorkload:
    w = TOK_WORKLOADS[key]
    return w.with_dtype(dtype) if dtype else w


def _rng(seed: int, key: Sequence[int]) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def _mlp_weights(rng: np.random.Generator, d_in: int, hidden: int, d_out: int, dtype: str) -> dict:
    p = dict(w1=_normal(rng, (hidden, d_in), 1.0 / np.sqrt(d_in)), b1=_normal(rng, (hidden,), 0.1),
             w2=_normal(rng, (d_out, hidden), 1.0 / np.sqrt(hidden)), b2=_normal(rng, (d_out,), 0.1))
    return {k: _maybe_round(v.astype(np.float32), dtype) for k, v in p.items()}


def tokenizer_weights(w: TokWorkload) -> dict:
    """{"seq": [MLP_i weights], "sep": [n_seq][d], "ns": Auto-Split MLP weights or None}."""
    m = w.model
    seq = [_mlp_weights(_rng(w.weight_seed, (i,)), w.seq_dims[i], w.seq_hidden[i], m.d_model, m.dtype)
           for i in range(w.n_seq)]
    ns = None
    if m.l_ns > 0:
        ns = _mlp_weights(_rng(w.weight_seed, (100,)), w.ns_dim, w.ns_hidden, m.l_ns * m.d_model, m.dtype)
    sep = _maybe_round(sep_vectors(m, w.n_seq), m.dtype)
    return {"seq": seq, "sep": sep, "ns": ns}


def tokenizer_sample(w: TokWorkload, b: int):
    """Raw inputs of sample b: ([events_i [L_i][D_i]], ns_feat [F])."""
    rng = _rng(w.input_seed, (b,))
    ev = [_maybe_round(_normal(rng, (w.seq_lens[i], w.seq_dims[i])), w.model.dtype) for i in range(w.n_seq)]
    ns = _maybe_round(_normal(rng, (w.ns_dim,)), w.model.dtype)
    return ev, ns


def tokenizer_times(w: TokWorkload, b: int):
    """Timestamps of sample b: [times_i [L_i] int64, non-decreasing within each type]."""
    rng = _rng(w.input_seed, (b, 7))
    out = []
    for i, L in enumerate(w.seq_lens):
        start = int(rng.integers(0, 1000))
        gaps = np.maximum(rng.geometric(1.0 / (20.0 * (i + 1)), size=L) - 2, 0)
        out.append((start + np.cumsum(gaps)).astype(np.int64))
    return out


def tokenizer_times_batch(w: TokWorkload, samples: Optional[Sequence[int]] = None):
    samples = range(w.batch) if samples is None else samples
    per = [tokenizer_times(w, b) for b in samples]
    return [np.stack([p[i] for p in per]) for i in range(w.n_seq)]


def tokenizer_batch(w: TokWorkload, samples: Optional[Sequence[int]] = None):
    """Batched raw inputs: ([events_i [B][L_i][D_i]], ns_feat [B][F])."""
    samples = range(w.batch) if samples is None else samples
    per = [tokenizer_sample(w, b) for b in samples]
    ev = [np.stack([p[0][i] for p in per]) for i in range(w.n_seq)]
    ns = np.stack([p[1] for p in per])
    return ev, ns
