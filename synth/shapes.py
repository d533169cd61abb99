"""Model shapes and workloads (sizes only, no arithmetic of the method).

Block notation used across the project: block n (0-based here) takes s_n S rows
plus l_ns NS rows and keeps the tail q_n S rows plus all NS rows
(fun-rec-mdbook "OneTrans", section 7.5.2 "Pyramid Stack": queries are the tail
index set, keys/values span every input row of the block). s_0 = L_S and
s_{n+1} = q_n.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


def linear_pyramid(l_s: int, q_min: int, n_blocks: int) -> Tuple[int, ...]:
    """Linear pyramid schedule: q_n = L_S - floor(n (L_S - q_min) / (N - 1)).

    The pages print a halving example 1190 -> 595 -> 297 -> ... -> 12
    (section 7.5.2) that cannot land on 12 exactly; the workloads ask for a
    linear shrink, so block 0 keeps every S row and the last keeps q_min.
    """
    if n_blocks == 1:
        return (l_s,)
    return tuple(l_s - (n * (l_s - q_min)) // (n_blocks - 1) for n in range(n_blocks))


@dataclass(frozen=True)
class ModelShape:
    """Architecture of a OneTrans block stack."""
    name: str
    n_blocks: int
    d_model: int
    n_heads: int
    d_ff: int
    l_ns: int
    norm: str            # "rms" or "layer"
    norm_eps: float
    dtype: str           # storage dtype of X(0), weights and the K/V cache: "f32" or "bf16"
    weight_seed: int
    sep_seed: int

    @property
    def d_head(self) -> int:
        return self.d_model // self.n_heads

    @property
    def n_groups(self) -> int:
        """Weight groups per matrix: index 0 is the shared S set, 1+j is NS token j."""
        return 1 + self.l_ns


@dataclass(frozen=True)
class Workload:
    """One measured / tested configuration."""
    key: str
    description: str
    model: ModelShape
    kind: str                          # "forward", "two_stage", "append" or "train"
    l_s: int
    s_queries: Tuple[int, ...]         # q_n per block
    seq_lens: Tuple[int, ...] = ()     # behaviour sequences in merge order (each followed by [SEP])
    batch: int = 0                     # forward: samples (one candidate each)
    n_users: int = 0                   # two_stage / append
    n_cand: int = 0                    # candidates per user
    l_old: int = 0                     # append: cached rows before the append
    d_l: int = 0                       # append: new rows
    l_old_min: int = 0                 # ragged append: users' cached rows drawn uniformly from
                                       # [l_old_min, l_old] (0: every user has l_old)
    input_seed: int = 0
    parity_subset: Tuple[int, ...] = field(default_factory=tuple)

    @property
    def sep_rows(self) -> Tuple[int, ...]:
        """Row indices of the [SEP] rows inside the S-tokens (one after each sequence)."""
        rows, pos = [], 0
        for n in self.seq_lens:
            pos += n
            rows.append(pos)
            pos += 1
        return tuple(rows)

    def with_dtype(self, dtype: str) -> "Workload":
        return replace(self, model=replace(self.model, dtype=dtype))


def _cfg(i: int, **kw) -> ModelShape:
    return ModelShape(weight_seed=1000 + i, sep_seed=3000 + i, **kw)


_TINY = _cfg(1, name="tiny", n_blocks=1, d_model=64, n_heads=4, d_ff=256, l_ns=4,
             norm="layer", norm_eps=1e-5, dtype="f32")
_ONETRANS_S = _cfg(2, name="OneTransS-shaped", n_blocks=6, d_model=256, n_heads=8, d_ff=1024,
                   l_ns=16, norm="rms", norm_eps=1e-6, dtype="bf16")
_ONETRANS_L = _cfg(5, name="OneTransL-shaped", n_blocks=8, d_model=512, n_heads=16, d_ff=2048,
                   l_ns=16, norm="rms", norm_eps=1e-6, dtype="bf16")

_S_PYR = linear_pyramid(1190, 12, 6)
_L_PYR = linear_pyramid(2048, 32, 8)

WORKLOADS = {
    "tiny": Workload(
        key="tiny", description="1 block, d=64, 4 heads, FFN 256, LayerNorm; L_S=32, L_NS=4; batch 8; fp32",
        model=_TINY, kind="forward", l_s=32, s_queries=(32,), seq_lens=(15, 15), batch=8,
        input_seed=2001, parity_subset=tuple(range(8))),
    "onetrans_s": Workload(
        key="onetrans_s",
        description="OneTransS-shaped forward: 6 blocks, d=256, 8 heads, FFN 1024; L_S=1190, L_NS=16; "
                    "pyramid 1190->12 linear; batch 256; bf16 storage, fp32 accumulation",
        model=_ONETRANS_S, kind="forward", l_s=1190, s_queries=_S_PYR, seq_lens=(187, 200, 800),
        batch=256, input_seed=2002, parity_subset=(0, 1, 37, 101, 128, 199, 254, 255)),
    "two_stage": Workload(
        key="two_stage",
        description="Two-stage KV cache on the OneTransS-shaped model: Stage I encodes 64 users "
                    "(L_S=1190, pyramid); Stage II scores 512 candidates/user x 16 NS tokens; bf16",
        model=_ONETRANS_S, kind="two_stage", l_s=1190, s_queries=_S_PYR, seq_lens=(187, 200, 800),
        n_users=64, n_cand=512, input_seed=2003, parity_subset=(0, 63)),
    "append": Workload(
        key="append",
        description="Cross-request append on the OneTransS-shaped model without pyramid: 128 users, "
                    "1158 cached rows, append 32 new rows, 1 candidate/user; bf16",
        model=_ONETRANS_S, kind="append", l_s=1190, s_queries=(1190,) * 6, n_users=128, n_cand=1,
        l_old=1158, d_l=32, input_seed=2004, parity_subset=(0, 1, 64, 127)),
    "append_ragged": Workload(
        key="append_ragged",
        description="Cross-request append with ragged users on the OneTransS-shaped model without pyramid: "
                    "128 users with 579..1158 cached rows (uniform), append 32 new rows, 1 candidate/user; bf16",
        model=_ONETRANS_S, kind="append", l_s=1190, s_queries=(1190,) * 6, n_users=128, n_cand=1,
        l_old=1158, d_l=32, l_old_min=579, input_seed=2005, parity_subset=(0, 1, 64, 127)),
    "append_pyramid": Workload(
        key="append_pyramid",
        description="Cross-request append on the OneTransS-shaped model with its pyramid: 128 users whose 1158 "
                    "cached rows were prefilled with the schedule 1158->955->719->484->248->12, append 32 new rows "
                    "(the schedule grows to 1190->955->...->12: blocks 3-6 are recomputed over their slid windows), "
                    "1 candidate/user; bf16",
        model=_ONETRANS_S, kind="append", l_s=1190, s_queries=(1158, 955, 719, 484, 248, 12), n_users=128, n_cand=1,
        l_old=1158, d_l=32, input_seed=2006, parity_subset=(0, 127)),
    "train_s": Workload(
        key="train_s",
        description="Training step on the OneTransS-shaped model: the forward over the batch keeping each "
                    "block's input rows, then the backward with activation recomputation (gradients of "
                    "X(0) and of every parameter, per weight set); batch 256, L_S=1190, pyramid 1190->12; "
                    "bf16 storage, fp32 accumulation and gradients",
        model=_ONETRANS_S, kind="train", l_s=1190, s_queries=_S_PYR, seq_lens=(187, 200, 800),
        batch=256, input_seed=2007, parity_subset=(0, 255)),
    "onetrans_l": Workload(
        key="onetrans_l",
        description="OneTransL-shaped forward: 8 blocks, d=512, 16 heads, FFN 2048; L_S=2048, L_NS=16; "
                    "pyramid 2048->32 linear; batch 512; bf16 storage, fp32 accumulation",
        model=_ONETRANS_L, kind="forward", l_s=2048, s_queries=_L_PYR, seq_lens=(245, 400, 1400),
        batch=512, input_seed=2005, parity_subset=(0, 200, 511, 333)),
}

# Small multi-block shapes for invariants that need several blocks and a pyramid.
_T3 = ModelShape(name="tiny3", n_blocks=3, d_model=64, n_heads=4, d_ff=256, l_ns=4, norm="rms",
                 norm_eps=1e-6, dtype="f32", weight_seed=1100, sep_seed=3100)
TEST_SHAPES = {
    "tiny3_fwd": Workload(key="tiny3_fwd", description="3 blocks, pyramid 32->20->8", model=_T3,
                          kind="forward", l_s=32, s_queries=(32, 20, 8), seq_lens=(10, 9, 10),
                          batch=4, input_seed=2100),
    "tiny3_two_stage": Workload(key="tiny3_two_stage", description="3 blocks, 2 users x 3 candidates",
                                model=_T3, kind="two_stage", l_s=32, s_queries=(32, 20, 8),
                                seq_lens=(10, 9, 10), n_users=2, n_cand=3, input_seed=2101),
    "tiny3_append": Workload(key="tiny3_append", description="3 blocks, no pyramid, 24 + 8 rows",
                             model=_T3, kind="append", l_s=32, s_queries=(32, 32, 32), n_users=2,
                             n_cand=1, l_old=24, d_l=8, input_seed=2102),
}


def workload(key: str, dtype: str | None = None) -> Workload:
    w = WORKLOADS[key]
    return w.with_dtype(dtype) if dtype else w


def test_workload(key: str, dtype: str | None = None) -> Workload:
    w = TEST_SHAPES[key]
    return w.with_dtype(dtype) if dtype else w
