"""CPU oracle for the OneTrans block stack (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the HIP library and its
Python binding) never imports, calls or links anything here.
"""

from .onetrans_oracle import (rms_norm, layer_norm, norm, gelu, weight_group, block_forward,
                              forward, forward_batch, prefill_user, score_candidate,
                              append_events, append_recompute, grown_schedule, BlockTrace)
from .tokenizer_oracle import mlp, s_tokens, s_tokens_by_time, ns_tokens, tokenize, tokenize_batch
from .onetrans_backward import backward, backward_batch

__all__ = ["mlp", "s_tokens", "s_tokens_by_time", "ns_tokens", "tokenize", "tokenize_batch",
           "rms_norm", "layer_norm", "norm", "gelu", "weight_group", "block_forward", "forward",
           "forward_batch", "prefill_user", "score_candidate", "append_events", "append_recompute",
           "grown_schedule", "BlockTrace", "backward", "backward_batch"]
