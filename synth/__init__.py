"""Seeded synthetic inputs and workload shapes for the OneTrans block stack.

This package is shared by the CPU oracle, the tests and the benchmark. It only
draws random numbers and lays them out; it holds none of the method's
arithmetic (no norm, projection, attention or FFN code).

Shapes follow the OneTrans pages (fun-rec-mdbook, "OneTrans", section 7.5.0
"Unified Tokenization": X(0) = [S-tokens; NS-tokens], S rows first) and the
five workloads this project is measured on. Value distributions:

* model matrices and biases ~ N(0, 0.02^2) (std 0.02);
* norm gains gamma = 1 + 0.02 * N(0, 1), norm shifts beta = 0.02 * N(0, 1)
  (non-trivial so that a dropped gain/shift shows up in parity);
* event embeddings and NS-token vectors ~ N(0, 1);
* one learnable-[SEP] stand-in vector per sequence boundary, drawn once per
  model and shared by every sample (section 7.5.0, timestamp-agnostic merge:
  sequences in intent order order > cart > click, a [SEP] after each).

Every sample / user / candidate draws from its own child stream of a
``numpy.random.SeedSequence``, so any single one can be regenerated alone.
"""

from .shapes import (ModelShape, Workload, WORKLOADS, TEST_SHAPES, linear_pyramid,
                     workload, test_workload)
from .gen import (round_bf16, bf16_bits, BlockWeights, make_weights, sep_vectors,
                  forward_sample, forward_batch, user_sequence, user_sequences,
                  candidate_tokens, candidate_batch, append_rows, append_batch,
                  user_cached_lengths, grad_out_sample, grad_out_batch)

from .tokenizer import (TokWorkload, TOK_WORKLOADS, tok_workload, tokenizer_weights, tokenizer_sample,
                        tokenizer_batch, tokenizer_times, tokenizer_times_batch)

__all__ = [
    "TokWorkload", "TOK_WORKLOADS", "tok_workload", "tokenizer_weights", "tokenizer_sample", "tokenizer_batch",
    "tokenizer_times", "tokenizer_times_batch",
    "ModelShape", "Workload", "WORKLOADS", "TEST_SHAPES", "linear_pyramid", "workload",
    "test_workload", "round_bf16", "bf16_bits", "BlockWeights", "make_weights", "sep_vectors",
    "forward_sample", "forward_batch", "user_sequence", "user_sequences", "candidate_tokens",
    "candidate_batch", "append_rows", "append_batch", "user_cached_lengths", "grad_out_sample", "grad_out_batch",
]
