"""Seeded synthetic inputs for the batched speculative-decoding verify step
for the N-gram proposer that feeds its one-hot mode, and verify-round
outcomes for the acceptance statistics and draft-length controllers.

This package produces the *inputs* of the verify step (logits rows, proposed
tokens, per-sequence draft lengths, temperatures and modes) and of the
proposer (ragged token histories), and nothing else.
It holds none of the verify arithmetic (no softmax, no acceptance test, no
residual sampling), so that the CPU oracle and the HIP library can both be fed
from it without sharing any of the method's code.
"""
from .synth import (  # noqa: F401
    MODE_SAMPLE, MODE_GREEDY, MODE_ONEHOT, MODE_STRICT, Batch, CONFIG_NAMES, STRICT_SUFFIX,
    make_config_batch, make_random_batch, bf16_round, bf16_widen,
    config_description, NgramBatch, NGRAM_WORKLOAD, make_ngram_batch, make_ngram_workload,
    ROUNDS_WORKLOAD, make_rounds_workload, sequence_slice,
)
