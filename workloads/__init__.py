"""Seeded synthetic inputs for the batched speculative-decoding verify step.

This package produces the *inputs* of the verify step (logits rows, proposed
tokens, per-sequence draft lengths, temperatures and modes) and nothing else.
It holds none of the verify arithmetic (no softmax, no acceptance test, no
residual sampling), so that the CPU oracle and the HIP library can both be fed
from it without sharing any of the method's code.
"""
from .synth import (  # noqa: F401
    MODE_SAMPLE, MODE_GREEDY, MODE_ONEHOT, Batch, CONFIG_NAMES,
    make_config_batch, make_random_batch, bf16_round, bf16_widen,
    config_description,
)
