"""CPU oracle of the batched speculative-decoding verify step, of the
N-gram (prompt-lookup) proposer that feeds its one-hot mode, and of the
acceptance statistics and draft-length controllers fed by its results.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 statement
of what the verify step computes, used to check the HIP library.  Only the
test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it.  It shares no code with the library: its own
Philox4x32-10, its own softmax, its own bfloat16 widening.

Every function here is pinned by CPU tests against facts the source pages
or mathematics fix (worked example, losslessness, the acceptance law,
one-hot and greedy special cases, brute force over the uniform grid,
published Philox known-answer vectors and an independent Philox
implementation).
"""
from .philox import philox4x32_10, philox4x32_10_np, u24, verify_uniform, verify_uniforms_np  # noqa: F401
from .verify import (  # noqa: F401
    SAMPLE, GREEDY, ONEHOT, STRICT,
    ST_BAD_LAYOUT, ST_K_TOO_LARGE, ST_BAD_MODE, ST_BAD_TEMPERATURE, ST_NO_DRAFT_LOGITS,
    ST_BAD_TOKEN, ST_NONFINITE, ST_ZERO_RESIDUAL, ST_ERROR_MASK,
    BAND, BatchResult, SeqResult, softmax, accept_ratio, residual, inverse_cdf, widen,
    verify_sequence, verify_batch, verify_batch_from, cdf_interval, strict_correction,
)
from .compare import CompareReport, compare  # noqa: F401
from .ngram import ngram_propose, ngram_propose_batch, valid_starts  # noqa: F401
from .stats import (  # noqa: F401
    WINDOW, MULTIPLICATIVE, OPTIMAL_K, COUNT_EMITTED, COUNT_DRAFT_ONLY, Controller, acceptance_counters,
    acceptance_summary, adapt_step, adapt_batch, controller_ratio,
)
from .filter import filter_threshold, filtered_softmax, kept_by_definition, topk_threshold  # noqa: F401
