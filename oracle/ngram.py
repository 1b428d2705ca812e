"""N-gram (prompt-lookup) proposer: the reference the GPU proposer is checked
against.  TEST INFRASTRUCTURE ONLY: used by tests/, smoke() and the
cpu_baseline leg of bench.py, never by the library.

The method ("5.2 Draft 模型与无模型方案", AIInfraGuide, sections 4.1-4.3 and
the experiment of section 6): the last n token ids of a sequence's history
are looked up earlier in the same history; a hit proposes the tokens that
followed it, which a target model then verifies as a one-hot (deterministic)
proposal.  Matching is on token ids; n (the lookup window) and the proposal
length are separate parameters; longer windows are tried before shorter ones
and the most recent earlier occurrence is taken.

Readings (where the pages leave a point open):
  * a valid occurrence lies wholly before the current tail and leaves at
    least one token between its end and the start of the tail: with history
    h of length L and window n, a start s is valid iff s + n < L - n and
    h[s:s+n] == h[L-n:];
  * the proposal is h[s+n : min(s+n+max_tokens, L-n)]: it never copies from
    the tail itself;
  * the choice is the valid (n, s) with the largest n, then the largest s;
  * no valid pair (including L < 2*min_n + 1): no proposal.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np


def valid_starts(history: np.ndarray, n: int) -> np.ndarray:
    """Every start s with h[s:s+n] equal to the last n tokens and room for
    at least one continuation token before the tail (s + n < L - n)."""
    L = len(history)
    if n < 1 or 2 * n + 1 > L:
        return np.zeros(0, dtype=np.int64)
    tail = history[L - n:]
    last = L - 2 * n - 1                       # largest start with s + n < L - n
    ok = np.ones(last + 1, dtype=bool)
    for i in range(n):                          # compare position i of every window
        ok &= history[i:i + last + 1] == tail[i]
    return np.nonzero(ok)[0]


def ngram_propose(history: Sequence[int], min_n: int, max_n: int,
                  max_tokens: int) -> Tuple[Optional[int], List[int], Optional[int]]:
    """(window n, proposed tokens, start s) of the best valid occurrence, or
    (None, [], None).  Best = largest n in [min_n, max_n], then largest s."""
    h = np.asarray(history, dtype=np.int64)
    L = len(h)
    best = None
    for n in range(min_n, max_n + 1):
        starts = valid_starts(h, n)
        if len(starts):
            cand = (n, int(starts[-1]))
            if best is None or cand > best:
                best = cand
    if best is None or max_tokens < 1:
        return None, [], None
    n, s = best
    end = min(s + n + max_tokens, L - n)
    return n, [int(t) for t in h[s + n:end]], s


def ngram_propose_batch(history: np.ndarray, offsets: np.ndarray, min_n: int, max_n: int, max_tokens: int):
    """Per sequence b (tokens history[offsets[b]:offsets[b+1]]): the padded
    proposals [B, max_tokens] (-1 after the proposal), their lengths [B] and
    the matched window [B] (0 when there is none)."""
    B = len(offsets) - 1
    drafts = np.full((B, max_tokens), -1, dtype=np.int32)
    num = np.zeros(B, dtype=np.int32)
    win = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n, toks, _ = ngram_propose(history[offsets[b]:offsets[b + 1]], min_n, max_n, max_tokens)
        if n is not None:
            drafts[b, :len(toks)] = toks
            num[b] = len(toks)
            win[b] = n
    return drafts, num, win
