"""Acceptance statistics and adaptive draft-length controllers: the reference
the GPU versions are checked against.  TEST INFRASTRUCTURE ONLY: used by
tests/, smoke() and the cpu_baseline leg of bench.py, never by the library.

Statistics ("5.2 Draft 模型与无模型方案", AIInfraGuide, section 7).  Over an
observation window of R verify rounds that proposed D draft tokens, of which
C were accepted:
  * draft acceptance rate C / D                                    (7.1)
  * mean acceptance length 1 + C / R (each complete round also commits a
    corrected or bonus token)                                       (7.1)
  * candidate coverage: the share of rounds that had any candidate  (7.1)
  * with a fixed proposal length gamma, D = gamma * R and the mean length is
    1 + gamma * C / D; with dynamic lengths the real D and R are used (7.2)
  * per position i, the conditional acceptance rate (accepted at i among
    rounds that reached i with a proposal there) differs from the rate of
    being accepted all the way through i (among rounds that proposed i) (7.2)

Counters.  A round is one sequence of one verify call: K = proposed draft
tokens, A = accepted ones (0..K), A = -1 when the call did not verify it.
  [0] R  rounds counted               [4] rounds with K > 0 and A = K (bonus)
  [1] D  = sum K                      [5] rounds not counted (A < 0, K outside
  [2] C  = sum A                          0..max_k, or A > K)
  [3] rounds with K > 0 (candidates)  [6] emitted tokens = sum (A + 1)
                                      [7] 0
  [8 + i]            proposed_i = #rounds with K > i
  [8 + max_k + i]    reached_i  = #rounds with K > i and A >= i
  [8 + 2 max_k + i]  accepted_i = #rounds with A > i
Summary (float64; NaN where a denominator is 0):
  [0] C / D  [1] 1 + C / R  [2] coverage [3] / R  [3] bonus share [4] / [3]
  [4 + i]          conditional acceptance accepted_i / reached_i
  [4 + max_k + i]  accepted through i      accepted_i / proposed_i

Controllers, one per sequence, fed after every round with (K, A); a round
with A < 0 leaves the state alone.  Readings where the pages leave a point
open: the ratio a controller sees is A / max(K, 1), accepted DRAFT tokens
only (the section 7 C); the tutorial's decoder counts the corrected token
too, which makes a round with a rejection look fully accepted.
  window          (gitcode.csdn.net tutorial, section 5.2 动态草稿长度策略):
                  keep the last `window` ratios; once at least `min_samples`
                  are held, compare their mean (summed oldest first) with
                  target +- 0.1 and move the length by one within
                  [min_k, max_k].
  multiplicative  (same tutorial, section 4.4 完整的解码器): above target + 0.1
                  the length becomes min(max_k, int(L * (1 + rate))), below
                  target - 0.1 max(min_k, int(L * (1 - rate))); int truncates.
  optimal_k       (wmrh.cn, "Speculative Decoding在分布式推理中的应用",
                  section 三, adapt_draft_length): with a = max(ratio, 0.01),
                  k* = floor(ln(1 / (1 - a)) / a) (infinite at a = 1), and
                  L becomes min(clamp(k*, 2, 16), max(L, 2)).
All arithmetic in float64, in the order written above.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List

import numpy as np

WINDOW, MULTIPLICATIVE, OPTIMAL_K = 0, 1, 2
BAND = 0.1


def acceptance_counters(num_draft, accepted_len, max_k: int, into=None) -> np.ndarray:
    """Add one call's rounds to the counters (a fresh array when `into` is None)."""
    c = np.zeros(8 + 3 * max_k, dtype=np.uint64) if into is None else into
    for K, A in zip(np.asarray(num_draft).tolist(), np.asarray(accepted_len).tolist()):
        if A < 0 or K < 0 or K > max_k or A > K:
            c[5] += 1
            continue
        c[0] += 1
        c[1] += K
        c[2] += A
        c[3] += K > 0
        c[4] += K > 0 and A == K
        c[6] += A + 1
        for i in range(K):
            c[8 + i] += 1
            if A >= i:
                c[8 + max_k + i] += 1
            if A > i:
                c[8 + 2 * max_k + i] += 1
    return c


def _ratio(num, den) -> float:
    return float(num) / float(den) if den else math.nan


def acceptance_summary(c, max_k: int) -> np.ndarray:
    c = [int(x) for x in c]
    R, D, C = c[0], c[1], c[2]
    out = np.full(4 + 2 * max_k, math.nan)
    out[0] = _ratio(C, D)
    out[1] = 1.0 + C / R if R else math.nan
    out[2] = _ratio(c[3], R)
    out[3] = _ratio(c[4], c[3])
    for i in range(max_k):
        out[4 + i] = _ratio(c[8 + 2 * max_k + i], c[8 + max_k + i])
        out[4 + max_k + i] = _ratio(c[8 + 2 * max_k + i], c[8 + i])
    return out


@dataclass
class Controller:
    """One sequence's controller state."""
    length: int
    window: List[float] = field(default_factory=list)


def adapt_step(st: Controller, K: int, A: int, kind: int, *, min_k: int, max_k: int, window: int = 100,
               min_samples: int = 10, target: float = 0.7, rate: float = 0.1) -> int:
    """Feed one round (K proposed, A accepted) and return the next length."""
    if A < 0:
        return st.length
    ratio = A / max(K, 1)
    if kind == WINDOW:
        st.window.append(ratio)
        if len(st.window) > window:
            st.window.pop(0)
        if len(st.window) >= min_samples:
            acc = 0.0
            for r in st.window:
                acc += r
            avg = acc / len(st.window)
            if avg > target + BAND:
                st.length = min(max_k, st.length + 1)
            elif avg < target - BAND:
                st.length = max(min_k, st.length - 1)
    elif kind == MULTIPLICATIVE:
        if ratio > target + BAND:
            st.length = min(max_k, int(st.length * (1 + rate)))
        elif ratio < target - BAND:
            st.length = max(min_k, int(st.length * (1 - rate)))
    elif kind == OPTIMAL_K:
        a = max(ratio, 0.01)
        x = math.log(1.0 / (1.0 - a)) / a if a < 1.0 else math.inf
        k = 16 if x >= 16 else max(2, int(x))
        st.length = min(k, max(st.length, 2))
    else:
        raise ValueError(f"unknown controller kind {kind}")
    return st.length


def adapt_batch(states: List[Controller], num_draft, accepted_len, kind: int, **kw) -> np.ndarray:
    """One round for every sequence of a batch; returns the next lengths."""
    return np.array([adapt_step(s, int(K), int(A), kind, **kw)
                     for s, K, A in zip(states, np.asarray(num_draft), np.asarray(accepted_len))], dtype=np.int32)
