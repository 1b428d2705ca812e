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
with A < 0 leaves the state alone.  The ratio a controller sees, by default,
is the tutorial's own: its verifier (gitcode.csdn.net tutorial, section 4.3
验证器实现) returns the accepted draft tokens plus the token drawn after a
rejection (no bonus token), and its decoder (section 4.4 完整的解码器) feeds
len(accepted_tokens) / draft_len, 0 when nothing was proposed; so the count
is min(A + 1, K).  "Speculative Decoding在分布式推理中的应用" (wmrh.cn),
section 三, counts the same way (the resampled token still counts as
produced).  COUNT_DRAFT_ONLY gives A / max(K, 1) instead (the section 7 C).
  window          (tutorial, section 5.2 动态草稿长度策略): the mean of the
                  most recent `window` ratios, once at least `min_samples`
                  are held, moves the length one step up above target + 0.1
                  and one step down below target - 0.1, within [min_k, max_k].
  multiplicative  (tutorial, section 4.4): the ratio of the round itself moves
                  the length to int(L * (1 + rate)) (at most max_k) above
                  target + 0.1, to int(L * (1 - rate)) (at least min_k) below
                  target - 0.1; int truncates.
  optimal_k       (wmrh.cn, section 三, adapt_draft_length): with
                  a = max(ratio, 0.01), k* = floor(ln(1 / (1 - a)) / a)
                  (infinite at a = 1), and L becomes min(clamp(k*, 2, 16),
                  max(L, 2)).
All arithmetic in float64; a mean is summed oldest first, as a plain sum
over a list of the window's ratios is.
"""
from __future__ import annotations

import math
from collections import deque
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


COUNT_EMITTED, COUNT_DRAFT_ONLY = 0, 1


def controller_ratio(K: int, A: int, count: int = COUNT_EMITTED) -> float:
    """The acceptance ratio of one round as a controller sees it."""
    if count == COUNT_EMITTED:
        return min(A + 1, K) / K if K > 0 else 0.0
    if count == COUNT_DRAFT_ONLY:
        return A / max(K, 1)
    raise ValueError(f"unknown count {count}")


@dataclass
class Controller:
    """One sequence's controller state: its length and, for the window rule,
    the most recent ratios (oldest first)."""
    length: int
    recent: deque = field(default_factory=deque)


def _band(v: float, target: float) -> int:
    """+1 above the dead band around the target, -1 below it, 0 inside."""
    return 1 if v > target + BAND else (-1 if v < target - BAND else 0)


def _move(L: int, direction: int, up: int, down: int, min_k: int, max_k: int) -> int:
    """The new length: `up` capped at max_k, `down` floored at min_k, or L."""
    if direction > 0:
        return min(max_k, up)
    if direction < 0:
        return max(min_k, down)
    return L


def adapt_step(st: Controller, K: int, A: int, kind: int, *, min_k: int, max_k: int, window: int = 100,
               min_samples: int = 10, target: float = 0.7, rate: float = 0.1, count: int = COUNT_EMITTED) -> int:
    """Feed one round (K proposed, A accepted) and return the next length."""
    if A < 0:
        return st.length
    ratio = controller_ratio(K, A, count)
    L = st.length
    if kind == WINDOW:
        st.recent.append(ratio)
        while len(st.recent) > window:
            st.recent.popleft()
        if len(st.recent) >= min_samples:
            mean = sum(st.recent) / len(st.recent)
            L = _move(L, _band(mean, target), L + 1, L - 1, min_k, max_k)
    elif kind == MULTIPLICATIVE:
        L = _move(L, _band(ratio, target), int(L * (1 + rate)), int(L * (1 - rate)), min_k, max_k)
    elif kind == OPTIMAL_K:
        a = max(ratio, 0.01)
        x = math.log(1.0 / (1.0 - a)) / a if a < 1.0 else math.inf
        L = min(16 if x >= 16 else max(2, int(x)), max(L, 2))
    else:
        raise ValueError(f"unknown controller kind {kind}")
    st.length = L
    return L


def adapt_batch(states: List[Controller], num_draft, accepted_len, kind: int, **kw) -> np.ndarray:
    """One round for every sequence of a batch; returns the next lengths."""
    return np.array([adapt_step(s, int(K), int(A), kind, **kw)
                     for s, K, A in zip(states, np.asarray(num_draft), np.asarray(accepted_len))], dtype=np.int32)
