"""Top-k / top-p (nucleus) filtering of a verify row: the reference the GPU
filter is checked against.  TEST INFRASTRUCTURE ONLY: used by tests/,
smoke() and the cpu_baseline leg of bench.py, never by the library.

The pages list top-k and nucleus rejection sampling among the verification
strategies that keep the target's distribution ("Draft Model（草稿模型）",
compassingai.com, 常见误读纠偏 误读 4; the gitcode.csdn.net tutorial, section
5.4 采样策略对比) without giving formulas.  Readings taken here:

* the filter acts on each row's temperature softmax before the
  accept/correct rule, the same filter (same k and p) on the target row and
  on the draft row; the method then runs unchanged on the filtered,
  renormalised distributions p~ and q~, so the output follows p~;
* top-k: a token is kept iff fewer than k tokens have a strictly larger
  logit (ties at the k-th value are all kept); k <= 0 or k >= V: no top-k;
* top-p, applied after top-k on the renormalised top-k distribution: a
  token is kept iff the probability mass of the tokens with a strictly
  larger logit is below p; the tokens with the largest logit are always
  kept; p >= 1 (or NaN): no top-p;
* both are thresholds on the logit: keep iff x >= tau; greedy mode ignores
  the filter (the argmax is always kept).

Top-k membership depends only on comparisons of stored values and is exact.
Top-p membership depends on sums of probabilities: where the crossing of p
lies within BAND of the mass above a tie group or of the mass including it,
the neighbouring threshold is recorded as an equally valid alternative.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np

BAND = 1e-5


def topk_threshold(x: np.ndarray, k: int) -> float:
    """The k-th largest logit (counting equal values), or -inf when off."""
    V = len(x)
    if k <= 0 or k >= V:
        return -np.inf
    return float(np.sort(x)[::-1][k - 1])


def filter_threshold(x: np.ndarray, T: float, top_k: int, top_p: float) -> Tuple[float, List[float]]:
    """(tau, alternatives): keep the tokens with x >= tau.  ``x`` are the
    row's exact logits (float64), T the temperature."""
    tau_k = topk_threshold(x, int(top_k))
    tau = tau_k
    alts: List[float] = []
    if top_p < 1.0:                       # NaN compares false: no top-p
        kept = x[x >= tau_k]
        z = kept / T
        r = np.exp(z - z.max())
        r = r / r.sum()
        order = np.argsort(-kept, kind="stable")
        vals = kept[order]
        cum = np.cumsum(r[order])
        m = int(np.searchsorted(cum, top_p, side="left")) if top_p > 0 else 0
        m = min(m, len(vals) - 1)
        tau_p = float(vals[m])
        above = float(r[kept > tau_p].sum())
        incl = float(r[kept >= tau_p].sum())
        if top_p > 0 and top_p - above < BAND and (kept > tau_p).any():
            alts.append(float(kept[kept > tau_p].min()))     # the crossing may fall one group higher
        if incl - top_p < BAND and (kept < tau_p).any():
            alts.append(float(kept[kept < tau_p].max()))     # or one group lower
        tau = max(tau_k, tau_p)
        alts = [max(tau_k, a) for a in alts]
    return tau, alts


def filtered_softmax(x: np.ndarray, T: float, tau: float) -> np.ndarray:
    """Temperature softmax restricted to x >= tau and renormalised."""
    z = x / T
    e = np.where(x >= tau, np.exp(z - z.max()), 0.0)
    return e / e.sum()


def kept_by_definition(x: np.ndarray, T: float, top_k: int, top_p: float) -> np.ndarray:
    """The kept set written straight from the definitions (for pins, small V):
    fewer than k strictly larger logits, then mass strictly above < p."""
    V = len(x)
    keep = np.ones(V, bool)
    if 0 < top_k < V:
        keep = np.array([(x > x[i]).sum() < top_k for i in range(V)])
    if top_p < 1.0:
        z = x / T
        r = np.where(keep, np.exp(z - z.max()), 0.0)
        r = r / r.sum()
        top = x[keep].max()
        keep = keep & np.array([x[i] == top or r[x > x[i]].sum() < top_p for i in range(V)])
    return keep


def filter_row(x: np.ndarray, T: float, top_k: Optional[int], top_p: Optional[float]):
    """Convenience: (tau, alternatives) with None meaning 'off'."""
    return filter_threshold(x, T, 0 if top_k is None else int(top_k), 1.0 if top_p is None else float(top_p))
