"""Plain float64 CPU oracle of the batched speculative-decoding verify step.

Test infrastructure.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module; the library never does.

Sources (page title, then section):

* [DM]   "Draft Model（草稿模型）" (compassingai.com): 15 分钟专家深入 §2
         接受-拒绝准则 (accept with probability min(1, p/q); on rejection
         draw from norm(max(0, p - q))); 技术原理, the one-step algorithm
         box (left-to-right scan, stop at the first rejection, one extra
         token from the target's next distribution when all K are accepted;
         1..K+1 tokens per round).
* [TUT]  gitcode.csdn.net speculative-decoding tutorial: §3.2 (reject
         probability max(0, 1 - p/q), corrected distribution
         max(0, p - q)/Z), §4.3 验证器实现 (both logit rows divided by the
         temperature before softmax; q(x) <= 0 rejects).
* [DIST] "Speculative Decoding在分布式推理中的应用" (wmrh.cn): §三 (stable
         softmax: subtract the max, exponentiate, sum, divide; accept when a
         uniform draw is below the ratio).
* [AIG]  "5.2 Draft 模型与无模型方案" (AIInfraGuide): §4.3 (a deterministic
         proposal is the one-hot distribution q(y) = 1 and is verified with
         the same accept/correct rule).
* [DIST] §二 and §三 also describe a strict check: the target samples its
         own token at the position and the draft token is accepted iff the
         two agree; on a mismatch the target's sample is emitted.

Readings where the pages leave a step open (each is a row of the design
notes):

* accept iff u < r with r = min(1, p/q), u uniform in [0, 1);
* q(x) = 0 gives r = 0 (reject);
* one-hot proposal: r = p(x); on rejection w = p with the proposed token
  removed (that is max(0, p - e_x));
* greedy mode: accept iff the proposed token is the lowest-index argmax of
  the raw target logits; emit that argmax on mismatch and as the bonus; the
  temperature plays no part (reported p uses T = 1);
* inverse CDF: C = inclusive cumulative sum of w, t = u * C[-1], the
  emitted token is the first k with C[k] > t, clamped to the last k with
  w[k] > 0; zero-mass tokens are never emitted;
* if a residual has no mass (only reachable by rounding) the token is drawn
  from p at that position with the same uniform and status bit 128 is set;
* uniforms: Philox4x32-10, key = seed, counter = (position, purpose, seq_id,
  0); purpose 0 for the acceptance test at positions 0..K-1, purpose 1 for
  the final draw at position A; u = (word0 >> 8) * 2^-24;
* strict mode: the target's own sample at position i is the inverse-CDF
  draw y_i = inverse_cdf(p_i, u_i) with the acceptance uniform u_i; x_i is
  accepted iff y_i = x_i; at the first mismatch y_A itself is emitted (so
  the correction uses u_A, purpose 0); all K accepted: the bonus from p_K
  with purpose 1.  No draft logits are used; reported q is 1.

Near-ties.  A decision is flagged when its uniform lies within 1e-5 of the
acceptance ratio, or within 1e-5 of a boundary of the emitted token's
interval of the normalised CDF; the comparison then also admits the other
branch or a neighbouring token.  Two further flags mark inputs that float32
cannot resolve at all and are counted apart: q(x) below 1e-30 (float32
underflow of the ratio's denominator) and a residual with less than 1e-6 of
mass (cancellation leaves no correct digit of max(0, p - q)).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from .filter import filter_threshold, filtered_softmax
from .philox import PURPOSE_ACCEPT, PURPOSE_SAMPLE, verify_uniform

# verify modes, as encoded in the library's per-sequence mode input
SAMPLE, GREEDY, ONEHOT, STRICT = 0, 1, 2, 3

# per-sequence status bits, as defined by the library's C interface
ST_BAD_LAYOUT = 1         # num_draft negative or not summing to total_draft
ST_K_TOO_LARGE = 2        # K_s > max_k
ST_BAD_MODE = 4           # mode not in {SAMPLE, GREEDY, ONEHOT, STRICT}
ST_BAD_TEMPERATURE = 8    # SAMPLE/ONEHOT/STRICT with T not finite or below MIN_TEMPERATURE
ST_NO_DRAFT_LOGITS = 16   # SAMPLE sequence with K > 0 but no draft logits given
ST_BAD_TOKEN = 32         # a proposed token outside [0, V)
ST_NONFINITE = 64         # NaN, +inf, or an all -inf row among the used rows
ST_ZERO_RESIDUAL = 128    # residual had no mass; drew from p instead (valid)
ST_ERROR_MASK = 127

# tolerance bands
BAND = 1e-5               # a uniform this close to a ratio or CDF boundary is a near-tie
Q_UNDERFLOW = 1e-30       # q(x) below this is in float32's underflow zone
Z_DEGENERATE = 1e-6       # a residual with less mass than this is numerically empty in float32
MIN_TEMPERATURE = float(np.float32(1e-6))   # smallest valid SAMPLE/ONEHOT temperature (float32 value)


def widen(rows: np.ndarray, dtype: str) -> np.ndarray:
    """Stored logits -> exact float64 (bfloat16 bits are the top half of a float32)."""
    if dtype == "bf16":
        return (np.asarray(rows, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(rows, np.float32).astype(np.float64)


def softmax(x: np.ndarray, T: float) -> np.ndarray:
    """Temperature softmax of one logit row ([TUT] §4.3 divides by T first;
    [DIST] §三 subtracts the max, exponentiates, sums and divides)."""
    z = x / T
    e = np.exp(z - z.max())
    return e / e.sum()


def row_ok(x: np.ndarray) -> bool:
    """A usable logit row: no NaN, no +inf, and at least one finite entry
    (-inf entries are allowed: they have probability 0)."""
    return (not np.isnan(x).any()) and (not np.isposinf(x).any()) and bool(np.isfinite(x).any())


def accept_ratio(mode: int, p_x: float, q_x: float) -> float:
    """r for the acceptance test u < r ([DM] §2, [TUT] §3.2 and §4.3, [AIG] §4.3)."""
    if mode == ONEHOT:
        return float(p_x)
    if q_x <= 0.0:
        return 0.0
    return min(1.0, float(p_x) / float(q_x))


def residual(mode: int, p: np.ndarray, q: Optional[np.ndarray], x: int) -> np.ndarray:
    """Unnormalised correction distribution after a rejection ([DM] §2,
    [TUT] §3.2: max(0, p - q); one-hot q: p with the proposed token removed)."""
    if mode == ONEHOT:
        w = p.copy()
        w[x] = 0.0
        return w
    return np.maximum(p - q, 0.0)


def inverse_cdf(w: np.ndarray, u) -> np.ndarray:
    """First k with inclusive C[k] > u * C[-1]; clamped to the last k with w > 0.
    ``u`` may be an array (vectorised over uniforms)."""
    C = np.cumsum(w)
    t = np.asarray(u, dtype=np.float64) * C[-1]
    k = np.searchsorted(C, t, side="right")
    last = int(np.nonzero(w > 0)[0][-1])
    return np.minimum(k, last)


def cdf_interval(p: np.ndarray, x: int):
    """[lo, hi): the part of [0, sum p) that the inverse CDF maps to token x."""
    C = np.cumsum(p)
    return (float(C[x - 1]) if x > 0 else 0.0), float(C[x])


def strict_correction(p: np.ndarray, x: int, u: float):
    """Strict mode, only where a near-tie is followed down its rejecting
    branch although u lies inside x's own interval: the correction is then
    drawn from p with x removed (weights w) at the boundary where x's
    interval was, so that the tokens on both sides of x are candidates.
    Returns (w, u') with u' = t' / sum(w)."""
    w = p.copy()
    w[x] = 0.0
    lo, hi = cdf_interval(p, x)
    t = u * float(np.cumsum(p)[-1])
    if t < lo:
        tr = t
    elif t >= hi:
        tr = t - float(p[x])
    else:
        tr = lo
    Zr = float(np.cumsum(w)[-1])
    return w, (tr / Zr if Zr > 0 else u)


@dataclass
class FinalDraw:
    kind: str                       # "greedy", "residual", "bonus", "fallback"
    y: int
    u: float = float("nan")
    Z: float = float("nan")
    cdf_flag: bool = False          # u within BAND of a boundary of y's interval (normalised CDF)
    z_flag: bool = False            # residual numerically empty (degenerate, counted apart)
    candidates: Optional[set] = None        # tokens within the 1e-5 band (cdf_flag)
    z_candidates: Optional[set] = None      # every token with mass, when the residual is degenerate


@dataclass
class SeqResult:
    status: int
    A: int                                   # accepted draft tokens (-1 on error)
    emitted: np.ndarray                      # int32 [K+1]
    p_at: np.ndarray                         # float64 [K]
    q_at: np.ndarray                         # float64 [K]
    accept_flags: List[int] = field(default_factory=list)   # positions whose |u - r| < BAND
    underflow_flags: List[int] = field(default_factory=list)   # SAMPLE positions with q(x) < Q_UNDERFLOW
    u_acc: List[float] = field(default_factory=list)
    ratios: List[float] = field(default_factory=list)
    final: Optional[FinalDraw] = None
    forced: Dict[int, bool] = field(default_factory=dict)
    # top-p near-ties: (row key ("t", i) or ("d", i), an equally valid threshold)
    filter_alts: List[tuple] = field(default_factory=list)
    forced_tau: Dict[tuple, float] = field(default_factory=dict)

    @property
    def flagged(self) -> bool:
        f = self.final
        return bool(self.accept_flags or self.underflow_flags) or (f is not None and (f.cdf_flag or f.z_flag))


def _error_result(K: int, status: int) -> SeqResult:
    return SeqResult(status=status, A=-1, emitted=np.full(K + 1, -1, np.int32),
                     p_at=np.full(K, np.nan), q_at=np.full(K, np.nan))


def _final_from_weights(w: np.ndarray, u: float, z_check: bool, fallback_p: Optional[np.ndarray]):
    """Draw the final token from unnormalised weights w with uniform u, and
    work out the near-boundary flags and the candidate set."""
    w0 = w
    Z = float(np.cumsum(w)[-1])
    z_flag = bool(z_check and Z < Z_DEGENERATE)
    kind = "residual"
    status = 0
    if Z <= 0.0:
        w = fallback_p
        Z = float(np.cumsum(w)[-1])
        kind = "fallback"
        status = ST_ZERO_RESIDUAL
    y = int(inverse_cdf(w, u))
    C = np.cumsum(w)
    lo = C[y - 1] if y > 0 else 0.0
    hi = C[y]
    t = u * Z
    band = BAND * Z          # 1e-5 of the normalised CDF
    cdf_flag = (t - lo < band) or (hi - t < band)
    cands = None
    if cdf_flag:
        Cm = np.concatenate(([0.0], C[:-1]))
        ok = (w > 0) & (Cm <= t + band) & (C >= t - band)
        cands = set(int(k) for k in np.nonzero(ok)[0])
        cands.add(y)
    zc = None
    if z_flag:
        zc = set(int(k) for k in np.nonzero(w0 > 0)[0])
        if fallback_p is not None:
            zc |= set(int(k) for k in np.nonzero(fallback_p > 0)[0])
    return FinalDraw(kind=kind, y=y, u=u, Z=Z, cdf_flag=bool(cdf_flag), z_flag=z_flag, candidates=cands,
                     z_candidates=zc), status


def strict_emit(p: np.ndarray, x: int, u: float):
    """Strict mode, at the first position A whose proposal x was not the
    target's own sample: the emitted token is that sample itself,
    y_A = inverse_cdf(p_A, u_A) ([DIST] §二, §三).  Returns (FinalDraw, status)."""
    y = int(inverse_cdf(p, u))
    if y != x:
        f, st = _final_from_weights(p, u, False, None)
        if f.candidates is not None:
            f.candidates.discard(x)          # this branch rejected x
    else:
        # only when a near-tie at A is followed down its rejecting branch: u lies in x's own
        # interval, so the correction sits on the boundary where that interval was
        w, ur = strict_correction(p, x, u)
        f, st = _final_from_weights(w, ur, True, p)
    f.kind = "strict"
    return f, st


def verify_sequence(xt: np.ndarray, xd: Optional[np.ndarray], tokens: np.ndarray, T: float, mode: int,
                    seq_id: int, seed: int, vocab: int, max_k: int, draft_present: bool,
                    force: Optional[Dict[int, bool]] = None, top_k: int = 0, top_p: float = 1.0,
                    force_tau: Optional[Dict[tuple, float]] = None) -> SeqResult:
    """Verify one sequence.

    xt: [K+1, V] float64 target logits (row i judges draft slot i, row K is
        the bonus distribution); xd: [K, V] float64 draft logits or None;
    tokens: the K proposed token ids.  ``force`` maps a position to an
    accept decision that overrides the uniform test there (used only to
    follow the other branch of a near-tie).  ``top_k`` / ``top_p`` filter
    every used row (oracle/filter.py); ``force_tau`` replaces a row's
    threshold by a recorded alternative (the other side of a top-p
    near-tie)."""
    K = int(tokens.shape[0])
    force = force or {}
    status = 0
    if K > max_k:
        status |= ST_K_TOO_LARGE
    if mode not in (SAMPLE, GREEDY, ONEHOT, STRICT):
        status |= ST_BAD_MODE
    if mode in (SAMPLE, ONEHOT, STRICT) and not (np.isfinite(T) and T >= MIN_TEMPERATURE):
        status |= ST_BAD_TEMPERATURE
    if mode == SAMPLE and K > 0 and not draft_present:
        status |= ST_NO_DRAFT_LOGITS
    if K and ((tokens < 0).any() or (tokens >= vocab).any()):
        status |= ST_BAD_TOKEN
    if status:
        return _error_result(K, status)

    used = [xt[i] for i in range(K + 1)] + ([xd[i] for i in range(K)] if mode == SAMPLE else [])
    if not all(row_ok(r) for r in used):
        return _error_result(K, ST_NONFINITE)

    T_eff = float(T) if mode != GREEDY else 1.0
    force_tau = force_tau or {}
    alts: List[tuple] = []
    filtering = mode != GREEDY and ((0 < int(top_k) < vocab) or (top_p < 1.0))

    def row_dist(x, key):
        if not filtering:
            return softmax(x, T_eff)
        tau, al = filter_threshold(x, T_eff, int(top_k), float(top_p))
        alts.extend((key, a) for a in al)
        return filtered_softmax(x, T_eff, force_tau.get(key, tau))

    p = [row_dist(xt[i], ("t", i)) for i in range(K + 1)]
    q = [row_dist(xd[i], ("d", i)) for i in range(K)] if mode == SAMPLE else None
    tok = [int(t) for t in tokens]
    p_at = np.array([p[i][tok[i]] for i in range(K)], dtype=np.float64)
    q_at = np.array([q[i][tok[i]] for i in range(K)] if mode == SAMPLE else [1.0] * K, dtype=np.float64)

    res = SeqResult(status=0, A=K, emitted=np.full(K + 1, -1, np.int32), p_at=p_at, q_at=q_at,
                    forced=dict(force), filter_alts=alts, forced_tau=dict(force_tau))

    # left-to-right scan, stopping at the first rejection ([DM] algorithm box)
    A = K
    for i in range(K):
        if mode == GREEDY:
            acc = tok[i] == int(np.argmax(xt[i]))
        elif mode == STRICT:
            # the target's own sample at position i, with the acceptance uniform
            u = verify_uniform(seed, seq_id, i, PURPOSE_ACCEPT)
            y = int(inverse_cdf(p[i], u))
            acc = y == tok[i]
            res.u_acc.append(u)
            res.ratios.append(float(p_at[i]))
            lo, hi = cdf_interval(p[i], tok[i])
            t = u * float(np.cumsum(p[i])[-1])
            if p_at[i] > 0 and (abs(t - lo) < BAND or abs(t - hi) < BAND):
                res.accept_flags.append(i)
        else:
            u = verify_uniform(seed, seq_id, i, PURPOSE_ACCEPT)
            r = accept_ratio(mode, p_at[i], q_at[i])
            res.u_acc.append(u)
            res.ratios.append(r)
            acc = u < r
            if abs(u - r) < BAND:
                res.accept_flags.append(i)
            elif mode == SAMPLE and q_at[i] < Q_UNDERFLOW:
                res.underflow_flags.append(i)
        if i in force:
            acc = bool(force[i])
        if not acc:
            A = i
            break
    res.A = A
    res.emitted[:A] = tok[:A]

    # the final token at position A
    if mode == GREEDY:
        y = int(np.argmax(xt[A]))
        res.final = FinalDraw(kind="greedy", y=y)
    elif mode == STRICT and A < K:
        res.final, st = strict_emit(p[A], tok[A], verify_uniform(seed, seq_id, A, PURPOSE_ACCEPT))
        res.status |= st
    else:
        u = verify_uniform(seed, seq_id, A, PURPOSE_SAMPLE)
        if A < K:
            w = residual(mode, p[A], q[A] if q is not None else None, tok[A])
            res.final, st = _final_from_weights(w, u, True, p[A])
            res.status |= st
        else:
            res.final, _ = _final_from_weights(p[K], u, False, None)
            res.final.kind = "bonus"
    res.emitted[A] = res.final.y
    return res


@dataclass
class BatchResult:
    accepted_len: np.ndarray     # int32 [B]
    emitted: np.ndarray          # int32 [total_draft + B]
    p_at: np.ndarray             # float64 [total_draft]
    q_at: np.ndarray             # float64 [total_draft]
    status: np.ndarray           # int32 [B]
    seqs: List[Optional[SeqResult]]
    layout_ok: bool
    _ctx: dict = field(default_factory=dict, repr=False)

    def rerun(self, s: int, force: Dict[int, bool], force_tau: Optional[Dict[tuple, float]] = None) -> SeqResult:
        """Re-verify sequence s with some accept decisions (and filter
        thresholds) forced."""
        return _verify_one(self._ctx, s, force, force_tau)


def _verify_one(ctx: dict, s: int, force=None, force_tau=None) -> SeqResult:
    K = int(ctx["num_draft"][s])
    ot, od = int(ctx["off_t"][s]), int(ctx["off_d"][s])
    V, dtype = ctx["vocab"], ctx["dtype"]
    xt = widen(ctx["target"][ot:ot + K + 1, :V], dtype)
    draft = ctx["draft"]
    mode = int(ctx["mode"][s])
    xd = widen(draft[od:od + K, :V], dtype) if (draft is not None and mode == SAMPLE) else None
    tk = ctx["top_k"]
    tp = ctx["top_p"]
    return verify_sequence(xt, xd, ctx["draft_tokens"][od:od + K], float(ctx["temperature"][s]), mode,
                           int(ctx["seq_ids"][s]), ctx["seed"], V, ctx["max_k"], draft is not None, force,
                           top_k=0 if tk is None else int(tk[s]), top_p=1.0 if tp is None else float(tp[s]),
                           force_tau=force_tau)


def verify_batch(*, target, draft, dtype: str, vocab: int, num_draft, draft_tokens, temperature,
                 mode=None, seq_ids=None, seed: int = 0, max_k: int = 64,
                 total_draft: Optional[int] = None, top_k=None, top_p=None) -> BatchResult:
    """Verify a packed ragged batch (layout as in the library's C interface:
    sequence s owns target rows off_t[s] .. off_t[s]+K_s with
    off_t[s] = sum_{j<s}(K_j+1), and draft rows / tokens off_d[s] ..
    off_d[s]+K_s-1 with off_d[s] = sum_{j<s} K_j).  top_k (int [B]) and
    top_p (float32 [B]) filter every used row of a sequence; None: off."""
    num_draft = np.asarray(num_draft, dtype=np.int64)
    B = int(num_draft.shape[0])
    draft_tokens = np.asarray(draft_tokens, dtype=np.int64)
    if total_draft is None:
        total_draft = int(draft_tokens.shape[0])
    mode = np.zeros(B, np.int64) if mode is None else np.asarray(mode, dtype=np.int64)
    seq_ids = np.arange(B, dtype=np.int64) if seq_ids is None else np.asarray(seq_ids, dtype=np.int64)
    temperature = np.asarray(temperature, dtype=np.float32).astype(np.float64)

    acc = np.full(B, -1, np.int32)
    emitted = np.full(total_draft + B, -1, np.int32)
    p_at = np.full(total_draft, np.nan)
    q_at = np.full(total_draft, np.nan)
    status = np.zeros(B, np.int32)

    layout_ok = bool((num_draft >= 0).all()) and int(num_draft.sum()) == total_draft
    if not layout_ok:
        status[:] = ST_BAD_LAYOUT
        return BatchResult(acc, emitted, p_at, q_at, status, [None] * B, False)

    off_d = np.concatenate(([0], np.cumsum(num_draft)[:-1])).astype(np.int64)
    off_t = off_d + np.arange(B, dtype=np.int64)
    ctx = dict(target=target, draft=draft, dtype=dtype, vocab=int(vocab), num_draft=num_draft,
               draft_tokens=draft_tokens, temperature=temperature, mode=mode, seq_ids=seq_ids,
               seed=int(seed), max_k=int(max_k), off_t=off_t, off_d=off_d,
               top_k=None if top_k is None else np.asarray(top_k, np.int64),
               top_p=None if top_p is None else np.asarray(top_p, np.float32).astype(np.float64))
    seqs: List[Optional[SeqResult]] = []
    for s in range(B):
        r = _verify_one(ctx, s)
        seqs.append(r)
        K = int(num_draft[s])
        acc[s] = r.A
        status[s] = r.status
        emitted[off_t[s]:off_t[s] + K + 1] = r.emitted
        p_at[off_d[s]:off_d[s] + K] = r.p_at
        q_at[off_d[s]:off_d[s] + K] = r.q_at
    return BatchResult(acc, emitted, p_at, q_at, status, seqs, True, ctx)


def verify_batch_from(batch, max_k: int = 64) -> BatchResult:
    """Convenience: run ``verify_batch`` on an object with the input fields
    (target, draft, dtype, vocab, num_draft, draft_tokens, temperature, mode,
    seq_ids, seed)."""
    return verify_batch(target=batch.target, draft=batch.draft, dtype=batch.dtype, vocab=batch.vocab,
                        num_draft=batch.num_draft, draft_tokens=batch.draft_tokens,
                        temperature=batch.temperature, mode=batch.mode, seq_ids=batch.seq_ids,
                        seed=batch.seed, max_k=max_k, top_k=getattr(batch, "top_k", None),
                        top_p=getattr(batch, "top_p", None))
