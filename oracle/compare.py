"""Compare a verify-step result against the oracle, honouring near-ties.

Test infrastructure.  The rule:

* status words equal (bit 128, "residual had no mass", may differ only
  where the oracle marks the residual as numerically empty);
* sequences with an error status: accepted_len = -1, every emitted slot -1,
  p/q at proposal NaN;
* p/q at proposal within ``pq_tol`` absolute;
* accepted_len and emitted tokens identical, except where the oracle flags a
  near-tie: a uniform within 1e-5 of an acceptance ratio (then the other
  branch of that decision is followed in the oracle and compared again), or
  a uniform within 1e-5 of a boundary of the emitted token's interval of the
  normalised CDF (then the emitted token must lie in the oracle's candidate
  set), or a top-p crossing within 1e-5 of a tie group's mass (then the
  sequence may match the oracle run with the neighbouring filter threshold
  instead).  Such matches are counted in ``n_exempt``.
* inputs float32 cannot resolve (q(x) < 1e-30 at a SAMPLE position, a
  residual with less than 1e-6 of mass) are followed the same way but counted
  in ``n_degenerate``, so that a caller can require none; where the tokens
  are identical and only the informational status bit 128 differs on such a
  residual, the sequence counts as exact and is tallied in ``n_status_z``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .verify import BatchResult, ST_BAD_LAYOUT, ST_ERROR_MASK, ST_ZERO_RESIDUAL


@dataclass
class CompareReport:
    n_seq: int = 0
    n_exact: int = 0
    n_exempt: int = 0             # matched only thanks to a 1e-5 near-tie flag
    n_degenerate: int = 0         # matched only thanks to a degenerate-input flag (q underflow, empty residual)
    n_mismatch: int = 0
    n_status_z: int = 0           # tokens identical, only the informational bit 128 differs (empty residual)
    n_oracle_flagged: int = 0     # sequences the oracle flagged at all
    max_pq_err: float = 0.0
    messages: List[str] = field(default_factory=list)

    @property
    def ok(self) -> bool:
        return self.n_mismatch == 0

    def summary(self) -> str:
        return (f"seqs={self.n_seq} exact={self.n_exact} exempt={self.n_exempt} "
                f"degenerate={self.n_degenerate} mismatch={self.n_mismatch} status128_only={self.n_status_z} "
                f"oracle_flagged={self.n_oracle_flagged} max|dp,dq|={self.max_pq_err:.3g}")


def _fail(rep: CompareReport, msg: str):
    rep.n_mismatch += 1
    if len(rep.messages) < 20:
        rep.messages.append(msg)


def compare(res: BatchResult, accepted_len, emitted, p_at=None, q_at=None, status=None,
            pq_tol: float = 1e-5) -> CompareReport:
    accepted_len = np.asarray(accepted_len)
    emitted = np.asarray(emitted)
    B = accepted_len.shape[0]
    rep = CompareReport(n_seq=B)
    if not res.layout_ok:
        if status is not None and not (np.asarray(status) == ST_BAD_LAYOUT).all():
            _fail(rep, "bad layout: status words differ")
        if not (accepted_len == -1).all() or not (emitted == -1).all():
            _fail(rep, "bad layout: outputs not cleared")
        for arr, nm in ((p_at, "p_at"), (q_at, "q_at")):
            if arr is not None and not np.isnan(np.asarray(arr)).all():
                _fail(rep, f"bad layout: {nm} not NaN")
        return rep

    ctx = res._ctx
    for s in range(B):
        K = int(ctx["num_draft"][s])
        ot, od = int(ctx["off_t"][s]), int(ctx["off_d"][s])
        r = res.seqs[s]
        g_emit = emitted[ot:ot + K + 1]
        gA = int(accepted_len[s])
        gst = int(status[s]) if status is not None else None
        if r.flagged or r.filter_alts:
            rep.n_oracle_flagged += 1
        g_p = None if p_at is None else np.asarray(p_at, np.float64)[od:od + K]
        g_q = None if q_at is None else np.asarray(q_at, np.float64)[od:od + K]
        verdict, msg, pq_err, znote = _compare_seq(res, s, r, K, gA, g_emit, gst, g_p, g_q, pq_tol)
        if verdict is None and r.filter_alts:
            # a top-p near-tie: the filter threshold on one side of it is as valid as on the other
            for key, alt in r.filter_alts:
                r2 = res.rerun(s, {}, {key: alt})
                v2, _, e2, z2 = _compare_seq(res, s, r2, K, gA, g_emit, gst, g_p, g_q, pq_tol)
                if v2 is not None:
                    verdict, pq_err, znote = ("degenerate" if v2 == "degenerate" else "exempt"), e2, z2
                    break
        rep.max_pq_err = max(rep.max_pq_err, pq_err)
        rep.n_status_z += int(bool(znote) and verdict is not None)
        if verdict is None:
            _fail(rep, msg)
        elif verdict == "exact":
            rep.n_exact += 1
        elif verdict == "degenerate":
            rep.n_degenerate += 1
        else:
            rep.n_exempt += 1
    return rep


def _compare_seq(res: BatchResult, s: int, r, K: int, gA: int, g_emit, gst, g_p, g_q, pq_tol: float):
    """One sequence against one oracle result: (verdict, message, max |dp,dq|,
    status note) with verdict "exact", "exempt" (matched through a 1e-5
    near-tie), "degenerate" (through a degenerate-input flag) or None; the
    note is True when only status bit 128 differs on a numerically empty
    residual (the tokens themselves are compared as usual)."""
    if r.status & ST_ERROR_MASK:
        bad = (gA != -1) or (g_emit != -1).any() or (gst is not None and gst != r.status)
        for arr in (g_p, g_q):
            if arr is not None and K and not np.isnan(arr).all():
                bad = True
        if bad:
            return None, f"seq {s}: error status {r.status}: got A={gA} status={gst} emit={g_emit.tolist()}", 0.0, False
        return "exact", "", 0.0, False
    pq_err = 0.0
    for arr, ref in ((g_p, r.p_at), (g_q, r.q_at)):
        if arr is not None and K:
            d = np.abs(arr - ref)
            if not np.isfinite(d).all():
                return None, f"seq {s}: p/q at proposal not finite", float("inf"), False
            pq_err = max(pq_err, float(d.max()))
    if pq_err > pq_tol:
        return None, f"seq {s}: p/q at proposal differ by {pq_err:.3g} > {pq_tol}", pq_err, False
    # follow flagged branches of the acceptance scan
    cur = r
    exempt = degenerate = False
    for _ in range(K + 1):
        if gA == cur.A:
            break
        i = min(gA, cur.A)
        if 0 <= i < K and (i in cur.accept_flags or i in cur.underflow_flags):
            if i in cur.accept_flags:
                exempt = True
            else:
                degenerate = True
            cur = res.rerun(s, {**cur.forced, i: gA > i}, cur.forced_tau)
            continue
        return None, (f"seq {s}: accepted_len gpu={gA} oracle={cur.A} (no near-tie at {i}; "
                      f"u={cur.u_acc[i] if i < len(cur.u_acc) else None} "
                      f"r={cur.ratios[i] if i < len(cur.ratios) else None})"), pq_err, False
    if gA != cur.A:
        return None, f"seq {s}: accepted_len gpu={gA} oracle={cur.A}", pq_err, False
    A = cur.A
    if (g_emit[:A] != cur.emitted[:A]).any() or (g_emit[A + 1:] != -1).any():
        return None, f"seq {s}: emitted prefix/suffix differ: gpu={g_emit.tolist()} oracle={cur.emitted.tolist()}", pq_err, False
    gy = int(g_emit[A])
    f = cur.final
    if gy != f.y:
        if f.candidates is not None and gy in f.candidates:
            exempt = True
        elif f.z_candidates is not None and gy in f.z_candidates:
            degenerate = True
        else:
            return None, (f"seq {s}: final token gpu={gy} oracle={f.y} ({f.kind}, u={f.u:.9f}, Z={f.Z:.6g}, "
                          f"flags cdf={f.cdf_flag} z={f.z_flag})"), pq_err, False
    znote = False
    if gst is not None:
        mask = ~ST_ZERO_RESIDUAL if f.z_flag else ~0
        if (gst & mask) != (cur.status & mask):
            return None, f"seq {s}: status gpu={gst} oracle={cur.status}", pq_err, False
        znote = gst != cur.status
    if degenerate:
        return "degenerate", "", pq_err, znote
    return ("exempt" if exempt else "exact"), "", pq_err, znote
