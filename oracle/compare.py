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
  a uniform within 1e-5 of a boundary of the inverse-CDF interval (then the
  emitted token must lie in the oracle's candidate set).
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
    n_cond_exempt: int = 0        # matched only thanks to the float32-conditioning band
    n_mismatch: int = 0
    n_oracle_flagged: int = 0     # sequences the oracle flagged at all
    max_pq_err: float = 0.0
    messages: List[str] = field(default_factory=list)

    @property
    def ok(self) -> bool:
        return self.n_mismatch == 0

    def summary(self) -> str:
        return (f"seqs={self.n_seq} exact={self.n_exact} exempt={self.n_exempt} "
                f"cond_exempt={self.n_cond_exempt} mismatch={self.n_mismatch} "
                f"oracle_flagged={self.n_oracle_flagged} max|dp,dq|={self.max_pq_err:.3g}")


def _fail(rep: CompareReport, msg: str):
    rep.n_mismatch += 1
    if len(rep.messages) < 20:
        rep.messages.append(msg)


def compare(res: BatchResult, accepted_len, emitted, p_at=None, q_at=None, status=None,
            pq_tol: float = 1e-5, strict_band: bool = False) -> CompareReport:
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
        if r.flagged:
            rep.n_oracle_flagged += 1

        if r.status & ST_ERROR_MASK:
            bad = (gA != -1) or (g_emit != -1).any() or (gst is not None and gst != r.status)
            for arr in (p_at, q_at):
                if arr is not None and K and not np.isnan(np.asarray(arr)[od:od + K]).all():
                    bad = True
            if bad:
                _fail(rep, f"seq {s}: error status {r.status}: got A={gA} status={gst} emit={g_emit.tolist()}")
            else:
                rep.n_exact += 1
            continue

        # p/q at proposal
        pq_bad = False
        for arr, ref in ((p_at, r.p_at), (q_at, r.q_at)):
            if arr is not None and K:
                d = np.abs(np.asarray(arr, np.float64)[od:od + K] - ref)
                if not np.isfinite(d).all():
                    pq_bad = True
                    rep.max_pq_err = float("inf")
                else:
                    rep.max_pq_err = max(rep.max_pq_err, float(d.max()))
                    pq_bad |= bool(d.max() > pq_tol)
        if pq_bad:
            _fail(rep, f"seq {s}: p/q at proposal differ by more than {pq_tol}")
            continue

        # follow near-tie branches of the acceptance scan
        cur = r
        exempt = False
        ok = True
        for _ in range(K + 1):
            if gA == cur.A:
                break
            i = min(gA, cur.A)
            if 0 <= i < K and i in cur.accept_flags:
                cur = res.rerun(s, {**cur.forced, i: gA > i})
                exempt = True
                continue
            ok = False
            _fail(rep, f"seq {s}: accepted_len gpu={gA} oracle={cur.A} (no near-tie at {i}; "
                       f"u={cur.u_acc[i] if i < len(cur.u_acc) else None} r={cur.ratios[i] if i < len(cur.ratios) else None})")
            break
        if not ok:
            continue
        A = cur.A
        if (g_emit[:A] != cur.emitted[:A]).any() or (g_emit[A + 1:] != -1).any():
            _fail(rep, f"seq {s}: emitted prefix/suffix differ: gpu={g_emit.tolist()} oracle={cur.emitted.tolist()}")
            continue
        gy = int(g_emit[A])
        f = cur.final
        cond_only = False
        if gy != f.y:
            allowed = f.candidates is not None and gy in f.candidates
            if allowed and strict_band and not (f.cdf_flag or f.z_flag):
                allowed = False
            if not allowed:
                _fail(rep, f"seq {s}: final token gpu={gy} oracle={f.y} ({f.kind}, u={f.u:.9f}, Z={f.Z:.6g}, "
                           f"flags cdf={f.cdf_flag} cond={f.cdf_cond_flag} z={f.z_flag})")
                continue
            exempt = True
            cond_only = f.cdf_cond_flag and not (f.cdf_flag or f.z_flag)
        if gst is not None:
            mask = ~ST_ZERO_RESIDUAL if f.z_flag else ~0
            if (gst & mask) != (cur.status & mask):
                _fail(rep, f"seq {s}: status gpu={gst} oracle={cur.status}")
                continue
        if cond_only:
            rep.n_cond_exempt += 1
        elif exempt:
            rep.n_exempt += 1
        else:
            rep.n_exact += 1
    return rep
