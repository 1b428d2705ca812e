"""The oracle's handling of invalid inputs (status bits defined by the C
interface) and the comparator's near-tie rule."""
import numpy as np

import oracle
from oracle import verify as ov
from oracle.philox import verify_uniform, PURPOSE_ACCEPT


def _one(target, draft, tokens, T=1.0, mode=ov.SAMPLE, max_k=64, V=None):
    target = np.asarray(target, np.float32)
    return oracle.verify_batch(target=target, draft=None if draft is None else np.asarray(draft, np.float32),
                               dtype="f32", vocab=V or target.shape[1], num_draft=[len(tokens)],
                               draft_tokens=np.asarray(tokens, np.int32), temperature=[T], mode=[mode],
                               seq_ids=[0], seed=0, max_k=max_k)


def _cleared(res, K):
    return res.accepted_len[0] == -1 and (res.emitted == -1).all() and np.isnan(res.p_at).all() \
        and np.isnan(res.q_at).all() and len(res.emitted) == K + 1


def test_status_bits():
    t = np.zeros((3, 4))
    d = np.zeros((2, 4))
    assert _one(t, d, [0, 1]).status[0] == 0
    r = _one(t, d, [0, 1], max_k=1)
    assert r.status[0] == ov.ST_K_TOO_LARGE and _cleared(r, 2)
    assert _one(t, d, [0, 1], mode=7).status[0] == ov.ST_BAD_MODE
    assert _one(t, d, [0, 1], T=0.0).status[0] == ov.ST_BAD_TEMPERATURE
    assert _one(t, d, [0, 1], T=np.inf, mode=ov.ONEHOT).status[0] == ov.ST_BAD_TEMPERATURE
    assert _one(t, d, [0, 1], T=0.0, mode=ov.GREEDY).status[0] == 0          # greedy ignores T
    assert _one(t, d, [0, 1], T=np.float32(1e-6)).status[0] == 0
    assert _one(t, d, [0, 1], T=np.float32(9.9e-7)).status[0] == ov.ST_BAD_TEMPERATURE
    assert _one(t, None, [0, 1]).status[0] == ov.ST_NO_DRAFT_LOGITS
    assert _one(t, None, [0, 1], mode=ov.ONEHOT).status[0] == 0
    assert _one(t[:1], None, []).status[0] == 0                  # K = 0 reads no draft row
    assert _one(t, d, [0, 4]).status[0] == ov.ST_BAD_TOKEN
    assert _one(t, d, [-1, 0]).status[0] == ov.ST_BAD_TOKEN
    assert _one(t, None, [9, 0], T=-1.0).status[0] == ov.ST_BAD_TEMPERATURE | ov.ST_NO_DRAFT_LOGITS | ov.ST_BAD_TOKEN


def test_nonfinite_rows():
    t = np.zeros((3, 4))
    d = np.zeros((2, 4))
    tn = t.copy(); tn[1, 2] = np.nan
    assert _one(tn, d, [0, 1]).status[0] == ov.ST_NONFINITE
    tp = t.copy(); tp[2, 0] = np.inf            # bonus row is used
    assert _one(tp, d, [0, 1]).status[0] == ov.ST_NONFINITE
    ti = t.copy(); ti[0, :] = -np.inf
    r = _one(ti, d, [0, 1])
    assert r.status[0] == ov.ST_NONFINITE and _cleared(r, 2)
    tm = t.copy(); tm[0, :3] = -np.inf          # some -inf entries: fine, they have p = 0
    r = _one(tm, d, [3, 1])
    assert r.status[0] == 0 and r.p_at[0] == 1.0
    dn = d.copy(); dn[0, 0] = np.nan
    assert _one(t, dn, [0, 1]).status[0] == ov.ST_NONFINITE
    assert _one(t, dn, [0, 1], mode=ov.ONEHOT).status[0] == 0               # draft rows unused
    assert _one(tn, dn, [0, 1], mode=7).status[0] == ov.ST_BAD_MODE         # pre-checks win


def test_bad_layout_clears_everything():
    t = np.zeros((5, 4), np.float32)
    res = oracle.verify_batch(target=t, draft=None, dtype="f32", vocab=4, num_draft=[1, 2],
                              draft_tokens=np.zeros(2, np.int32), temperature=[1, 1], mode=[1, 1])
    assert not res.layout_ok
    assert (res.status == ov.ST_BAD_LAYOUT).all() and (res.accepted_len == -1).all()
    assert (res.emitted == -1).all() and len(res.emitted) == 4
    res = oracle.verify_batch(target=t, draft=None, dtype="f32", vocab=4, num_draft=[-1, 2],
                              draft_tokens=np.zeros(1, np.int32), temperature=[1, 1], mode=[1, 1])
    assert (res.status == ov.ST_BAD_LAYOUT).all()


def _near_tie_case(delta):
    """One SAMPLE sequence, K=2, whose ratio at position 0 is u0 + delta."""
    u0 = verify_uniform(0, 0, 0, PURPOSE_ACCEPT)
    r = u0 + delta
    qx = 0.9
    t = np.log([[r * qx, 1 - r * qx, 1e-9], [0.3, 0.3, 0.4], [0.2, 0.3, 0.5]])
    d = np.log([[qx, 0.05, 0.05], [0.3, 0.3, 0.4]])
    return _one(t, d, [0, 2])


def test_comparator_follows_near_tie_branch():
    res = _near_tie_case(4e-6)
    s = res.seqs[0]
    assert s.accept_flags == [0] and s.A >= 1
    alt = res.rerun(0, {0: False})
    assert alt.A == 0
    # a device that rejected at the near-tie and drew from the residual is accepted
    rep = oracle.compare(res, [alt.A], alt.emitted, alt.p_at, alt.q_at, [alt.status])
    assert rep.ok and rep.n_exempt == 1
    # the oracle's own outputs match exactly
    rep = oracle.compare(res, res.accepted_len, res.emitted, res.p_at, res.q_at, res.status)
    assert rep.ok and rep.n_exact == 1


def test_comparator_rejects_unflagged_difference():
    res = _near_tie_case(3e-3)
    s = res.seqs[0]
    assert not s.accept_flags and s.A >= 1
    alt = res.rerun(0, {0: False})
    rep = oracle.compare(res, [alt.A], alt.emitted, alt.p_at, alt.q_at, [alt.status])
    assert not rep.ok


def test_comparator_pq_tolerance():
    res = _near_tie_case(3e-3)
    rep = oracle.compare(res, res.accepted_len, res.emitted, res.p_at + 5e-6, res.q_at, res.status)
    assert rep.ok
    rep = oracle.compare(res, res.accepted_len, res.emitted, res.p_at + 2e-5, res.q_at, res.status)
    assert not rep.ok


def test_comparator_final_token_candidates():
    """A uniform right at a CDF boundary: both neighbouring tokens are allowed."""
    from workloads import make_random_batch
    found = False
    for seed in range(200):
        b = make_random_batch(seed, B=8, V=6, kmax=2, dtype="f32", modes=(ov.ONEHOT, ov.SAMPLE))
        res = oracle.verify_batch_from(b)
        for s, r in enumerate(res.seqs):
            if r.final is not None and r.final.candidates and len(r.final.candidates) > 1:
                found = True
                other = sorted(r.final.candidates - {r.final.y})[0]
                em = res.emitted.copy()
                ot = int(res._ctx["off_t"][s])
                em[ot + r.A] = other
                assert oracle.compare(res, res.accepted_len, em, res.p_at, res.q_at, res.status).ok
    # flags are rare by construction (band 1e-5); make sure the path is at least reachable
    if not found:
        w = np.array([0.5, 0.5])
        f, _ = ov._final_from_weights(w, 0.5 - 1e-6, False, None)
        assert f.cdf_flag and f.candidates == {0, 1}


def test_no_absolute_band_in_the_final_draw():
    """The only final-draw band is 1e-5 of the normalised CDF: on a residual of
    mass 1e-3, a uniform 2e-7 of mass (2e-4 of the CDF) from a boundary is
    no near-tie, so no other token is admitted."""
    w = np.array([5e-4, 5e-4])
    f, _ = ov._final_from_weights(w, (5e-4 - 2e-7) / 1e-3, False, None)
    assert f.y == 0 and not f.cdf_flag and f.candidates is None
    f, _ = ov._final_from_weights(w, (5e-4 - 4e-9) / 1e-3, False, None)     # 4e-6 of the CDF: flagged
    assert f.cdf_flag and f.candidates == {0, 1}


def test_strict_near_tie_followed_to_rejection():
    """STRICT, K = 1: u_0 lies 4e-6 inside the proposal's interval, so the
    oracle accepts and flags the decision; a device that rejected there must
    emit a neighbour of the proposal (the correction lands on the boundary
    where its interval was), and is counted as a near-tie match."""
    for seed in range(50):
        u0 = verify_uniform(seed, 0, 0, PURPOSE_ACCEPT)
        if 0.1 < u0 < 0.6:
            break
    p0 = np.array([u0 - 4e-6, 0.3, 0.0])
    p0[2] = 1.0 - p0[0] - p0[1]
    t = np.log(np.stack([p0, [0.2, 0.3, 0.5]]))
    res = oracle.verify_batch(target=t.astype(np.float32), draft=None, dtype="f32", vocab=3, num_draft=[1],
                              draft_tokens=np.array([1], np.int32), temperature=[1.0], mode=[ov.STRICT], seed=seed,
                              max_k=4)
    s = res.seqs[0]
    assert s.A == 1 and s.accept_flags == [0]
    alt = res.rerun(0, {0: False})
    assert alt.A == 0 and alt.final.cdf_flag and alt.final.candidates == {0, 2}
    for y in (0, 2):
        em = np.array([y, -1], np.int32)
        rep = oracle.compare(res, [0], em, res.p_at, res.q_at, [0])
        assert rep.ok and rep.n_exempt == 1, rep.messages
    rep = oracle.compare(res, [0], np.array([1, -1], np.int32), res.p_at, res.q_at, [0])
    assert not rep.ok                                   # the proposal itself is never the correction


def test_empty_residual_status_bit_only():
    """top-k 1 with the same kept token in p and q and a proposal outside it:
    rejected, the residual is exactly empty, so the oracle draws from p and
    sets bit 128.  A device whose rounding left a residual on the same token
    emits the same token without the bit: identical tokens, counted as exact
    and tallied apart; a different token is a mismatch."""
    t = np.array([[2.0, 0.0, 0.0], [0.0, 1.0, 0.5]], np.float32)
    d = np.array([[2.0, 0.1, 0.0]], np.float32)
    res = oracle.verify_batch(target=t, draft=d, dtype="f32", vocab=3, num_draft=[1],
                              draft_tokens=np.array([1], np.int32), temperature=[1.0], mode=[ov.SAMPLE],
                              top_k=np.array([1], np.int32), max_k=4)
    s = res.seqs[0]
    assert s.A == 0 and s.status == ov.ST_ZERO_RESIDUAL and s.final.z_flag and s.emitted[0] == 0
    rep = oracle.compare(res, [0], np.array([0, -1], np.int32), res.p_at, res.q_at, [0])
    assert rep.ok and rep.n_exact == 1 and rep.n_status_z == 1 and rep.n_degenerate == 0
    rep = oracle.compare(res, [0], np.array([0, -1], np.int32), res.p_at, res.q_at, [ov.ST_ZERO_RESIDUAL])
    assert rep.ok and rep.n_exact == 1 and rep.n_status_z == 0
