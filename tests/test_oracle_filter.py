"""CPU pins of the top-k / top-p filter oracle: the threshold form against
the kept set written straight from the definitions (ties included), the
reduction to the unfiltered path, losslessness with respect to the filtered
target distribution, the reported p/q at the proposal, and planted
mistakes that each pin must catch."""
import numpy as np
import pytest
from scipy import special, stats

import oracle
from oracle import filter as of
from oracle import verify as ov
from workloads import make_random_batch

P_MIN = 1e-4


def _rows_with_ties(rng, V):
    """Logits on a coarse grid, so equal values are common."""
    return np.round(rng.standard_normal(V) * 1.5 * 4) / 4


def _check_threshold_vs_definition(threshold_fn, trials=600, seed=0):
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        V = int(rng.integers(1, 40))
        x = _rows_with_ties(rng, V)
        T = float(rng.uniform(0.3, 1.5))
        k = int(rng.integers(-1, V + 2))
        p = float(rng.choice([1.0, 0.0, 0.3, 0.5, 0.8, 0.9, 0.95, 0.99, 1.5, rng.uniform(0, 1)]))
        tau, alts = threshold_fn(x, T, k, p)
        want = of.kept_by_definition(x, T, k, p)
        got_sets = [x >= t for t in [tau] + list(alts)]
        assert any(np.array_equal(g, want) for g in got_sets), (x, T, k, p, tau, alts)
        assert (x >= tau).any()                            # something is always kept
        assert (x >= tau)[np.argmax(x)]                    # the argmax always is


def test_threshold_matches_definition():
    _check_threshold_vs_definition(of.filter_threshold)


def test_topk_keeps_ties_and_counts():
    x = np.array([3.0, 1.0, 3.0, 2.0, 2.0, 0.0])
    assert of.topk_threshold(x, 1) == 3.0 and (x >= 3.0).sum() == 2      # both tied maxima
    assert of.topk_threshold(x, 3) == 2.0 and (x >= 2.0).sum() == 4      # the tie at the 3rd value
    assert of.topk_threshold(x, 6) == -np.inf and of.topk_threshold(x, 0) == -np.inf


def _check_topp_examples(threshold_fn):
    """Probabilities 0.5, 0.3, 0.2 (T = 1): p = 0.5 keeps one token (the mass
    above the second, 0.5, is not below 0.5), p = 0.6 keeps two, p = 0.85
    keeps all three."""
    x = np.log(np.array([0.5, 0.3, 0.2]))
    for p, n in ((0.5, 1), (0.6, 2), (0.85, 3), (0.79, 2), (0.81, 3), (1e-9, 1)):
        tau, _ = threshold_fn(x, 1.0, 0, p)
        assert (x >= tau).sum() == n, (p, tau)


def test_topp_examples():
    _check_topp_examples(of.filter_threshold)


def test_filters_off_reduce_to_plain_path():
    for seed in (1, 2):
        b = make_random_batch(seed, B=24, V=60, kmax=5, dtype="f32", modes=(0, 1, 2, 3))
        plain = oracle.verify_batch_from(b)
        b.top_k = np.where(np.arange(b.batch) % 2 == 0, 0, b.vocab).astype(np.int32)
        b.top_p = np.where(np.arange(b.batch) % 3 == 0, 1.0, 2.0).astype(np.float32)
        filt = oracle.verify_batch_from(b)
        assert np.array_equal(plain.accepted_len, filt.accepted_len)
        assert np.array_equal(plain.emitted, filt.emitted)
        assert np.allclose(plain.p_at, filt.p_at, equal_nan=True)


def _run(t, d, toks, T, mode, k, p, n, seed=0):
    t = np.asarray(t, np.float32)
    K = t.shape[0] - 1
    return oracle.verify_batch(target=np.tile(t, (n, 1)), draft=None if d is None else np.tile(d, (n, 1)),
                               dtype="f32", vocab=t.shape[1], num_draft=np.full(n, K, np.int32),
                               draft_tokens=np.asarray(toks, np.int32).reshape(-1),
                               temperature=np.full(n, T, np.float32), mode=np.full(n, mode, np.uint8),
                               seq_ids=np.arange(n, dtype=np.uint32), seed=seed,
                               top_k=np.full(n, k, np.int32), top_p=np.full(n, p, np.float32))


def _filtered(x, T, k, p):
    keep = of.kept_by_definition(x.astype(np.float64), T, k, p)
    r = special.softmax(x.astype(np.float64) / T)
    r = np.where(keep, r, 0.0)
    return r / r.sum()


def _chi2(obs, probs, what):
    exp = probs * obs.sum()
    keep = exp > 0
    assert obs[~keep].sum() == 0, f"{what}: mass outside the kept set"
    if keep.sum() == 1:                  # a single kept token: all draws on it (checked just above)
        return
    pv = stats.chisquare(obs[keep], exp[keep]).pvalue
    assert pv > P_MIN, f"{what}: p-value {pv:.3g}"


def _check_lossless(mode, k, p, n=8000, K=2, V=12, T=0.8, seed=3):
    """Proposals drawn from the filtered draft distribution (SAMPLE) or
    uniformly (one-hot / strict): every emitted position follows the filtered
    target distribution."""
    rng = np.random.default_rng(seed)
    t = (1.3 * rng.standard_normal((K + 1, V))).astype(np.float32)
    d = (t[:K] + rng.standard_normal((K, V))).astype(np.float32)
    pt = [_filtered(t[i], T, k, p) for i in range(K + 1)]
    if mode == ov.SAMPLE:
        qd = [_filtered(d[i], T, k, p) for i in range(K)]
        toks = np.stack([rng.choice(V, size=n, p=qd[i]) for i in range(K)], axis=1)
    else:
        toks = rng.integers(0, V, size=(n, K))
    res = _run(t, d if mode == ov.SAMPLE else None, toks, T, mode, k, p, n)
    em = res.emitted.reshape(n, K + 1)
    for j in range(K + 1):
        reached = res.accepted_len >= j
        _chi2(np.bincount(em[reached, j], minlength=V).astype(float), pt[j], f"mode {mode} k={k} p={p} pos {j}")
    return res, t, d, toks


@pytest.mark.parametrize("mode", [ov.SAMPLE, ov.ONEHOT, ov.STRICT])
@pytest.mark.parametrize("k,p", [(4, 1.0), (0, 0.9), (6, 0.8)])
def test_lossless_filtered(mode, k, p):
    _check_lossless(mode, k, p)


def _check_pq_reported(k=5, p=0.75):
    rng = np.random.default_rng(8)
    K, V, T, n = 3, 15, 0.9, 40
    t = (1.2 * rng.standard_normal((K + 1, V))).astype(np.float32)
    d = (t[:K] + rng.standard_normal((K, V))).astype(np.float32)
    toks = rng.integers(0, V, size=(n, K))
    res = _run(t, d, toks, T, ov.SAMPLE, k, p, n)
    pt = [_filtered(t[i], T, k, p) for i in range(K)]
    qd = [_filtered(d[i], T, k, p) for i in range(K)]
    want_p = np.array([[pt[i][toks[s, i]] for i in range(K)] for s in range(n)]).reshape(-1)
    want_q = np.array([[qd[i][toks[s, i]] for i in range(K)] for s in range(n)]).reshape(-1)
    assert np.allclose(res.p_at, want_p, atol=1e-12) and np.allclose(res.q_at, want_q, atol=1e-12)


def test_reported_pq_are_filtered():
    _check_pq_reported()


# ---- planted mistakes ----------------------------------------------------------

def test_plant_topk_distinct_values(monkeypatch):
    """The k-th largest DISTINCT value as the top-k threshold (equal values
    counted once): keeps too many tokens when there are ties."""
    real = of.topk_threshold

    def bad(x, k):
        u = np.unique(x)[::-1]
        return float(u[k - 1]) if 0 < k < len(x) and k <= len(u) else real(x, k)
    monkeypatch.setattr(of, "topk_threshold", bad)
    with pytest.raises(AssertionError):
        _check_threshold_vs_definition(of.filter_threshold, trials=300)


def test_plant_topp_inclusive(monkeypatch):
    """Mass above <= p instead of < p (keeps one more group at exact hits)."""
    def bad(x, T, k, p):
        tau, alts = of.filter_threshold(x, T, k, p)
        if p < 1:
            tau_k = of.topk_threshold(x, k)
            kept = x[x >= tau_k]
            r = special.softmax(kept / T)
            vals = np.unique(kept)[::-1]
            for v in vals:
                if r[kept > v].sum() <= p + 1e-12:
                    tau = max(tau_k, v)
            return tau, []
        return tau, alts
    caught = 0
    for pin in (lambda: _check_threshold_vs_definition(bad, trials=300), lambda: _check_topp_examples(bad)):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1


def test_plant_draft_row_unfiltered(monkeypatch):
    """The target rows filtered but the draft rows not (with K = 2 a sequence
    builds 3 target rows, then 2 draft rows): proposals drawn from the
    filtered draft then come out with the wrong law."""
    real = ov.filtered_softmax
    seen = {"i": 0}

    def fs(x, T, tau):
        seen["i"] += 1
        return real(x, T, tau if seen["i"] % 5 in (1, 2, 3) else -np.inf)
    monkeypatch.setattr(ov, "filtered_softmax", fs)
    with pytest.raises(AssertionError):
        _check_lossless(ov.SAMPLE, 4, 0.8)
