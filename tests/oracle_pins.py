"""Checks that pin the CPU oracle to facts fixed by the pages or by mathematics.

Each ``check_*`` raises AssertionError when the oracle disagrees.  They are
plain functions so that the mutation tests can run them against an oracle
with a planted mistake and expect them to fail.

Sources: [DM] "Draft Model（草稿模型）" (compassingai.com) §2 接受-拒绝准则,
接受率分析, the one-step algorithm box; [TUT] gitcode.csdn.net tutorial
§3.2, §3.3, §4.3; [AIG] "5.2 Draft 模型与无模型方案" §4.3, §7.
Independent references used here: scipy.special.softmax, numpy.argmax.
"""
from __future__ import annotations

import json
import os

import numpy as np
from scipy import special, stats

import oracle
from oracle import verify as ov
from oracle.philox import verify_uniform, PURPOSE_ACCEPT, PURPOSE_SAMPLE

HERE = os.path.dirname(os.path.abspath(__file__))
P_MIN = 1e-4   # chi-square p-value floor at fixed seeds (deterministic)


def golden_worked_example():
    with open(os.path.join(HERE, "golden", "worked_example_reject_one_third.json")) as f:
        return json.load(f)


def run_replicated(rows_t, rows_d, tokens, T, mode, n, seed=0, seq_base=0, tokens_per_seq=None):
    """Verify n copies of one sequence (identical rows, K = len(tokens)) that
    differ only in seq_id, so each copy draws its own uniforms."""
    rows_t = np.asarray(rows_t, np.float32)
    K = rows_t.shape[0] - 1
    V = rows_t.shape[1]
    target = np.tile(rows_t, (n, 1))
    draft = np.tile(np.asarray(rows_d, np.float32), (n, 1)) if rows_d is not None else None
    if tokens_per_seq is None:
        toks = np.tile(np.asarray(tokens, np.int32), n)
    else:
        toks = np.asarray(tokens_per_seq, np.int32).reshape(-1)
    return oracle.verify_batch(target=target, draft=draft, dtype="f32", vocab=V,
                               num_draft=np.full(n, K, np.int32), draft_tokens=toks,
                               temperature=np.full(n, T, np.float32),
                               mode=np.full(n, mode, np.uint8),
                               seq_ids=np.arange(seq_base, seq_base + n, dtype=np.uint32), seed=seed)


def chi2_ok(observed, probs, what=""):
    observed = np.asarray(observed, np.float64)
    probs = np.asarray(probs, np.float64)
    n = observed.sum()
    assert n > 0, what
    exp = probs / probs.sum() * n
    keep = exp > 0
    assert observed[~keep].sum() == 0, f"{what}: mass on zero-probability tokens"
    pv = stats.chisquare(observed[keep], exp[keep]).pvalue
    assert pv > P_MIN, f"{what}: chi-square p-value {pv:.3g}"


def _emitted_matrix(res, K):
    return res.emitted.reshape(-1, K + 1)


# ---------------------------------------------------------------------------
# [TUT] §3.3 worked example: p=0.4, q=0.6 -> reject with probability 1/3
# ---------------------------------------------------------------------------

def check_worked_example(n=30000):
    g = golden_worked_example()
    p, q, x = np.array(g["p"]), np.array(g["q"]), int(g["proposed"])
    r = ov.accept_ratio(ov.SAMPLE, p[x], q[x])
    assert abs(r - g["accept_probability"]) < 1e-12
    assert abs((1 - r) - g["reject_probability"]) < 1e-12
    w = ov.residual(ov.SAMPLE, p, q, x)
    assert np.allclose(w / w.sum(), g["residual_normalised"], atol=1e-12)

    lt, ld = np.log(p), np.log(q)
    res = run_replicated([lt, lt], [ld], [x], 1.0, ov.SAMPLE, n)
    em = _emitted_matrix(res, 1)
    rej = res.accepted_len == 0
    frac = rej.mean()
    sigma = np.sqrt(g["reject_probability"] * (1 - g["reject_probability"]) / n)
    assert abs(frac - g["reject_probability"]) < 5 * sigma, f"reject fraction {frac}"
    assert (em[rej, 0] == 1).all(), "a rejection must redraw the other token"
    assert (em[~rej, 0] == x).all()
    # the exact count: rejections are exactly the copies whose uniform is >= r
    u = np.array([verify_uniform(0, s, 0, PURPOSE_ACCEPT) for s in range(n)])
    assert (rej == (u >= res.seqs[0].ratios[0])).all()


def check_marginal_with_q_proposals(n=30000):
    g = golden_worked_example()
    p, q = np.array(g["p"]), np.array(g["q"])
    rng = np.random.default_rng(123)
    toks = rng.choice(2, size=n, p=q)
    lt, ld = np.log(p), np.log(q)
    res = run_replicated([lt, lt], [ld], None, 1.0, ov.SAMPLE, n, tokens_per_seq=toks)
    y0 = _emitted_matrix(res, 1)[:, 0]
    chi2_ok(np.bincount(y0, minlength=2), g["marginal_with_proposal_from_q"], "worked example marginal")


# ---------------------------------------------------------------------------
# [DM] §2: the emitted token at every reached position is distributed as p
# ---------------------------------------------------------------------------

def _tiny_rows(seed, K, V, scale=1.2, noise=1.0):
    rng = np.random.default_rng(seed)
    t = (scale * rng.standard_normal((K + 1, V))).astype(np.float32)
    d = (t[:K] + noise * rng.standard_normal((K, V))).astype(np.float32)
    return t, d


def check_lossless(n=20000, T=1.0, mode=ov.SAMPLE, K=3, V=6, seed=1):
    t, d = _tiny_rows(seed, K, V)
    p = [special.softmax(t[i].astype(np.float64) / T) for i in range(K + 1)]
    q = [special.softmax(d[i].astype(np.float64) / T) for i in range(K)]
    rng = np.random.default_rng(seed + 100)
    if mode == ov.SAMPLE:
        toks = np.stack([rng.choice(V, size=n, p=q[i]) for i in range(K)], axis=1)
    else:   # one-hot proposals: any proposal rule, here uniform over the vocabulary
        toks = rng.integers(0, V, size=(n, K))
    res = run_replicated(t, d if mode == ov.SAMPLE else None, None, T, mode, n, tokens_per_seq=toks)
    em = _emitted_matrix(res, K)
    A = res.accepted_len
    for j in range(K + 1):
        reached = A >= j
        obs = np.bincount(em[reached, j], minlength=V)
        chi2_ok(obs, p[j], f"mode={mode} T={T} position {j}")
    # the bonus row is p_K given every proposal was accepted
    allacc = A == K
    chi2_ok(np.bincount(em[allacc, K], minlength=V), p[K], "bonus")
    return res


def check_k_zero_is_plain_sampling(n=20000, V=7, T=0.8):
    rng = np.random.default_rng(9)
    t = (1.5 * rng.standard_normal((1, V))).astype(np.float32)
    p = special.softmax(t[0].astype(np.float64) / T)
    res = run_replicated(t, np.zeros((0, V), np.float32), [], T, ov.SAMPLE, n)
    assert (res.accepted_len == 0).all()
    chi2_ok(np.bincount(res.emitted, minlength=V), p, "K=0")


# ---------------------------------------------------------------------------
# exact law over the whole 2^24 grid of uniforms (no statistics)
# ---------------------------------------------------------------------------

GRID = np.arange(2 ** 24, dtype=np.float64) * 2.0 ** -24


def _grid_accept_prob(r):
    return np.count_nonzero(GRID < r) / 2 ** 24


def check_grid_exact(seed=3, V=5, T=1.0):
    rng = np.random.default_rng(seed)
    xt = rng.standard_normal(V) * 1.3
    xd = xt + rng.standard_normal(V)
    p, q = special.softmax(xt / T), special.softmax(xd / T)
    law = np.zeros(V)
    acc_total = 0.0
    for x in range(V):
        r = ov.accept_ratio(ov.SAMPLE, p[x], q[x])
        a = _grid_accept_prob(r)
        assert abs(a - min(1.0, p[x] / q[x])) <= 2.0 ** -24
        acc_total += q[x] * a
        law[x] += q[x] * a
        if a < 1:
            w = ov.residual(ov.SAMPLE, p, q, x)
            ys = ov.inverse_cdf(w, GRID)
            cnt = np.bincount(ys, minlength=V) / 2 ** 24
            assert np.all(np.abs(cnt - w / w.sum()) <= 2.0 ** -24 + 1e-15)
            assert cnt[w == 0].sum() == 0
            law += q[x] * (1 - a) * cnt
    # [DM] 接受率分析: acceptance = sum min(p, q) = 1 - TV(p, q)
    assert abs(acc_total - np.minimum(p, q).sum()) < V * 2.0 ** -23
    assert abs(acc_total - (1 - 0.5 * np.abs(p - q).sum())) < V * 2.0 ** -23
    # [DM] §2: the emitted token's law is p
    assert np.max(np.abs(law - p)) < V * 2.0 ** -22


def check_grid_onehot(seed=4, V=6):
    """[AIG] §4.3: q = one-hot on x; for every x the emitted law is p."""
    rng = np.random.default_rng(seed)
    p = special.softmax(rng.standard_normal(V) * 1.5)
    for x in range(V):
        r = ov.accept_ratio(ov.ONEHOT, p[x], 1.0)
        a = _grid_accept_prob(r)
        w = ov.residual(ov.ONEHOT, p, None, x)
        cnt = np.bincount(ov.inverse_cdf(w, GRID), minlength=V) / 2 ** 24
        law = (1 - a) * cnt
        law[x] += a
        assert np.max(np.abs(law - p)) < V * 2.0 ** -22


# ---------------------------------------------------------------------------
# [DM] 接受率分析 / [AIG] §7 on a benchmark workload: mean accepted length
# ---------------------------------------------------------------------------

def check_acceptance_law_on_workload(steps=300):
    from workloads import make_config_batch, bf16_widen
    got, want, var = [], [], []
    for step in range(steps):
        b = make_config_batch(0, step)
        res = oracle.verify_batch_from(b)
        K = int(b.num_draft[0])
        T = float(b.temperature[0])
        beta = []
        for i in range(K):
            p = special.softmax(b.target[i].astype(np.float64)[:b.vocab] / T)
            q = special.softmax(b.draft[i].astype(np.float64)[:b.vocab] / T)
            beta.append(np.minimum(p, q).sum())
        reach = np.cumprod([1.0] + beta)          # P(A >= j), j = 0..K
        EA = reach[1:].sum()
        EA2 = sum((2 * j - 1) * reach[j] for j in range(1, K + 1))
        got.append(res.accepted_len[0])
        want.append(EA)
        var.append(EA2 - EA ** 2)
    got, want = np.array(got, float), np.array(want)
    se = np.sqrt(np.sum(var)) / steps
    assert abs(got.mean() - want.mean()) < 5 * se, (got.mean(), want.mean(), se)


# ---------------------------------------------------------------------------
# greedy equivalence, special cases, uniform wiring
# ---------------------------------------------------------------------------

def check_greedy_equivalence():
    from workloads import make_random_batch, bf16_widen
    for seed, dtype in ((0, "f32"), (1, "bf16"), (2, "bf16")):
        b = make_random_batch(seed, B=40, V=50, kmax=6, dtype=dtype, modes=(ov.GREEDY,), p_hit=0.8)
        outs = []
        for philox_seed, Tmul in ((0, 1.0), (999, 3.0)):
            res = oracle.verify_batch(target=b.target, draft=None, dtype=dtype, vocab=b.vocab,
                                      num_draft=b.num_draft, draft_tokens=b.draft_tokens,
                                      temperature=b.temperature * Tmul, mode=b.mode,
                                      seq_ids=b.seq_ids, seed=philox_seed)
            outs.append((res.accepted_len.copy(), res.emitted.copy()))
            rt = rd = 0
            for s in range(b.batch):
                K = int(b.num_draft[s])
                rows = b.target[rt:rt + K + 1]
                rows = bf16_widen(rows) if dtype == "bf16" else rows
                am = [int(np.argmax(rows[i])) for i in range(K + 1)]
                A = next((i for i in range(K) if b.draft_tokens[rd + i] != am[i]), K)
                assert res.accepted_len[s] == A
                want = list(b.draft_tokens[rd:rd + A]) + [am[A]] + [-1] * (K - A)
                assert list(res.emitted[rt:rt + K + 1]) == want
                rt += K + 1
                rd += K
        assert (outs[0][0] == outs[1][0]).all() and (outs[0][1] == outs[1][1]).all()


def check_identical_draft_always_accepts():
    from workloads import make_random_batch
    for seed in range(4):
        b = make_random_batch(seed, B=30, V=40, kmax=6, modes=(ov.SAMPLE,), identical_draft=True,
                              dtype="bf16" if seed % 2 else "f32")
        res = oracle.verify_batch_from(b)
        assert (res.accepted_len == b.num_draft).all()


def check_onehot_certain_token_accepted():
    V, K, n = 8, 3, 200
    t = np.full((K + 1, V), -np.inf, np.float32)
    toks = [2, 5, 0]
    for i, x in enumerate(toks):
        t[i, x] = 0.0
    t[K, :] = 0.0
    res = run_replicated(t, None, toks, 1.0, ov.ONEHOT, n)
    assert (res.accepted_len == K).all()
    assert (res.status == 0).all()


def check_uniform_wiring(seed=17, seq_id=5):
    """Position i's acceptance uses the uniform at (seq_id, i, purpose 0):
    set r_i just above u_i for i < j and just below at j, expect A = j."""
    K = 5
    u = [verify_uniform(seed, seq_id, i, PURPOSE_ACCEPT) for i in range(K)]
    for j in range(K + 1):
        t_rows, d_rows = [], []
        for i in range(K):
            r = u[i] + 3e-5 if i < j else u[i] - 3e-5
            r = min(max(r, 1e-6), 1 - 1e-6)
            qx = 0.9
            px = r * qx
            t_rows.append(np.log([px, 1 - px]))
            d_rows.append(np.log([qx, 1 - qx]))
        t_rows.append(np.log([0.5, 0.5]))
        res = oracle.verify_batch(target=np.array(t_rows, np.float64).astype(np.float32),
                                  draft=np.array(d_rows).astype(np.float32), dtype="f32", vocab=2,
                                  num_draft=[K], draft_tokens=np.zeros(K, np.int32), temperature=[1.0],
                                  mode=[ov.SAMPLE], seq_ids=[seq_id], seed=seed)
        want = j if j < K else K
        # a rounding-level r on the far side of u would be flagged; the margins avoid that
        assert not res.seqs[0].accept_flags
        assert res.accepted_len[0] == want, (j, res.accepted_len[0])


def check_final_uniform_wiring(n=400, m=6, seed=23):
    """The final draw uses the uniform at (seq_id, A, purpose 1): with a
    uniform target over V = 2^m tokens and all proposals accepted, the
    inverse CDF returns floor(u * V) exactly."""
    V = 2 ** m
    K = 2
    t = np.zeros((K + 1, V), np.float32)
    res = run_replicated(t, None, [0, 0], 1.0, ov.GREEDY, 1)   # greedy sanity: argmax ties -> 0
    assert res.emitted[-1] == 0
    t[:K, 0] = 50.0          # make the one-hot proposals certain
    res = run_replicated(t, None, [0, 0], 1.0, ov.ONEHOT, n, seed=seed)
    assert (res.accepted_len == K).all()
    u = np.array([verify_uniform(seed, s, K, PURPOSE_SAMPLE) for s in range(n)])
    assert (res.emitted.reshape(n, K + 1)[:, K] == np.floor(u * V).astype(int)).all()


def check_inverse_cdf_convention():
    w = np.array([1.0, 1.0, 1.0, 1.0])
    assert int(ov.inverse_cdf(w, 0.0)) == 0
    assert int(ov.inverse_cdf(w, 0.25)) == 1          # first k with C[k] > t
    assert int(ov.inverse_cdf(w, 1 - 2 ** -24)) == 3
    w = np.array([0.0, 2.0, 0.0, 1.0, 0.0])
    assert int(ov.inverse_cdf(w, 0.0)) == 1            # zero-mass tokens are never chosen
    assert int(ov.inverse_cdf(w, 2 / 3)) == 3
    assert int(ov.inverse_cdf(w, 1.0)) == 3            # clamp to the last positive weight


# ---------------------------------------------------------------------------
# strict (sample-match) mode ([DIST] §二, §三): accept iff the target's own
# sample equals the proposal, emit that sample on a mismatch
# ---------------------------------------------------------------------------

def _page_sample(p, u):
    """The target's own inverse-CDF sample, written out independently:
    first k whose inclusive cumulative sum exceeds u * total."""
    C = np.cumsum(np.asarray(p, np.float64))
    return np.searchsorted(C, np.asarray(u) * C[-1], side="right")


def check_grid_strict(seed=5, V=6):
    """Over all 2^24 uniforms: the proposal x is accepted exactly on x's
    interval (probability p(x) to the grid), and for a sample of rejected
    uniforms the emitted correction is the target's own sample; so is the
    draw from p without x at the shifted point t (t - p(x) above x's
    interval), the form the forced-branch helper uses."""
    rng = np.random.default_rng(seed)
    p = special.softmax(rng.standard_normal(V) * 1.4)
    ys = _page_sample(p, GRID)
    for x in range(V):
        acc = ys == x
        assert abs(acc.mean() - p[x]) <= 2.0 ** -24 + 1e-15, (x, acc.mean(), p[x])
        rej = np.nonzero(~acc)[0]
        for j in rng.choice(rej, size=min(3000, len(rej)), replace=False):
            u = float(GRID[j])
            f, st = ov.strict_emit(p, x, u)
            assert f.y == ys[j] and f.y != x and st == 0, (x, u, f.y, ys[j])
            w, ur = ov.strict_correction(p, x, u)
            y = int(ov.inverse_cdf(w, ur))
            assert y == ys[j], (x, u, y, ys[j])


def check_strict_acceptance_rate(n=40000, V=8, seed=6):
    """Proposals drawn from q: the first position is accepted with
    probability sum_x q(x) p(x)."""
    rng = np.random.default_rng(seed)
    t = (1.3 * rng.standard_normal((2, V))).astype(np.float32)
    p = special.softmax(t[0].astype(np.float64))
    q = special.softmax(rng.standard_normal(V) * 1.3)
    toks = rng.choice(V, size=n, p=q)
    res = run_replicated(t, None, None, 1.0, ov.STRICT, n, tokens_per_seq=toks.reshape(n, 1))
    a = (res.accepted_len == 1).mean()
    want = float((p * q).sum())
    assert abs(a - want) < 5 * np.sqrt(want * (1 - want) / n), (a, want)


def check_strict_wiring(seed=29, n=300, K=4, V=9):
    """Each decision of the batch oracle is 'the target's sample at i with
    the purpose-0 uniform of position i equals x_i', and the correction at A
    is that same sample (purpose 0 at A, not the final-draw purpose)."""
    t, _ = _tiny_rows(seed, K, V, scale=1.0)
    rng = np.random.default_rng(seed)
    p = [special.softmax(t[i].astype(np.float64) / 0.9) for i in range(K + 1)]
    toks = np.stack([np.argsort(-p[i])[rng.integers(0, 2, n)] for i in range(K)], axis=1)   # likely tokens
    res = run_replicated(t, None, None, 0.9, ov.STRICT, n, seed=seed, tokens_per_seq=toks)
    em = _emitted_matrix(res, K)
    seen_reject = 0
    for s in range(n):
        A = int(res.accepted_len[s])
        for i in range(A + (1 if A < K else 0)):
            y = int(_page_sample(p[i], verify_uniform(seed, s, i, PURPOSE_ACCEPT)))
            assert (y == toks[s, i]) == (i < A), (s, i)
            if i == A:
                assert em[s, A] == y
                seen_reject += 1
        if A == K:
            y = int(_page_sample(p[K], verify_uniform(seed, s, K, PURPOSE_SAMPLE)))
            assert em[s, K] == y
    assert seen_reject > n // 10
