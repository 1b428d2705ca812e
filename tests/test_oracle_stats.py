"""CPU pins of the acceptance-statistics and draft-length-controller oracle:
counts derived by hand on a tiny batch, the closed forms of the
AIInfraGuide page's section 7.2 under a fixed proposal length, a Bernoulli
acceptance model whose rates are known, traced controller runs, and planted
mistakes that each pin must catch."""
import math

import numpy as np
import pytest

from oracle import stats as os_
from oracle import verify as ov
from workloads import make_config_batch


# ---- counters and summary ----------------------------------------------------

def _hand_case():
    """Rounds (K, A) with max_k = 4 and their counters, worked out by hand:
    (3,1) (3,3) (0,0) (2,0) (4,-1: not verified) (5,2: K > max_k) (4,4) (1,2: A > K)."""
    K = [3, 3, 0, 2, 4, 5, 4, 1]
    A = [1, 3, 0, 0, -1, 2, 4, 2]
    # counted rounds: (3,1) (3,3) (0,0) (2,0) (4,4)
    want = {0: 5, 1: 12, 2: 8, 3: 4, 4: 2, 5: 3, 6: 13, 7: 0}
    proposed = [4, 4, 3, 1]          # K > i
    reached = [4, 3, 2, 1]           # K > i and A >= i
    accepted = [3, 2, 2, 1]          # A > i
    return K, A, want, proposed, reached, accepted


def _check_hand(counters):
    K, A, want, pr, re_, ac = _hand_case()
    c = counters(K, A, 4)
    for k, v in want.items():
        assert int(c[k]) == v, (k, int(c[k]), v)
    assert [int(x) for x in c[8:12]] == pr
    assert [int(x) for x in c[12:16]] == re_
    assert [int(x) for x in c[16:20]] == ac


def test_hand_counted_case():
    _check_hand(os_.acceptance_counters)
    K, A, *_ = _hand_case()
    s = os_.acceptance_summary(os_.acceptance_counters(K, A, 4), 4)
    assert s[0] == 8 / 12 and s[1] == 1 + 8 / 5 and s[2] == 4 / 5 and s[3] == 2 / 4
    assert list(s[4:8]) == [3 / 4, 2 / 3, 2 / 2, 1 / 1]
    assert list(s[8:12]) == [3 / 4, 2 / 4, 2 / 3, 1 / 1]


def _fixed_gamma_rounds(rng, gamma, n, beta):
    """n rounds proposing gamma tokens, each accepted independently with
    probability beta until the first rejection."""
    u = rng.random((n, gamma))
    ok = u < beta
    A = np.where(ok.all(axis=1), gamma, np.argmin(ok, axis=1))
    return np.full(n, gamma), A


def _check_closed_forms(counters, summary):
    rng = np.random.default_rng(5)
    for gamma in (1, 3, 6):
        K, A = _fixed_gamma_rounds(rng, gamma, 4000, 0.7)
        c = counters(K, A, 8)
        s = summary(c, 8)
        R, D, C = int(c[0]), int(c[1]), int(c[2])
        assert D == gamma * R                                      # 7.2: D = gamma R
        assert math.isclose(s[1], 1 + gamma * C / D, rel_tol=1e-12)  # 7.2: 1 + gamma C / D
        assert int(c[6]) == C + R                                  # every round commits one more token
        assert int(c[3]) == R                                      # every round had candidates
        for i in range(gamma):                                     # through-rate = product of conditionals
            assert math.isclose(s[4 + 8 + i], float(np.prod(s[4:4 + i + 1])), rel_tol=1e-12)
        for i in range(gamma, 8):
            assert math.isnan(s[4 + i]) and math.isnan(s[4 + 8 + i])


def test_closed_forms_fixed_length():
    _check_closed_forms(os_.acceptance_counters, os_.acceptance_summary)


def _check_bernoulli(counters, summary):
    """Independent acceptance with probability beta at every position, lengths
    K ~ U{0..6}: the conditional rate is beta at every position and the rate
    through i is beta^(i+1); coverage is 6/7 (within 5 sigma)."""
    rng = np.random.default_rng(6)
    n, beta = 60000, 0.65
    K = rng.integers(0, 7, n)
    u = rng.random((n, 6))
    A = np.array([k if (u[j, :k] < beta).all() else int(np.argmin(u[j, :k] < beta)) for j, k in enumerate(K)])
    c = counters(K, A, 6)
    s = summary(c, 6)
    for i in range(6):
        m = int(c[8 + 6 + i])
        assert abs(s[4 + i] - beta) < 5 * math.sqrt(beta * (1 - beta) / m), (i, s[4 + i])
        m = int(c[8 + i])
        b = beta ** (i + 1)
        assert abs(s[10 + i] - b) < 5 * math.sqrt(b * (1 - b) / m), (i, s[10 + i])
    assert abs(s[2] - 6 / 7) < 5 * math.sqrt((6 / 7) * (1 / 7) / n)


def test_bernoulli_model_rates():
    _check_bernoulli(os_.acceptance_counters, os_.acceptance_summary)


def test_counters_from_the_verify_oracle():
    """Rounds produced by the verify oracle on a seeded batch: C is the sum of
    accepted lengths and the emitted-token count is the number of emitted
    tokens the verify step reports."""
    b = make_config_batch(0, 0)
    for seed in range(5):
        b.seed = seed
        r = ov.verify_batch_from(b)
        c = os_.acceptance_counters(b.num_draft, r.accepted_len, 8)
        assert int(c[2]) == int(r.accepted_len.sum())
        assert int(c[6]) == int((r.emitted >= 0).sum())


def test_accumulation_over_calls():
    rng = np.random.default_rng(9)
    K = rng.integers(0, 5, 50)
    A = np.minimum(rng.integers(-1, 5, 50), K)
    whole = os_.acceptance_counters(K, A, 4)
    acc = os_.acceptance_counters(K[:20], A[:20], 4)
    os_.acceptance_counters(K[20:], A[20:], 4, into=acc)
    assert (acc == whole).all()


# ---- controllers -------------------------------------------------------------
#
# The ratio a controller sees, by default, is the tutorial's (section 4.3
# verifier, section 4.4 decoder): len(accepted_tokens) / draft_len, where the
# verifier returns the accepted draft tokens and, after a rejection, the token
# drawn in its place (no bonus).  Traced by hand: K = 4 with A = 1 gives
# accepted_tokens = [x0, y1], ratio 2/4; A = 4 gives [x0..x3], ratio 1; K = 0
# gives an empty list, ratio 0 (the decoder's `else 0`).

EMIT, DRAFT = os_.COUNT_EMITTED, os_.COUNT_DRAFT_ONLY


def _run(kind, rounds, length, **kw):
    st = os_.Controller(length)
    return [os_.adapt_step(st, K, A, kind, **kw) for K, A in rounds]


def test_controller_ratio_traced():
    assert [os_.controller_ratio(4, a) for a in range(5)] == [1 / 4, 2 / 4, 3 / 4, 4 / 4, 4 / 4]
    assert os_.controller_ratio(0, 0) == 0.0 and os_.controller_ratio(1, 0) == 1.0
    assert [os_.controller_ratio(4, a, DRAFT) for a in range(5)] == [0.0, 0.25, 0.5, 0.75, 1.0]
    assert os_.controller_ratio(0, 0, DRAFT) == 0.0


def _check_window(step_fn, count=EMIT):
    kw = dict(min_k=1, max_k=7, window=12, min_samples=10, target=0.7, count=count)
    st = os_.Controller(5)
    full = [step_fn(st, 4, 4, os_.WINDOW, **kw) for _ in range(14)]
    # nine rounds: too few samples; from the tenth on the mean (1.0) is above 0.8
    assert full == [5] * 9 + [6, 7, 7, 7, 7]
    # now rounds of ratio 1/4: (4, 0) as the tutorial counts (one token returned),
    # (4, 1) counted by draft tokens; the 12-entry window's mean drops as the full
    # rounds leave it
    low = [step_fn(st, 4, 0 if count == EMIT else 1, os_.WINDOW, **kw) for _ in range(12)]
    means = [(12 - j - 1 + 0.25 * (j + 1)) / 12 for j in range(12)]
    want, L = [], 7
    for m in means:
        if m > 0.8:
            L = min(7, L + 1)
        elif m < 0.6:
            L = max(1, L - 1)
        want.append(L)
    assert low == want and want[-1] == 1 and want[0] == 7
    # a mean inside the band changes nothing: (10, 6) is 7/10 counted the tutorial's way,
    # (10, 7) is 7/10 counted by draft tokens
    st = os_.Controller(3)
    mid = [step_fn(st, 10, 6 if count == EMIT else 7, os_.WINDOW, **kw) for _ in range(15)]
    assert mid == [3] * 15
    # K = 0 counts as ratio 0
    st = os_.Controller(3)
    assert [step_fn(st, 0, 0, os_.WINDOW, **kw) for _ in range(11)][-1] == 1
    # a round that was not verified is no sample
    st = os_.Controller(5)
    assert [step_fn(st, 4, -1, os_.WINDOW, **kw) for _ in range(20)] == [5] * 20


@pytest.mark.parametrize("count", [EMIT, DRAFT])
def test_window_controller_traced(count):
    _check_window(os_.adapt_step, count)


def _check_multiplicative(step_fn, count=EMIT):
    kw = dict(min_k=1, max_k=20, target=0.7, rate=0.1, count=count)
    st = os_.Controller(10)
    assert step_fn(st, 4, 4, os_.MULTIPLICATIVE, **kw) == 11          # int(11.0)
    assert step_fn(st, 4, 4, os_.MULTIPLICATIVE, **kw) == 12          # int(12.100000000000001)
    if count == EMIT:
        # (4, 3): the rejected round still returns 4 tokens, ratio 1.0 -> int(13.200000000000001)
        assert step_fn(st, 4, 3, os_.MULTIPLICATIVE, **kw) == 13
        assert step_fn(st, 4, 2, os_.MULTIPLICATIVE, **kw) == 13      # 3/4 is inside 0.6..0.8
        assert step_fn(st, 4, 1, os_.MULTIPLICATIVE, **kw) == 11      # 2/4: int(11.700000000000001)
    else:
        assert step_fn(st, 4, 3, os_.MULTIPLICATIVE, **kw) == 12      # 0.75 is inside 0.6..0.8
        assert step_fn(st, 4, 2, os_.MULTIPLICATIVE, **kw) == 10      # int(10.8)
    st = os_.Controller(5)                                             # int(5.5) = 5: stuck, as written
    assert [step_fn(st, 5, 5, os_.MULTIPLICATIVE, **kw) for _ in range(3)] == [5, 5, 5]
    st = os_.Controller(2)                                             # (3, 0): 1/3 or 0, both below 0.6
    assert [step_fn(st, 3, 0, os_.MULTIPLICATIVE, **kw) for _ in range(2)] == [1, 1]   # floor min_k
    st = os_.Controller(19)
    assert step_fn(st, 3, 3, os_.MULTIPLICATIVE, min_k=1, max_k=20, target=0.7, rate=0.5,
                   count=count) == 20                                  # int(28.5) capped


@pytest.mark.parametrize("count", [EMIT, DRAFT])
def test_multiplicative_controller_traced(count):
    _check_multiplicative(os_.adapt_step, count)


def _series_x(a, terms=4000):
    """-ln(1 - a) / a as the power series sum_{j>=0} a^j / (j + 1)."""
    return sum(a ** j / (j + 1) for j in range(terms))


def _check_optimal_k(step_fn, count=EMIT):
    kw = dict(min_k=1, max_k=16, count=count)
    st = os_.Controller(8)
    assert step_fn(st, 4, 4, os_.OPTIMAL_K, **kw) == 8      # a = 1: k* infinite -> 16, min with L
    st = os_.Controller(40)
    assert step_fn(st, 4, 4, os_.OPTIMAL_K, **kw) == 16
    st = os_.Controller(1)
    assert step_fn(st, 4, 4, os_.OPTIMAL_K, **kw) == 2      # max(L, 2)
    # (K, A) with the accepted count as each reading has it: the correction counted, or not
    for K, A, n_emit in [(2, 0, 1), (100, 98, 99), (1000, 998, 999), (5, 0, 1), (128, 126, 127), (128, 119, 120)]:
        n = n_emit if count == EMIT else A
        a = max(n / K, 0.01)
        want = min(16, max(2, math.floor(_series_x(a, 20000))))
        st = os_.Controller(16)
        assert step_fn(st, K, A, os_.OPTIMAL_K, **kw) == want, (K, A)


@pytest.mark.parametrize("count", [EMIT, DRAFT])
def test_optimal_k_controller_against_series(count):
    _check_optimal_k(os_.adapt_step, count)


def test_optimal_k_has_no_near_integer_case():
    """The device takes floor(ln(1/(1-a))/a) with its own float64 log: for every
    ratio A/K with K <= 128 the value stays clear of an integer in 2..16 by far
    more than a few ulps, so both sides take the same floor."""
    worst = 1.0
    for K in range(1, 129):
        for A in range(0, K):
            a = max(A / K, 0.01)
            x = math.log(1.0 / (1.0 - a)) / a
            if 2 <= x < 17:
                worst = min(worst, abs(x - round(x)) / x)
    assert worst > 1e-9, worst


# ---- planted mistakes ----------------------------------------------------------

def _mut_reached_strict(K, A, max_k, into=None):
    c = os_.acceptance_counters(K, A, max_k, into)
    for k, a in zip(K, A):
        if 0 <= a <= k <= max_k and a < k:
            c[8 + max_k + a] -= 1          # "reached" as A > i
    return c


def _mut_no_bonus_check(K, A, max_k, into=None):
    c = os_.acceptance_counters(K, A, max_k, into)
    c[3] = c[0]                            # coverage counts rounds without candidates
    return c


def _mut_summary_no_one(c, max_k):
    s = os_.acceptance_summary(c, max_k)
    s[1] -= 1.0                            # mean length without the committed token
    return s


def _mut_through_uses_reached(c, max_k):
    s = os_.acceptance_summary(c, max_k)
    s[4 + max_k:] = s[4:4 + max_k]
    return s


@pytest.mark.parametrize("mut", ["reached", "coverage", "mean_len", "through"])
def test_pins_catch_counter_mistakes(mut):
    counters, summary = os_.acceptance_counters, os_.acceptance_summary
    if mut == "reached":
        counters = _mut_reached_strict
    elif mut == "coverage":
        counters = _mut_no_bonus_check
    elif mut == "mean_len":
        summary = _mut_summary_no_one
    else:
        summary = _mut_through_uses_reached
    caught = 0
    for pin in (lambda: _check_hand(counters), lambda: _check_closed_forms(counters, summary),
                lambda: _check_bernoulli(counters, summary)):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, mut


def _mut_window_ge(st, K, A, kind, **kw):
    """>= instead of > against target + 0.1, and no sample gate."""
    if A < 0:
        return st.length
    st.recent.append(os_.controller_ratio(K, A, kw["count"]))
    while len(st.recent) > kw["window"]:
        st.recent.popleft()
    avg = sum(st.recent) / len(st.recent)
    if avg >= kw["target"] + os_.BAND:
        st.length = min(kw["max_k"], st.length + 1)
    elif avg < kw["target"] - os_.BAND:
        st.length = max(kw["min_k"], st.length - 1)
    return st.length


def _mut_ratio_without_correction(st, K, A, kind, **kw):
    """The tutorial's count without the token drawn after a rejection."""
    return os_.adapt_step(st, K, A, kind, **{**kw, "count": DRAFT})


def _mut_ratio_with_bonus(st, K, A, kind, **kw):
    """The bonus token counted as well: (A + 1) / K after a fully accepted round."""
    if A < 0:
        return st.length
    if A == K and K > 0 and kind == os_.MULTIPLICATIVE:
        r = (A + 1) / K
        if r > kw["target"] + os_.BAND:
            st.length = min(kw["max_k"], int(st.length * (1 + kw["rate"]) * r))
        return st.length
    return os_.adapt_step(st, K, A, kind, **kw)


def _mut_round_not_trunc(st, K, A, kind, **kw):
    if A < 0:
        return st.length
    r = os_.controller_ratio(K, A, kw["count"])
    if r > kw["target"] + os_.BAND:
        st.length = min(kw["max_k"], round(st.length * (1 + kw["rate"])))
    elif r < kw["target"] - os_.BAND:
        st.length = max(kw["min_k"], round(st.length * (1 - kw["rate"])))
    return st.length


def _mut_optimal_no_floor_two(st, K, A, kind, **kw):
    a = max(os_.controller_ratio(K, A, kw["count"]), 0.01)
    x = math.log(1.0 / (1.0 - a)) / a if a < 1 else math.inf
    st.length = min(16 if x >= 16 else int(x), max(st.length, 2))
    return st.length


@pytest.mark.parametrize("mut,check", [(_mut_window_ge, _check_window),
                                       (_mut_ratio_without_correction, _check_window),
                                       (_mut_ratio_without_correction, _check_multiplicative),
                                       (_mut_ratio_without_correction, _check_optimal_k),
                                       (_mut_ratio_with_bonus, _check_multiplicative),
                                       (_mut_round_not_trunc, _check_multiplicative),
                                       (_mut_optimal_no_floor_two, _check_optimal_k)])
def test_pins_catch_controller_mistakes(mut, check):
    with pytest.raises(AssertionError):
        check(mut)
