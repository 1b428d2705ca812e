"""CPU pins of the N-gram proposer oracle: the worked example the page
asserts, the definition checked property by property on random histories,
and planted mistakes that each pin must catch."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import ngram as on

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ngram_propose_examples.json")


def _check_golden(propose):
    with open(GOLDEN) as f:
        g = json.load(f)
    for c in g["cases"]:
        n, toks, _ = propose(c["history"], c["min_n"], c["max_n"], c["max_tokens"])
        assert n == c["window"] and toks == c["proposal"], (c, n, toks)


def _check_properties(propose, trials=400, seed=0):
    """The returned (n, s, proposal) against the definition, without
    re-running a search: the window really matches, it leaves a gap before
    the tail, no longer window matches anywhere, no later start matches for
    this window, and the proposal is the continuation clipped at the tail."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        L = int(rng.integers(0, 40))
        vocab = int(rng.integers(1, 6))
        h = rng.integers(0, vocab, L)
        min_n = int(rng.integers(1, 4))
        max_n = min_n + int(rng.integers(0, 4))
        mt = int(rng.integers(1, 7))
        n, toks, s = propose(h, min_n, max_n, mt)
        if n is None:
            for m in range(min_n, max_n + 1):     # no window of any length has a valid start
                for t in range(0, L - 2 * m):
                    assert not np.array_equal(h[t:t + m], h[L - m:]), (h, m, t)
            assert toks == []
            continue
        assert min_n <= n <= max_n
        assert s + n < L - n and np.array_equal(h[s:s + n], h[L - n:])
        for m in range(n + 1, max_n + 1):        # no longer window matches
            for t in range(0, L - 2 * m):
                assert not np.array_equal(h[t:t + m], h[L - m:]), (h, m, t)
        for t in range(s + 1, L - 2 * n):        # no more recent start for this window
            assert not np.array_equal(h[t:t + n], h[L - n:]), (h, n, t)
        want = list(h[s + n:min(s + n + mt, L - n)])
        assert toks == want and 1 <= len(toks) <= mt


def test_golden_examples():
    _check_golden(oracle.ngram_propose)


def test_definition_on_random_histories():
    _check_properties(oracle.ngram_propose)


def test_batch_wrapper_pads_and_counts():
    hist = np.array([10, 11, 12, 20, 21, 99, 10, 11, 12, 1, 2, 3, 4, 5, 7, 7, 7, 7, 7], np.int32)
    off = np.array([0, 9, 14, 19, 19])
    d, num, win = oracle.ngram_propose_batch(hist, off, 2, 4, 3)
    assert d[0].tolist() == [20, 21, 99] and num[0] == 3 and win[0] == 3
    assert num[1] == 0 and win[1] == 0 and (d[1] == -1).all()
    # five equal tokens: the 2-gram at s = 0 is the only start that leaves a gap before the tail
    assert win[2] == 2 and d[2].tolist() == [7, -1, -1] and num[2] == 1
    assert num[3] == 0                            # empty history


# ---- planted mistakes: each must fail at least one of the two pins ---------

def _mut_overlap(h, min_n, max_n, mt):           # lets the match touch the tail (empty continuation allowed)
    h = np.asarray(h)
    L = len(h)
    for n in range(max_n, min_n - 1, -1):
        for s in range(L - 2 * n, -1, -1):
            if s >= 0 and np.array_equal(h[s:s + n], h[L - n:]):
                return n, list(h[s + n:min(s + n + mt, L - n)]), s
    return None, [], None


def _mut_earliest(h, min_n, max_n, mt):          # oldest occurrence instead of the most recent
    h = np.asarray(h)
    L = len(h)
    for n in range(max_n, min_n - 1, -1):
        st = on.valid_starts(h, n)
        if len(st):
            s = int(st[0])
            return n, list(h[s + n:min(s + n + mt, L - n)]), s
    return None, [], None


def _mut_short_first(h, min_n, max_n, mt):       # shortest window first
    h = np.asarray(h)
    L = len(h)
    for n in range(min_n, max_n + 1):
        st = on.valid_starts(h, n)
        if len(st):
            s = int(st[-1])
            return n, list(h[s + n:min(s + n + mt, L - n)]), s
    return None, [], None


def _mut_copy_into_tail(h, min_n, max_n, mt):    # continuation runs on into the tail
    n, toks, s = oracle.ngram_propose(h, min_n, max_n, mt)
    if n is None:
        return n, toks, s
    h = np.asarray(h)
    return n, list(h[s + n:s + n + mt]), s


@pytest.mark.parametrize("mutant", [_mut_overlap, _mut_earliest, _mut_short_first, _mut_copy_into_tail])
def test_pins_catch_planted_mistakes(mutant):
    caught = False
    for pin in (lambda: _check_golden(mutant), lambda: _check_properties(mutant, trials=400, seed=1)):
        try:
            pin()
        except AssertionError:
            caught = True
    assert caught, mutant.__name__


def test_bench_scan_bytes_match_oracle_starts():
    """bench.py counts the bytes a scan from the end must read from the
    proposer's window lengths alone; on a seeded batch they must equal the
    depth down to the oracle's chosen start (whole history otherwise)."""
    import bench
    from workloads import make_ngram_batch
    b = make_ngram_batch(11, B=40, min_len=1, max_len=3000, vocab=200, p_tail_hit=0.6)
    _, _, win = oracle.ngram_propose_batch(b.history, b.offsets, b.min_n, b.max_n, b.max_tokens)
    want = 0
    for i in range(b.batch):
        h = b.history[b.offsets[i]:b.offsets[i + 1]]
        L = len(h)
        n, _, s = oracle.ngram_propose(h, b.min_n, b.max_n, b.max_tokens)
        want += 4 * ((L - s) if n is not None and n == min(b.max_n, (L - 1) // 2) else L)
    assert (win == min(b.max_n, 4)).sum() > 0            # some histories stop early
    assert bench.ngram_scan_bytes(b, win) == want
