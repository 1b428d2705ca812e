"""GPU-vs-oracle parity of the acceptance statistics and the draft-length
controllers through the C interface.  Counters and lengths are integers and
must be identical; the summary's rates are single correctly rounded float64
divisions on both sides and must be bitwise equal (NaN where undefined)."""
import numpy as np
import pytest

import oracle
from workloads import make_config_batch

from . import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _rounds(rng, B, max_k, p_bad=0.05):
    """Random rounds: K in 0..max_k (a few above), A in 0..K, some not verified."""
    K = rng.integers(0, max_k + 1, B)
    A = (rng.random(B) * (K + 1)).astype(np.int64)
    A = np.where(rng.random(B) < 0.3, K, A)                  # many fully accepted rounds
    bad = rng.random(B) < p_bad
    A = np.where(bad & (rng.random(B) < 0.5), -1, A)
    K = np.where(bad & (A >= 0), max_k + 1 + rng.integers(0, 3, B), K)
    return K.astype(np.int32), A.astype(np.int32)


def _dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _same_doubles(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


@pytest.mark.parametrize("max_k,sizes", [(1, [1, 7]), (8, [256, 300, 2500]), (16, [33]), (128, [1024, 1025, 64]),
                                         (70, [500])])
def test_counters_and_summary(torch_mod, max_k, sizes):
    import rejection_sampling_verify_06_amd as sv
    rng = np.random.default_rng(100 + max_k)
    st = sv.AcceptanceStats(max_k, "cuda")
    ref = np.zeros(8 + 3 * max_k, np.uint64)
    for B in sizes:
        gu.log(f"[gpu] stats max_k={max_k} B={B}")
        K, A = _rounds(rng, B, max_k)
        st.add(_dev(torch_mod, K), _dev(torch_mod, A))
        oracle.acceptance_counters(K, A, max_k, into=ref)
        got = st.counters.cpu().numpy().astype(np.uint64)
        assert np.array_equal(got, ref), np.nonzero(got != ref)[0][:10]
        s = st.summary().cpu().numpy()
        assert _same_doubles(s, oracle.acceptance_summary(ref, max_k))
    st.reset()
    assert int(st.counters.abs().sum()) == 0


def test_empty_batch_and_fresh_counters(torch_mod):
    import rejection_sampling_verify_06_amd as sv
    st = sv.AcceptanceStats(4, "cuda")
    e = torch_mod.empty(0, dtype=torch_mod.int32, device="cuda")
    st.add(e, e)
    assert int(st.counters.abs().sum()) == 0
    s = st.summary().cpu().numpy()
    assert np.isnan(s).all()


def test_stats_of_a_verify_step(torch_mod):
    """The counters of the verify step's own outputs, on the same stream."""
    import rejection_sampling_verify_06_amd as sv
    b = make_config_batch(3, 0)
    d = gu.batch_to_device(b, torch_mod)
    v = sv.Verifier(max_batch=b.batch, max_k=8, max_vocab=b.vocab, device=0)
    out = v.run(d["target"], d["draft"], d["draft_tokens"], d["num_draft"], d["temperature"], d["mode"],
                d["seq_ids"], seed=b.seed, vocab=b.vocab)
    st = sv.AcceptanceStats(8, "cuda")
    st.add(d["num_draft"], out["accepted_len"])
    s = st.summary()
    acc = out["accepted_len"].cpu().numpy()
    ref = oracle.acceptance_counters(b.num_draft, acc, 8)
    assert np.array_equal(st.counters.cpu().numpy().astype(np.uint64), ref)
    assert _same_doubles(s.cpu().numpy(), oracle.acceptance_summary(ref, 8))
    gu.log(f"      C3 step 0: R={int(ref[0])} D={int(ref[1])} C={int(ref[2])} C/D={s[0].item():.4f} "
           f"mean length={s[1].item():.4f}")
    v.close()


CTRL_CASES = [
    ("window", 0, dict(min_k=1, max_k=10, window=100, min_samples=10, target=0.7), 5),
    ("window small", 0, dict(min_k=2, max_k=6, window=12, min_samples=10, target=0.6), 4),
    ("window 1", 0, dict(min_k=1, max_k=8, window=1, min_samples=1, target=0.5), 3),
    ("window max", 0, dict(min_k=1, max_k=16, window=256, min_samples=3, target=0.8), 8),
    ("multiplicative", 1, dict(min_k=1, max_k=5, target=0.7, rate=0.1), 5),
    ("multiplicative wide", 1, dict(min_k=1, max_k=40, target=0.5, rate=0.35), 12),
    ("optimal-k", 2, dict(min_k=1, max_k=16, target=0.7), 16),
    ("window draft-only", 0, dict(min_k=1, max_k=10, window=100, min_samples=10, target=0.7, count=1), 5),
    ("multiplicative draft-only", 1, dict(min_k=1, max_k=40, target=0.5, rate=0.35, count=1), 12),
    ("optimal-k draft-only", 2, dict(min_k=1, max_k=16, target=0.7, count=1), 16),
]


@pytest.mark.parametrize("name,kind,kw,init_k", CTRL_CASES, ids=[c[0] for c in CTRL_CASES])
def test_controllers_match_oracle(torch_mod, name, kind, kw, init_k):
    import rejection_sampling_verify_06_amd as sv
    rng = np.random.default_rng(sum(map(ord, name)))
    B, steps = 300, 300
    gu.log(f"[gpu] controller {name}: B={B} steps={steps}")
    ctl = sv.DraftLengthController(B, kind, init_k=init_k, device="cuda", **kw)
    states = [oracle.Controller(init_k) for _ in range(B)]
    okw = {k: v for k, v in kw.items()}
    L = np.full(B, init_k, np.int32)
    # each sequence has its own acceptance probability, drifting over time
    beta = rng.random(B)
    for t in range(steps):
        if t % 50 == 0:
            beta = np.clip(beta + rng.normal(0, 0.3, B), 0, 1)
        K = np.minimum(L, 16).astype(np.int32)
        K = np.where(rng.random(B) < 0.03, 0, K).astype(np.int32)
        u = rng.random((B, 16))
        A = np.array([k if (u[j, :k] < beta[j]).all() else int(np.argmin(u[j, :k] < beta[j]))
                      for j, k in enumerate(K)], np.int32)
        A = np.where(rng.random(B) < 0.02, -1, A).astype(np.int32)
        got = ctl.update(_dev(torch_mod, K), _dev(torch_mod, A)).cpu().numpy()
        want = oracle.adapt_batch(states, K, A, kind, **okw)
        assert np.array_equal(got, want), (t, np.nonzero(got != want)[0][:5])
        L = want
    gu.log(f"      lengths after {steps} rounds: min {L.min()} mean {L.mean():.2f} max {L.max()}")


def test_controller_reset_and_small_batches(torch_mod):
    import rejection_sampling_verify_06_amd as sv
    kw = dict(min_k=1, max_k=7, window=12, min_samples=10, target=0.7)
    for B in (1, 3, 5):
        ctl = sv.DraftLengthController(B, 0, init_k=5, device="cuda", **kw)
        states = [oracle.Controller(5) for _ in range(B)]
        K = np.full(B, 4, np.int32)
        for t in range(14):
            got = ctl.update(_dev(torch_mod, K), _dev(torch_mod, K)).cpu().numpy()
            want = oracle.adapt_batch(states, K, K, 0, **kw)
            assert np.array_equal(got, want)
        assert (got == 7).all()
        ctl.reset(3)
        states = [oracle.Controller(3) for _ in range(B)]
        A = np.ones(B, np.int32)
        for t in range(12):
            got = ctl.update(_dev(torch_mod, K), _dev(torch_mod, A)).cpu().numpy()
            want = oracle.adapt_batch(states, K, A, 0, **kw)
            assert np.array_equal(got, want)
        assert (got == 1).all()


def test_bound_calls_match_unbound(torch_mod):
    """bind() queues the same work as add() / update()."""
    import rejection_sampling_verify_06_amd as sv
    rng = np.random.default_rng(77)
    K, A = _rounds(rng, 200, 8, p_bad=0.0)
    Kd, Ad = _dev(torch_mod, K), _dev(torch_mod, A)
    s1, s2 = sv.AcceptanceStats(8, "cuda"), sv.AcceptanceStats(8, "cuda")
    kw = dict(min_k=1, max_k=10, window=20, min_samples=3, target=0.5, init_k=5, device="cuda")
    c1, c2 = sv.DraftLengthController(200, 0, **kw), sv.DraftLengthController(200, 0, **kw)
    add, upd = s2.bind(Kd, Ad), c2.bind(Kd, Ad)
    for _ in range(6):
        s1.add(Kd, Ad)
        a = c1.update(Kd, Ad).clone()
        add()
        upd()
        assert torch_mod.equal(a, c2.next_k)
    assert torch_mod.equal(s1.counters, s2.counters)


def test_bad_arguments_enqueue_nothing(torch_mod):
    import rejection_sampling_verify_06_amd as sv
    with pytest.raises(sv.VerifyError):
        sv.AcceptanceStats(0, "cuda").summary()
    with pytest.raises(sv.VerifyError):
        sv.DraftLengthController(4, 0, window=257, device="cuda")
    with pytest.raises(sv.VerifyError):
        sv.DraftLengthController(4, 1, min_k=3, max_k=2, device="cuda")
    with pytest.raises(sv.VerifyError):
        sv.DraftLengthController(4, 5, device="cuda")
    with pytest.raises(sv.VerifyError):
        sv.DraftLengthController(4, 0, target=1.5, device="cuda")
    with pytest.raises(sv.VerifyError):
        sv.DraftLengthController(4, 0, count=2, device="cuda")


def test_random_controller_parameters(torch_mod):
    """40 seeded random controllers (kind, bounds, window, samples, target,
    rate, batch, initial length) over random rounds, and random counter
    batches: identical to the oracle."""
    import rejection_sampling_verify_06_amd as sv
    for case in range(40):
        rng = np.random.default_rng(600_000 + case)
        kind = int(rng.integers(0, 3))
        max_k = int(rng.integers(1, 65))
        kw = dict(min_k=int(rng.integers(1, max_k + 1)), max_k=max_k, target=float(rng.uniform(0.05, 0.95)),
                  count=int(case % 3 == 2))
        if kind == 0:
            kw.update(window=int(rng.integers(1, 257)), min_samples=int(rng.integers(1, 40)))
        if kind == 1:
            kw.update(rate=float(rng.uniform(0.01, 0.9)))
        B, init_k = int(rng.integers(1, 600)), int(rng.integers(1, 65))
        ctl = sv.DraftLengthController(B, kind, init_k=init_k, device="cuda", **kw)
        states = [oracle.Controller(init_k) for _ in range(B)]
        L = np.full(B, init_k, np.int32)
        beta = rng.random(B)
        for t in range(int(rng.integers(5, 60))):
            K = np.minimum(L, 128).astype(np.int32)
            K = np.where(rng.random(B) < 0.05, rng.integers(0, 130, B), K).astype(np.int32)
            A = np.minimum(rng.geometric(np.clip(1 - beta, 1e-3, 1)) - 1, K).astype(np.int32)
            A = np.where(rng.random(B) < 0.03, -1, A).astype(np.int32)
            got = ctl.update(_dev(torch_mod, K), _dev(torch_mod, A)).cpu().numpy()
            want = oracle.adapt_batch(states, K, A, kind, **kw)
            assert np.array_equal(got, want), (case, t, np.nonzero(got != want)[0][:5])
            L = want
        mk, Bs = int(rng.integers(1, 129)), int(rng.integers(0, 5000))
        K = rng.integers(0, mk + 3, Bs).astype(np.int32)
        A = np.minimum(rng.integers(-1, mk + 1, Bs), K).astype(np.int32)
        st = sv.AcceptanceStats(mk, "cuda")
        st.add(_dev(torch_mod, K), _dev(torch_mod, A))
        ref = oracle.acceptance_counters(K, A, mk)
        assert np.array_equal(st.counters.cpu().numpy().astype(np.uint64), ref), case
        assert _same_doubles(st.summary().cpu().numpy(), oracle.acceptance_summary(ref, mk)), case
