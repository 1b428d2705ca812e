"""CPU pins of the oracle (no GPU), plus planted-mistake tests that show each
pin catches a plausible error in the oracle."""
import numpy as np
import pytest
from scipy import special

import oracle
from oracle import verify as ov

from . import oracle_pins as pins


def test_softmax_matches_scipy():
    rng = np.random.default_rng(0)
    for T in (1.0, 0.3, 1.7):
        x = rng.standard_normal(1000) * 4
        x[rng.integers(0, 1000, 20)] = -np.inf
        assert np.allclose(ov.softmax(x, T), special.softmax(x / T), rtol=0, atol=1e-12)
    x = np.array([1000.0, 999.0, -1000.0])          # overflow-safe
    assert np.allclose(ov.softmax(x, 1.0), special.softmax(x), atol=1e-15)


def test_bf16_widening_is_exact():
    from workloads import bf16_round
    x = np.array([1.0, -2.5, 3.140625, 1e-3, -0.0, 65280.0], np.float32)
    b = bf16_round(x)
    w = ov.widen(b, "bf16")
    # bfloat16 keeps 8 significant bits: these values are representable or rounded once
    assert w[0] == 1.0 and w[1] == -2.5 and w[2] == 3.140625 and w[5] == 65280.0
    assert abs(w[3] - 1e-3) <= 2 ** -8 * 1e-3
    assert (ov.widen(np.array([0x3F80, 0xC020], np.uint16), "bf16") == [1.0, -2.5]).all()


def test_worked_example():
    pins.check_worked_example()


def test_worked_example_marginal():
    pins.check_marginal_with_q_proposals()


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_lossless_sample_mode(T):
    pins.check_lossless(T=T, mode=ov.SAMPLE)


def test_lossless_onehot_mode():
    pins.check_lossless(T=0.9, mode=ov.ONEHOT, seed=7)


def test_lossless_strict_mode():
    pins.check_lossless(mode=ov.STRICT)


def test_grid_exact_strict():
    pins.check_grid_strict()


def test_strict_acceptance_rate():
    pins.check_strict_acceptance_rate()


def test_strict_wiring():
    pins.check_strict_wiring()


def test_k_zero_is_plain_sampling():
    pins.check_k_zero_is_plain_sampling()


def test_grid_exact_law():
    pins.check_grid_exact(seed=3)
    pins.check_grid_exact(seed=8, V=4, T=0.5)


def test_grid_exact_onehot():
    pins.check_grid_onehot()


def test_acceptance_law_on_gaussian_workload():
    pins.check_acceptance_law_on_workload()


def test_greedy_equivalence():
    pins.check_greedy_equivalence()


def test_identical_draft_always_accepts():
    pins.check_identical_draft_always_accepts()


def test_onehot_certain_token_accepted():
    pins.check_onehot_certain_token_accepted()


def test_uniform_wiring():
    pins.check_uniform_wiring()


def test_final_uniform_wiring():
    pins.check_final_uniform_wiring()


def test_inverse_cdf_convention():
    pins.check_inverse_cdf_convention()


def test_output_length_is_one_to_k_plus_one():
    """[DM] algorithm box: a round emits between 1 and K+1 tokens."""
    from workloads import make_random_batch
    b = make_random_batch(11, B=64, V=30, kmax=8, dtype="f32")
    res = oracle.verify_batch_from(b)
    ot = 0
    for s in range(b.batch):
        K = int(b.num_draft[s])
        n_emit = int((res.emitted[ot:ot + K + 1] >= 0).sum())
        assert n_emit == res.accepted_len[s] + 1 and 1 <= n_emit <= K + 1
        ot += K + 1


# ---------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------

def test_plant_swapped_ratio(monkeypatch):
    real = ov.accept_ratio
    monkeypatch.setattr(ov, "accept_ratio", lambda m, p, q: real(m, q, p) if m == ov.SAMPLE else real(m, p, q))
    with pytest.raises(AssertionError):
        pins.check_worked_example(n=5000)


def test_plant_residual_sign(monkeypatch):
    monkeypatch.setattr(ov, "residual", lambda m, p, q, x: np.maximum(q - p, 0.0) if m == ov.SAMPLE else p)
    with pytest.raises(AssertionError):
        pins.check_worked_example(n=5000)


def test_plant_temperature_on_target_only(monkeypatch):
    orig = ov.verify_sequence

    def vs(xt, xd, tokens, T, *a, **k):
        if xd is not None:
            xd = xd * T        # q then comes out as softmax(draft logits) at T = 1
        return orig(xt, xd, tokens, T, *a, **k)
    monkeypatch.setattr(ov, "verify_sequence", vs)
    with pytest.raises(AssertionError):
        pins.check_lossless(n=6000, T=0.6, mode=ov.SAMPLE)


def test_plant_bonus_from_wrong_row(monkeypatch):
    orig = ov.verify_sequence

    def vs(xt, *a, **k):
        xt = xt.copy()
        xt[-1] = xt[-2]        # bonus drawn from the last draft position's distribution
        return orig(xt, *a, **k)
    monkeypatch.setattr(ov, "verify_sequence", vs)
    with pytest.raises(AssertionError):
        pins.check_lossless(n=8000, T=1.0, mode=ov.SAMPLE)


def test_plant_inverse_cdf_left_side(monkeypatch):
    def bad(w, u):
        C = np.cumsum(w)
        k = np.searchsorted(C, np.asarray(u) * C[-1], side="left")
        return np.minimum(k, int(np.nonzero(w > 0)[0][-1]))
    monkeypatch.setattr(ov, "inverse_cdf", bad)
    with pytest.raises(AssertionError):
        pins.check_inverse_cdf_convention()


def test_plant_uniform_position_offset(monkeypatch):
    import oracle.philox as ph
    real = ph.verify_uniform
    monkeypatch.setattr(ov, "verify_uniform", lambda seed, sid, pos, pur: real(seed, sid, pos + 1, pur))
    with pytest.raises(AssertionError):
        pins.check_uniform_wiring()


def test_plant_onehot_residual_keeps_token(monkeypatch):
    real = ov.residual
    monkeypatch.setattr(ov, "residual", lambda m, p, q, x: p.copy() if m == ov.ONEHOT else real(m, p, q, x))
    with pytest.raises(AssertionError):
        pins.check_grid_onehot()


def test_plant_strict_without_remap(monkeypatch):
    """The correction drawn from p without the proposal at the raw point t
    (tokens above the proposal shift by one)."""
    def bad(p, x, u):
        w = p.copy()
        w[x] = 0.0
        return w, u * float(np.cumsum(p)[-1]) / float(np.cumsum(w)[-1])
    monkeypatch.setattr(ov, "strict_correction", bad)
    with pytest.raises(AssertionError):
        pins.check_grid_strict()


def test_plant_strict_other_uniform(monkeypatch):
    """The correction drawn with another uniform than the position's own."""
    real = ov.strict_emit
    monkeypatch.setattr(ov, "strict_emit", lambda p, x, u: real(p, x, (u + 0.37) % 1.0))
    with pytest.raises(AssertionError):
        pins.check_strict_wiring()


def test_plant_strict_as_onehot_rule(monkeypatch):
    """Strict decisions taken with the one-hot rule u < p(x) (same acceptance
    probability, different uniforms accept)."""
    orig = ov.verify_sequence

    def vs(xt, xd, tokens, T, mode, *a, **k):
        return orig(xt, xd, tokens, T, ov.ONEHOT if mode == ov.STRICT else mode, *a, **k)
    monkeypatch.setattr(ov, "verify_sequence", vs)
    with pytest.raises(AssertionError):
        pins.check_strict_wiring()
