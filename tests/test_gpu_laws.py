"""The distribution laws of the verify step, checked on the HIP path's own
outputs (not through the oracle), over about 10^6 sequences per case:

* losslessness ("Draft Model（草稿模型）", compassingai.com, section 2 接受-拒绝准则
  and 常见误读纠偏 误读 1): the first emitted token follows p_0; given that
  position 0 was accepted, the token at position 1 follows p_1; given that
  all K were accepted, the bonus follows p_K;
* acceptance (same page, 接受率分析): position i is accepted with probability
  beta_i = sum_x min(p_i(x), q_i(x)) when the proposal is drawn from q_i; a
  deterministic (one-hot) or strict sample-match proposal drawn from r_i is
  accepted with probability sum_x r_i(x) p_i(x); all K are accepted with
  probability prod_i beta_i;
* with top-k / top-p, the same laws for the filtered distributions
  (same page, 误读 4).

Each call verifies 4096 sequences that share one set of logit rows and draw
their own proposals; global seq_ids (call * 4096 + s) give every sequence its
own Philox stream.  chi-square at fixed seeds (p-value above 1e-4) and
frequencies within 5 standard deviations, so the tests are deterministic."""
import numpy as np
import pytest
from scipy import stats

from workloads import MODE_ONEHOT, MODE_SAMPLE, MODE_STRICT
from . import gpu_util as gu

pytestmark = pytest.mark.gpu

B = 4096
CALLS = 245          # 1,003,520 sequences per case


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _softmax(x, T):
    z = np.asarray(x, np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


def _filtered(x, T, top_k, top_p):
    """The kept set written from the definitions (a token survives top-k when
    fewer than k logits are strictly larger; then top-p when the mass of the
    strictly larger kept tokens is below p), renormalised."""
    p = _softmax(x, T)
    keep = np.ones(len(x), bool)
    if 0 < top_k < len(x):
        keep &= np.array([(x > x[j]).sum() < top_k for j in range(len(x))])
    if top_p < 1.0:
        pk = np.where(keep, p, 0.0)
        pk = pk / pk.sum()
        keep &= np.array([pk[x > x[j]].sum() < top_p for j in range(len(x))])
    w = np.where(keep, p, 0.0)
    return w / w.sum()


CASES = [
    # name, mode, T, K, V, top_k, top_p
    ("sample T=1", MODE_SAMPLE, 1.0, 3, 6, 0, 1.0),
    ("sample T=0.6", MODE_SAMPLE, 0.6, 3, 8, 0, 1.0),
    ("one-hot", MODE_ONEHOT, 1.0, 3, 6, 0, 1.0),
    ("strict", MODE_STRICT, 0.8, 3, 6, 0, 1.0),
    ("sample top-k 4, top-p 0.9", MODE_SAMPLE, 1.0, 2, 8, 4, 0.9),
]


def _chi2_ok(counts, law, label):
    counts = np.asarray(counts, np.float64)
    n = counts.sum()
    zero = law <= 0
    assert counts[zero].sum() == 0, f"{label}: tokens outside the law's support were emitted"
    exp = law[~zero] * n
    chi = stats.chisquare(counts[~zero], exp)
    gu.log(f"      {label}: n={int(n)} chi2={chi.statistic:.2f} p={chi.pvalue:.4f}")
    assert chi.pvalue > 1e-4, (label, counts, exp)


def _freq_ok(k, n, prob, label):
    sd = np.sqrt(prob * (1 - prob) / n)
    gu.log(f"      {label}: {k / n:.6f} vs {prob:.6f} ({(k / n - prob) / max(sd, 1e-30):+.2f} sd)")
    assert abs(k / n - prob) <= 5 * sd + 1e-12, label


@pytest.mark.parametrize("name,mode,T,K,V,top_k,top_p", CASES, ids=[c[0] for c in CASES])
def test_laws_on_device(torch_mod, name, mode, T, K, V, top_k, top_p):
    import rejection_sampling_verify_06_amd as sv
    torch = torch_mod
    dev = torch.device("cuda", 0)
    rng = np.random.default_rng(sum(map(ord, name)))
    xt = (1.5 * rng.standard_normal((K + 1, V))).astype(np.float32)
    xd = (xt[:K] + rng.standard_normal((K, V))).astype(np.float32)
    p = [_filtered(xt[i], T, top_k, top_p) for i in range(K + 1)]
    if mode == MODE_SAMPLE:
        prop = [_filtered(xd[i], T, top_k, top_p) for i in range(K)]      # proposals from the (filtered) draft
        beta = [float(np.minimum(p[i], prop[i]).sum()) for i in range(K)]
    else:
        prop = [_softmax(xd[i], 1.0) for i in range(K)]                   # any proposal distribution r_i
        beta = [float((prop[i] * p[i]).sum()) for i in range(K)]
    gu.log(f"[gpu] laws {name}: beta={np.round(beta, 4).tolist()}")
    tgt = torch.from_numpy(np.tile(xt, (B, 1))).to(dev)
    dft = torch.from_numpy(np.tile(xd, (B, 1))).to(dev) if mode == MODE_SAMPLE else None
    nd = torch.full((B,), K, dtype=torch.int32, device=dev)
    temp = torch.full((B,), T, dtype=torch.float32, device=dev)
    md = torch.full((B,), mode, dtype=torch.uint8, device=dev)
    tk = torch.full((B,), top_k, dtype=torch.int32, device=dev) if top_k else None
    tp = torch.full((B,), top_p, dtype=torch.float32, device=dev) if top_p < 1.0 else None
    v = sv.Verifier(max_batch=B, max_k=K, max_vocab=V, device=0)
    first = np.zeros(V, np.int64)
    second = np.zeros(V, np.int64)
    bonus = np.zeros(V, np.int64)
    reach = np.zeros(K + 1, np.int64)                 # sequences with A >= j
    n = 0
    try:
        cum = [np.cumsum(r) for r in prop]
        for call in range(CALLS):
            u = rng.random((B, K))
            toks = np.stack([np.minimum(np.searchsorted(cum[i], u[:, i] * cum[i][-1], side="right"), V - 1)
                             for i in range(K)], axis=1).astype(np.int32)
            ids = torch.arange(call * B, (call + 1) * B, dtype=torch.int32, device=dev)
            out = v.run(tgt, dft, torch.from_numpy(toks.reshape(-1)).to(dev), nd, temp, md, ids, seed=12345,
                        vocab=V, want_pq=False, top_k=tk, top_p=tp)
            A = out["accepted_len"].cpu().numpy()
            em = out["emitted"].cpu().numpy().reshape(B, K + 1)
            st = out["status"].cpu().numpy()
            assert (st & 127).sum() == 0 and (A >= 0).all()
            first += np.bincount(em[:, 0], minlength=V)
            second += np.bincount(em[A >= 1, 1], minlength=V)
            bonus += np.bincount(em[A == K, K], minlength=V)
            for j in range(K + 1):
                reach[j] += int((A >= j).sum())
            n += B
    finally:
        v.close()
    _chi2_ok(first, p[0], "first emitted token ~ p_0")
    _chi2_ok(second, p[1], "token at 1 given position 0 accepted ~ p_1")
    _chi2_ok(bonus, p[K], "bonus given all accepted ~ p_K")
    _freq_ok(reach[1], n, beta[0], "P(accept at 0) = beta_0")
    _freq_ok(reach[2], reach[1], beta[1], "P(accept at 1 | reached 1) = beta_1")
    _freq_ok(reach[K], n, float(np.prod(beta)), "P(all K accepted) = prod beta")
