"""GPU-vs-oracle parity of the strict (sample-match) mode through the C
interface, under the same rule as the other modes: accepted_len and emitted
tokens identical to the oracle except on the near-ties it flags (a uniform
within 1e-5 of a boundary of the proposal's CDF interval, or of the emitted
token's interval), p at proposal within 1e-5, status words equal.

The strict test splits each target row's sum at the proposal inside the row
statistics, so proposals are placed on chunk boundaries (8192 fp32 or 16384
bf16 elements), at the first and last token, on unaligned rows (scalar
path) and on tokens of zero probability."""
import numpy as np
import pytest

from workloads import (MODE_GREEDY, MODE_ONEHOT, MODE_SAMPLE, MODE_STRICT, Batch, bf16_round,
                       make_config_batch, make_random_batch)

from . import gpu_util as gu
from .test_gpu_parity import TINY

pytestmark = pytest.mark.gpu

ALL_MODES = (MODE_SAMPLE, MODE_GREEDY, MODE_ONEHOT, MODE_STRICT)


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def verifier(torch_mod):
    import rejection_sampling_verify_06_amd as sv
    v = sv.Verifier(max_batch=4096, max_k=16, max_vocab=152064, device=0)
    yield v
    v.close()


@pytest.mark.parametrize("seed,B,V,kmax,dtype,ld_pad", TINY)
def test_tiny_all_modes(verifier, torch_mod, seed, B, V, kmax, dtype, ld_pad):
    b = make_random_batch(300 + seed, B=B, V=V, kmax=kmax, dtype=dtype, ld_pad=ld_pad, modes=ALL_MODES)
    gu.check_batch(verifier, b, torch_mod, label=f"all modes seed={seed}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("temp", [(0.3, 0.6), (0.9, 1.6)])
def test_strict_only(verifier, torch_mod, dtype, temp):
    b = make_random_batch(400 + int(temp[0] * 10), B=64, V=20000, kmax=8, dtype=dtype, modes=(MODE_STRICT,),
                          temp=temp, with_draft=False)
    gu.check_batch(verifier, b, torch_mod, label=f"strict T in {temp}")


def _boundary_batch(dtype: str, V: int, ld_pad: int, seed: int, zero_prob: bool = False) -> Batch:
    """Strict sequences whose proposals sit on chunk edges, the first and
    the last token; the proposed token's logit is raised at half of the
    positions so that both outcomes occur.  With ``zero_prob`` some
    proposals have a -inf logit (probability 0)."""
    rng = np.random.default_rng(seed)
    ce = 16384 if dtype == "bf16" else 8192
    edges = sorted({0, 1, ce - 1, ce, ce + 1, 2 * ce - 1, 2 * ce, V - 2, V - 1} & set(range(V)))
    B, K = 24, 6
    rows, toks = [], []
    for s in range(B):
        for i in range(K + 1):
            row = rng.standard_normal(V).astype(np.float32) * 0.7
            if i < K:
                x = int(edges[rng.integers(0, len(edges))])
                toks.append(x)
                if rng.random() < 0.5:
                    row[x] += 12.0                     # most of the mass on the proposal
                if zero_prob and rng.random() < 0.25:
                    row[x] = -np.inf
            rows.append(row)
    tgt = np.stack(rows)
    ld = V + ld_pad
    store = bf16_round(tgt) if dtype == "bf16" else tgt
    pad = np.zeros((tgt.shape[0], ld), store.dtype)
    pad[:, :V] = store
    return Batch(name=f"strict edges V={V} {dtype} ld={ld}", vocab=V, dtype=dtype, target=pad, draft=None,
                 num_draft=np.full(B, K, np.int32), draft_tokens=np.array(toks, np.int32),
                 temperature=np.full(B, 1.0, np.float32), mode=np.full(B, MODE_STRICT, np.uint8),
                 seq_ids=np.arange(B, dtype=np.uint32), seed=seed)


@pytest.mark.parametrize("dtype,V,ld_pad", [("f32", 30000, 0), ("bf16", 50000, 0), ("f32", 20001, 3),
                                            ("bf16", 40000, 1)])
def test_proposals_on_chunk_edges(verifier, torch_mod, dtype, V, ld_pad):
    for seed in (1, 2, 3):
        b = _boundary_batch(dtype, V, ld_pad, seed)
        _, out, _ = gu.check_batch(verifier, b, torch_mod, label=f"edges seed={seed}")
        A = out["accepted_len"]
        assert (A < 6).any() and (A > 0).any()


def test_zero_probability_proposals_never_accepted(verifier, torch_mod):
    b = _boundary_batch("f32", 30000, 0, 7, zero_prob=True)
    _, out, _ = gu.check_batch(verifier, b, torch_mod, label="strict -inf proposals")
    tok = b.draft_tokens.reshape(b.batch, 6)
    rows = b.target[:, :b.vocab].reshape(b.batch, 7, b.vocab)
    for s in range(b.batch):
        A = int(out["accepted_len"][s])
        for i in range(A):
            assert np.isfinite(rows[s, i, tok[s, i]])
        if A < 6:     # the correction is never the rejected proposal
            assert out["emitted"][s * 7 + A] != tok[s, A]


def test_c3_strict_bench_context(torch_mod):
    """The C3 batches in strict mode (no draft logits) through a context
    sized the way bench.py sizes it."""
    import rejection_sampling_verify_06_amd as sv
    v = sv.Verifier(max_batch=256, max_k=8, max_vocab=152064, device=0)
    try:
        for step in (0, 1):
            b = make_config_batch(3, step, strict=True)
            _, out, _ = gu.check_batch(v, b, torch_mod, label=f"C3 strict step {step}, bench context")
            gu.log(f"      accepted {int(out['accepted_len'].sum())} of {int(b.num_draft.sum())} proposals")
    finally:
        v.close()


def test_small_batch_split_final(torch_mod):
    """A batch below 128 (split final kernel + select) in strict mode, fp32
    rows of 13 chunks (two scan lanes per slot)."""
    import rejection_sampling_verify_06_amd as sv
    v = sv.Verifier(max_batch=64, max_k=8, max_vocab=100000, device=0)
    try:
        b = make_random_batch(55, B=24, V=100000, kmax=8, dtype="f32", modes=(MODE_STRICT, MODE_SAMPLE))
        gu.check_batch(v, b, torch_mod, label="strict + sample, V 100000 f32")
    finally:
        v.close()
