"""Seeded random filtered batches, GPU against the oracle: vocabularies from 7
to 152064 tokens, fp32 and bf16, 1..32 sequences of 0..8 drafts in every
mode, padded rows, masked (-inf) parts of the vocabulary, tie-heavy rows,
temperatures 0.05..4, and per-sequence top-k / top-p values across every
path of the filter (the bounded selection, the bracket search for top-p
alone, the histogram path)."""
import numpy as np
import pytest

from workloads import bf16_round, make_random_batch

from . import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = 150


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _case(i: int):
    rng = np.random.default_rng(900_000 + i)
    V = int(rng.choice([7, 33, 100, 1000, 4096, 8191, 20000, 65536, 152064]))
    dtype = str(rng.choice(["f32", "bf16"]))
    B = int(rng.integers(1, 33))
    b = make_random_batch(910_000 + i, B=B, V=V, kmax=int(rng.integers(0, 9)), dtype=dtype,
                          ld_pad=int(rng.choice([0, 0, 1, 3, 8])), modes=(0, 1, 2, 3),
                          scale=(float(rng.uniform(0.1, 1.0)), float(rng.uniform(1.0, 5.0))),
                          temp=(float(rng.uniform(0.05, 0.5)), float(rng.uniform(0.5, 4.0))))
    if rng.random() < 0.3:                      # a masked part of the vocabulary (column 0 kept)
        neg = bf16_round(np.array([-np.inf], np.float32))[0] if dtype == "bf16" else np.float32(-np.inf)
        m = rng.random((b.target.shape[0], V)) < rng.uniform(0.1, 0.9)
        m[:, 0] = False
        sub = b.target[:, :V]
        sub[m] = neg
    if rng.random() < 0.3 and dtype == "f32":   # a coarse grid: many ties
        b.target[:, :V] = np.round(b.target[:, :V] * 2) / 2
    ks = rng.choice(np.array([0, 1, 2, 5, 20, 50, 200, 1000, 1024, 1025, max(V - 1, 1), V + 5], np.int64), size=B)
    ks = np.where(rng.random(B) < 0.4, 0, ks)  # top-p alone often
    ps = rng.choice(np.array([1.0, 0.999, 0.99, 0.95, 0.9, 0.7, 0.5, 0.2, 0.0, 1e-3], np.float64), size=B)
    b.top_k = ks.astype(np.int32)
    b.top_p = ps.astype(np.float32)
    return b


def test_random_filtered_batches(torch_mod):
    import rejection_sampling_verify_06_amd as sv
    v = sv.Verifier(max_batch=32, max_k=8, max_vocab=152064, device=0)
    try:
        for i in range(CASES):
            gu.check_batch(v, _case(i), torch_mod, label=f"random filtered case {i}")
    finally:
        v.close()
