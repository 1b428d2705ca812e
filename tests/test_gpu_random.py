"""Seeded random unfiltered batches, GPU against the oracle, over wide
shapes: vocabularies of 1 to 300000 tokens, fp32 and bf16, up to 1024
sequences of up to 64 drafts, every mode, padded rows, batches without draft
logits, identical drafts, temperatures 0.05..3."""
import numpy as np
import pytest

from workloads import make_random_batch

from . import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = 60


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _case(i: int):
    rng = np.random.default_rng(800_000 + i)
    V = int(rng.choice([1, 2, 3, 9, 64, 777, 8192, 8193, 32000, 128256, 152064, 300000]))
    dtype = str(rng.choice(["f32", "bf16"]))
    small = V <= 8193
    B = int(rng.integers(1, 1025 if small else 33))
    kmax = int(rng.choice([0, 1, 5, 8, 16, 64])) if small else int(rng.integers(0, 9))
    with_draft = None if rng.random() < 0.8 else False
    return make_random_batch(810_000 + i, B=B, V=V, kmax=kmax, dtype=dtype, ld_pad=int(rng.choice([0, 0, 1, 5])),
                             modes=(0, 1, 2, 3) if with_draft is None else (1, 2, 3), with_draft=with_draft,
                             scale=(0.1, float(rng.uniform(1.0, 6.0))),
                             temp=(float(rng.uniform(0.05, 0.6)), float(rng.uniform(0.6, 3.0))),
                             p_hit=float(rng.uniform(0.3, 0.99)), identical_draft=bool(rng.random() < 0.1))


def test_random_batches(torch_mod):
    import rejection_sampling_verify_06_amd as sv
    v = sv.Verifier(max_batch=1024, max_k=64, max_vocab=300000, device=0)
    try:
        for i in range(CASES):
            gu.check_batch(v, _case(i), torch_mod, label=f"random case {i}")
    finally:
        v.close()
