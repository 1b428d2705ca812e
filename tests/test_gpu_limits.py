"""GPU-vs-oracle parity at the library's size limits: K_s up to max_k = 128
(257 slots per sequence: the scan merges slots in a loop), a batch of 4096
sequences (the row statistics look owners up over the whole batch), and a
vocabulary of 2,097,152 tokens (256 chunks of fp32, 256 final-draw tiles)."""
import pytest

from workloads import (MODE_GREEDY, MODE_ONEHOT, MODE_SAMPLE, MODE_STRICT, make_random_batch)

from . import gpu_util as gu

pytestmark = pytest.mark.gpu

ALL_MODES = (MODE_SAMPLE, MODE_GREEDY, MODE_ONEHOT, MODE_STRICT)


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def test_max_k_128(torch_mod):
    import rejection_sampling_verify_06_amd as sv
    v = sv.Verifier(max_batch=16, max_k=128, max_vocab=5000, device=0)
    try:
        # every sequence at K = 128 with a draft close to the target (long accepted runs), then K mixed in 0..128
        for seed, dtype, k_min, noise in ((1, "f32", 128, (0.0, 0.05)), (2, "bf16", 0, (0.0, 0.3))):
            b = make_random_batch(700 + seed, B=8, V=300, kmax=128, k_min=k_min, dtype=dtype, modes=ALL_MODES,
                                  p_hit=0.97, temp=(0.2, 0.4), noise=noise)
            _, out, _ = gu.check_batch(v, b, torch_mod, label=f"max_k 128 {dtype}")
            gu.log(f"      K {b.num_draft.tolist()} accepted {out['accepted_len'].tolist()}")
    finally:
        v.close()


def test_batch_4096(torch_mod):
    import rejection_sampling_verify_06_amd as sv
    v = sv.Verifier(max_batch=4096, max_k=4, max_vocab=1000, device=0)
    try:
        b = make_random_batch(710, B=4096, V=64, kmax=3, dtype="bf16", modes=ALL_MODES)
        gu.check_batch(v, b, torch_mod, label="B 4096")
        b = make_random_batch(711, B=4093, V=200, kmax=4, dtype="f32", modes=ALL_MODES, ld_pad=3)
        gu.check_batch(v, b, torch_mod, label="B 4093, unaligned rows")
    finally:
        v.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_max_vocab(torch_mod, dtype):
    import rejection_sampling_verify_06_amd as sv
    V = 2097152
    v = sv.Verifier(max_batch=4, max_k=2, max_vocab=V, device=0)
    try:
        b = make_random_batch(720 + (dtype == "bf16"), B=3, V=V, kmax=2, k_min=1, dtype=dtype, modes=ALL_MODES[:3])
        gu.check_batch(v, b, torch_mod, label=f"V {V} {dtype}")
        b.mode[:] = MODE_STRICT
        b.draft = None
        gu.check_batch(v, b, torch_mod, label=f"V {V} {dtype} strict")
    finally:
        v.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_max_vocab_filtered(torch_mod, dtype):
    """Top-k / top-p at a 2,097,152-token vocabulary: the bounded selection
    (top-k 50 with top-p, top-k 1000), top-p alone on a peaked row and on a
    flat one (the histogram path: its nucleus spans most of the row)."""
    import numpy as np
    import rejection_sampling_verify_06_amd as sv
    V = 2097152
    v = sv.Verifier(max_batch=4, max_k=2, max_vocab=V, device=0)
    try:
        b = make_random_batch(730 + (dtype == "bf16"), B=4, V=V, kmax=2, k_min=1, dtype=dtype,
                              modes=(MODE_SAMPLE, MODE_ONEHOT, MODE_STRICT), scale=(0.3, 4.0))
        b.top_k = np.array([50, 1000, 0, 0], np.int32)
        b.top_p = np.array([0.9, 1.0, 0.95, 0.5], np.float32)
        b.temperature = np.array([1.0, 0.7, 0.3, 2.0], np.float32)
        gu.check_batch(v, b, torch_mod, label=f"V {V} {dtype} filtered")
    finally:
        v.close()


def _random_filters(seed, B, V):
    import numpy as np
    rng = np.random.default_rng(np.random.PCG64([79, seed]))
    top_k = rng.choice(np.array([0, 1, 3, 10, 40, V], np.int32), size=B).astype(np.int32)
    top_p = rng.choice(np.array([1.0, 0.3, 0.9, 0.99], np.float32), size=B).astype(np.float32)
    return top_k, top_p


def test_max_k_128_filtered(torch_mod):
    """Filtered rows at K up to 128: a SAMPLE sequence lists 257 rows (target
    rows 0..K, then its draft rows) for the filter kernel."""
    import rejection_sampling_verify_06_amd as sv
    v = sv.Verifier(max_batch=16, max_k=128, max_vocab=5000, device=0)
    try:
        for seed, dtype, k_min in ((3, "bf16", 128), (4, "f32", 0)):
            b = make_random_batch(740 + seed, B=8, V=300, kmax=128, k_min=k_min, dtype=dtype, modes=ALL_MODES,
                                  p_hit=0.97, temp=(0.2, 0.4), noise=(0.0, 0.3))
            b.top_k, b.top_p = _random_filters(seed, b.batch, b.vocab)
            _, out, _ = gu.check_batch(v, b, torch_mod, label=f"max_k 128 {dtype} filtered")
            gu.log(f"      K {b.num_draft.tolist()} accepted {out['accepted_len'].tolist()}")
    finally:
        v.close()


def test_batch_4096_filtered(torch_mod):
    """Filtered rows of 4096 sequences: the list of the filter's rows is
    built over the whole batch (16 sequences a thread of the order block)."""
    import rejection_sampling_verify_06_amd as sv
    v = sv.Verifier(max_batch=4096, max_k=4, max_vocab=1000, device=0)
    try:
        b = make_random_batch(750, B=4096, V=64, kmax=3, dtype="bf16", modes=ALL_MODES)
        b.top_k, b.top_p = _random_filters(5, b.batch, b.vocab)
        gu.check_batch(v, b, torch_mod, label="B 4096 filtered")
        b = make_random_batch(751, B=4093, V=200, kmax=4, dtype="f32", modes=ALL_MODES, ld_pad=3)
        b.top_k, b.top_p = _random_filters(6, b.batch, b.vocab)
        gu.check_batch(v, b, torch_mod, label="B 4093 filtered, unaligned rows")
    finally:
        v.close()
