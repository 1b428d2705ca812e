"""GPU-vs-oracle parity of the verify step through the C interface.

accepted_len and emitted tokens must be identical to the oracle except on
near-ties the oracle flags (a uniform within 1e-5 of an acceptance ratio or
a CDF boundary); p/q at proposal within 1e-5 absolute; status words equal."""
import numpy as np
import pytest

from workloads import (MODE_GREEDY, MODE_ONEHOT, MODE_SAMPLE, MODE_STRICT, Batch, bf16_widen,
                       make_config_batch, make_random_batch)
from . import gpu_util as gu

pytestmark = pytest.mark.gpu

MAX_K = 16


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def verifier(torch_mod):
    import rejection_sampling_verify_06_amd as sv
    v = sv.Verifier(max_batch=4096, max_k=MAX_K, max_vocab=152064, device=0)
    yield v
    v.close()


# ---------------------------------------------------------------------------
# small mixed batches: several tiles, ragged tails, odd ld, every mode
# ---------------------------------------------------------------------------

TINY = [
    # seed, B, V, kmax, dtype, ld_pad
    (0, 8, 2, 4, "f32", 0),
    (1, 8, 3, 3, "bf16", 0),
    (2, 16, 7, 8, "f32", 1),
    (3, 16, 64, 8, "bf16", 8),
    (4, 32, 1000, 6, "f32", 0),
    (5, 32, 1000, 6, "bf16", 3),
    (6, 12, 8193, 5, "f32", 0),        # one element past a tile
    (7, 12, 8193, 5, "bf16", 0),
    (8, 10, 16385, 4, "bf16", 16),     # one element past a bf16 chunk
    (9, 10, 20000, 8, "f32", 5),       # unaligned rows: scalar path
    (10, 40, 33000, 3, "bf16", 0),
    (11, 6, 65536, 2, "f32", 0),
    (12, 64, 500, 16, "bf16", 0),      # K up to max_k
    (13, 200, 300, 8, "f32", 4),
    (14, 3, 1, 3, "f32", 0),           # a one-token vocabulary
    (15, 6, 150000, 4, "f32", 0),      # 19 chunks per row: the scan merges in groups
]


@pytest.mark.parametrize("seed,B,V,kmax,dtype,ld_pad", TINY)
def test_tiny_mixed(verifier, torch_mod, seed, B, V, kmax, dtype, ld_pad):
    b = make_random_batch(seed, B=B, V=V, kmax=kmax, dtype=dtype, ld_pad=ld_pad)
    gu.check_batch(verifier, b, torch_mod, label=f"tiny seed={seed}")


@pytest.mark.parametrize("mode", [MODE_SAMPLE, MODE_GREEDY, MODE_ONEHOT, MODE_STRICT])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_mode(verifier, torch_mod, mode, dtype):
    b = make_random_batch(100 + mode, B=48, V=5000, kmax=8, dtype=dtype, modes=(mode,))
    gu.check_batch(verifier, b, torch_mod, label=f"mode={mode}")


def test_k_zero_and_empty_draft(verifier, torch_mod):
    b = make_random_batch(21, B=20, V=900, kmax=0, dtype="f32", modes=(MODE_SAMPLE, MODE_ONEHOT, MODE_GREEDY))
    assert b.total_draft == 0
    gu.check_batch(verifier, b, torch_mod, label="K=0")


def test_identical_draft_accepts_all(verifier, torch_mod):
    b = make_random_batch(22, B=30, V=4000, kmax=8, dtype="bf16", modes=(MODE_SAMPLE,), identical_draft=True)
    _, out, _ = gu.check_batch(verifier, b, torch_mod, label="identical draft")
    assert (out["accepted_len"] == b.num_draft).all()


def test_unaligned_base_pointer(verifier, torch_mod):
    b = make_random_batch(23, B=16, V=4096, kmax=5, dtype="f32")
    d = gu.batch_to_device(b, torch_mod, offset_elems=1)
    assert d["target"].data_ptr() % 16 != 0
    out = gu.run_gpu(verifier, b, torch_mod, d=d)
    rep = gu.compare(gu.oracle_for(b, MAX_K), out)
    gu.log(f"[gpu] unaligned base: {rep.summary()}")
    gu.assert_parity(rep)


@pytest.mark.parametrize("tdtype,ddtype", [("bf16", "f32"), ("f32", "bf16")])
def test_mixed_target_draft_dtypes(verifier, torch_mod, tdtype, ddtype):
    b = make_random_batch(24, B=20, V=3000, kmax=6, dtype=tdtype, modes=(MODE_SAMPLE,))
    if tdtype == "f32":
        # make the f32 draft exactly representable in bf16 so both sides see the same values
        from workloads import bf16_round
        b.draft = bf16_widen(bf16_round(b.draft))
    d = gu.batch_to_device(b, torch_mod, draft_as=ddtype)
    out = gu.run_gpu(verifier, b, torch_mod, d=d)
    tgt = bf16_widen(b.target) if tdtype == "bf16" else b.target
    dft = b.draft if tdtype == "f32" else bf16_widen(b.draft)
    ref = gu.oracle.verify_batch(target=tgt, draft=dft, dtype="f32", vocab=b.vocab, num_draft=b.num_draft,
                                 draft_tokens=b.draft_tokens, temperature=b.temperature, mode=b.mode,
                                 seq_ids=b.seq_ids, seed=b.seed, max_k=MAX_K)
    rep = gu.compare(ref, out)
    gu.log(f"[gpu] mixed dtypes {tdtype}/{ddtype}: {rep.summary()}")
    gu.assert_parity(rep)


# ---------------------------------------------------------------------------
# invalid inputs -> status bits, cleared outputs
# ---------------------------------------------------------------------------

def _poke(b: Batch, row: int, col, value, draft=False):
    arr = b.draft if draft else b.target
    if b.dtype == "bf16":
        from workloads import bf16_round
        arr[row, col] = bf16_round(np.array([value], np.float32))[0]
    else:
        arr[row, col] = value


def test_status_cases(verifier, torch_mod):
    b = make_random_batch(30, B=12, V=300, kmax=4, k_min=2, dtype="bf16",
                          modes=(MODE_SAMPLE,), ld_pad=0)
    off_d = np.concatenate(([0], np.cumsum(b.num_draft)[:-1]))
    off_t = off_d + np.arange(b.batch)
    b.draft_tokens[off_d[0]] = b.vocab            # bad token
    b.mode[1] = 9                                 # bad mode
    b.temperature[2] = 0.0                        # bad temperature
    b.temperature[3] = np.float32(5e-7)           # below the minimum
    _poke(b, off_t[4] + 1, 7, np.nan)             # NaN in a target row
    _poke(b, off_t[5] + int(b.num_draft[5]), 3, np.inf)   # +inf in the bonus row
    _poke(b, off_t[6], slice(None), -np.inf)      # all -inf row
    _poke(b, off_t[7], slice(0, 200), -np.inf)    # partly -inf: fine
    _poke(b, off_d[8], 5, np.nan, draft=True)     # NaN in a draft row
    b.mode[9] = MODE_GREEDY
    b.temperature[9] = 0.0                        # greedy ignores T
    b.mode[10] = MODE_ONEHOT
    _poke(b, off_d[10], 5, np.nan, draft=True)    # one-hot does not read draft rows
    rep, out, ref = gu.check_batch(verifier, b, torch_mod, label="status cases")
    st = out["status"]
    assert st[0] == 32 and st[1] == 4 and st[2] == 8 and st[3] == 8
    assert st[4] == 64 and st[5] == 64 and st[6] == 64 and st[7] == 0 and st[8] == 64
    assert st[9] == 0 and st[10] == 0
    assert (out["accepted_len"][:7] == -1).all()


def test_k_too_large(verifier, torch_mod):
    b = make_random_batch(31, B=4, V=100, kmax=MAX_K + 2, k_min=MAX_K + 1, dtype="f32")
    rep, out, _ = gu.check_batch(verifier, b, torch_mod, label="K > max_k")
    assert (out["status"] & 2).all() and (out["accepted_len"] == -1).all()


def test_sample_without_draft_logits(verifier, torch_mod):
    b = make_random_batch(32, B=10, V=200, kmax=3, dtype="f32", modes=(MODE_SAMPLE, MODE_GREEDY), with_draft=False)
    rep, out, _ = gu.check_batch(verifier, b, torch_mod, label="no draft logits")
    assert ((out["status"] == 16) == ((b.mode == MODE_SAMPLE) & (b.num_draft > 0))).all()


@pytest.mark.parametrize("nd,filtered", [([2, 3], False), ([-1, 5], False), ([2, 3], True), ([-1, 5], True),
                                         ([8, 8], True)])
def test_bad_layout(verifier, torch_mod, nd, filtered):
    """num_draft that does not add up to total_draft: every output cleared,
    status SV_ST_BAD_LAYOUT.  With filters, the filter's row list that row
    statistics writes is clamped to the n_t + n_d rows the call has (K = 8
    and 8 against total_draft 4 asks for 34 rows of 10)."""
    b = make_random_batch(33, B=2, V=50, kmax=2, k_min=2, dtype="f32")
    assert b.total_draft == 4
    b.num_draft = np.array(nd, np.int32)
    if filtered:
        b.top_k = np.array([5, 0], np.int32)
        b.top_p = np.array([0.9, 0.8], np.float32)
    out = gu.run_gpu(verifier, b, torch_mod, total_draft=4)
    ref = gu.oracle_for(b, MAX_K, total_draft=4)
    assert not ref.layout_ok
    rep = gu.compare(ref, out)
    gu.assert_parity(rep)


# ---------------------------------------------------------------------------
# determinism, split-batch invariance, graph replay
# ---------------------------------------------------------------------------

def test_repeatable_bitwise(verifier, torch_mod):
    b = make_random_batch(40, B=64, V=20000, kmax=8, dtype="bf16")
    d = gu.batch_to_device(b, torch_mod)
    o1 = gu.run_gpu(verifier, b, torch_mod, d=d)
    o2 = gu.run_gpu(verifier, b, torch_mod, d=d)
    for k in o1:
        if o1[k] is not None:
            assert np.array_equal(o1[k].view(np.uint32) if o1[k].dtype == np.float32 else o1[k],
                                  o2[k].view(np.uint32) if o2[k].dtype == np.float32 else o2[k]), k


def test_split_batch_matches_one_call(verifier, torch_mod):
    """A batch split across two calls (global seq_ids) gives identical outputs:
    the sequence-sharded multi-device layout needs nothing else."""
    b = make_random_batch(41, B=40, V=9000, kmax=6, dtype="f32")
    full = gu.run_gpu(verifier, b, torch_mod)
    cut = 17
    K = b.num_draft
    td = int(K[:cut].sum())
    parts = []
    for lo, hi in ((0, cut), (cut, b.batch)):
        d0 = int(K[:lo].sum())
        d1 = int(K[:hi].sum())
        sub = Batch(name="half", vocab=b.vocab, dtype=b.dtype, target=b.target[d0 + lo:d1 + hi],
                    draft=b.draft[d0:d1] if b.draft is not None else None, num_draft=K[lo:hi].copy(),
                    draft_tokens=b.draft_tokens[d0:d1].copy(), temperature=b.temperature[lo:hi].copy(),
                    mode=b.mode[lo:hi].copy(), seq_ids=b.seq_ids[lo:hi].copy(), seed=b.seed)
        parts.append(gu.run_gpu(verifier, sub, torch_mod))
    assert np.array_equal(np.concatenate([p["accepted_len"] for p in parts]), full["accepted_len"])
    assert np.array_equal(np.concatenate([p["emitted"] for p in parts]), full["emitted"])
    assert np.array_equal(np.concatenate([p["p_at"] for p in parts]).view(np.uint32), full["p_at"].view(np.uint32))
    assert td == len(parts[0]["p_at"])


def test_graph_replay_matches_eager(verifier, torch_mod):
    torch = torch_mod
    b = make_random_batch(42, B=32, V=12000, kmax=6, dtype="bf16")
    other = make_random_batch(43, B=20, V=12000, kmax=5, dtype="f32")
    d = gu.batch_to_device(b, torch)
    eager = gu.run_gpu(verifier, b, torch, d=d)
    out = verifier.make_outputs(b.batch, b.total_draft)
    args = verifier.build_args(d["target"], d["draft"], d["draft_tokens"], d["num_draft"], d["temperature"],
                               d["mode"], d["seq_ids"], b.seed, out, b.vocab)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        verifier.run_args(args)        # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        verifier.run_args(args)
    for rep_i in range(3):
        for v in out.values():
            if v is not None:
                v.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            if v is not None:
                got = v.cpu().numpy()
                want = eager[k]
                if got.dtype == np.float32:
                    got, want = got.view(np.uint32), want.view(np.uint32)
                assert np.array_equal(got, want), (rep_i, k)
        gu.run_gpu(verifier, other, torch)        # eager work on the same context between replays


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,steps", [(0, 200), (1, 20), (2, 2), (3, 2), (4, 2)])
def test_workload_parity(verifier, torch_mod, cfg, steps):
    tot = None
    for step in range(steps):
        b = make_config_batch(cfg, step)
        rep, _, _ = gu.check_batch(verifier, b, torch_mod, label=f"C{cfg} step {step}") if steps <= 20 or step % 50 == 0 \
            else _quiet(verifier, b, torch_mod)
        tot = gu.add_reports(tot, rep)
    gu.log(f"[gpu] C{cfg} x{steps}: {tot.summary()}")
    gu.assert_parity(tot)


def _quiet(verifier, b, torch_mod):
    out = gu.run_gpu(verifier, b, torch_mod)
    rep = gu.compare(gu.oracle_for(b, verifier.max_k), out)
    gu.assert_parity(rep)
    return rep, out, None


def test_small_max_k_mixed(torch_mod):
    """max_k = 8, fp32 rows of 13 chunks (two scan lanes per slot), a batch
    below 128 (split final kernel + select) with every mode."""
    import rejection_sampling_verify_06_amd as sv
    v = sv.Verifier(max_batch=64, max_k=8, max_vocab=100000, device=0)
    try:
        for seed in (50, 51):
            b = make_random_batch(seed, B=24, V=100000, kmax=8, dtype="f32")
            gu.check_batch(v, b, torch_mod, label=f"max_k 8, V 100000 f32, seed {seed}")
    finally:
        v.close()


def test_workload_c4_interleaved(verifier, torch_mod):
    b = make_config_batch(4, 7, interleave_modes=True)
    gu.check_batch(verifier, b, torch_mod, label="C4 interleaved")


def test_workload_padded_rows(verifier, torch_mod):
    b = make_config_batch(1, 3, ld_pad=64)
    gu.check_batch(verifier, b, torch_mod, label="C1 ld=V+64")
