"""The host contract of the verify call, through the C interface on the GPU:
every host-checkable fault returns its code with nothing enqueued (outputs
filled with sentinels stay untouched), the optional outputs may be NULL, the
one-shot ``verify`` binding holds one reusable context per device and
passes the filters through, and a call whose row-statistics grid exceeds
65535 blocks (laid out in two grid dimensions) still matches the oracle."""
import ctypes

import numpy as np
import pytest

from workloads import MODE_GREEDY, MODE_ONEHOT, MODE_SAMPLE, MODE_STRICT, make_random_batch
from . import gpu_util as gu

pytestmark = pytest.mark.gpu

ALL_MODES = (MODE_SAMPLE, MODE_GREEDY, MODE_ONEHOT, MODE_STRICT)


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def small(torch_mod):
    import rejection_sampling_verify_06_amd as sv
    v = sv.Verifier(max_batch=16, max_k=6, max_vocab=4000, device=0)
    yield v
    v.close()


def _sentinel_outputs(v, B, T, torch):
    out = v.make_outputs(B, T)
    for t in out.values():
        t.fill_(-7)
    return out


def _untouched(out, torch):
    torch.cuda.synchronize()
    return all(bool((t == -7).all()) for t in out.values() if t is not None)


def _faults(a, lib, _lib, d):
    """(name, change to the packed arguments, expected code) for every check the
    host can make; each change is undone before the next."""
    bad_ptr = ctypes.c_void_p(a.target_logits + 1).value      # not aligned to the element size
    return [
        ("batch < 0", dict(batch=-1), _lib.SV_ERR_INVALID),
        ("vocab 0", dict(vocab=0), _lib.SV_ERR_INVALID),
        ("vocab 2^31", dict(vocab=1 << 31), _lib.SV_ERR_INVALID),
        ("total_draft < 0", dict(total_draft=-1), _lib.SV_ERR_INVALID),
        ("target dtype", dict(target_dtype=7), _lib.SV_ERR_INVALID),
        ("draft dtype", dict(draft_dtype=2), _lib.SV_ERR_INVALID),
        ("no target", dict(target_logits=None), _lib.SV_ERR_INVALID),
        ("no num_draft", dict(num_draft=None), _lib.SV_ERR_INVALID),
        ("no accepted_len", dict(accepted_len=None), _lib.SV_ERR_INVALID),
        ("no emitted", dict(emitted_tokens=None), _lib.SV_ERR_INVALID),
        ("no draft_tokens", dict(draft_tokens=None), _lib.SV_ERR_INVALID),
        ("misaligned target", dict(target_logits=bad_ptr), _lib.SV_ERR_INVALID),
        ("ld_target < vocab", dict(ld_target=a.vocab - 1), _lib.SV_ERR_INVALID),
        ("ld_draft < vocab", dict(ld_draft=a.vocab - 1), _lib.SV_ERR_INVALID),
        ("batch > max_batch", dict(batch=17), _lib.SV_ERR_CAPACITY),
        ("vocab > max_vocab", dict(vocab=4001, ld_target=4001, ld_draft=4001), _lib.SV_ERR_CAPACITY),
        ("total_draft > max_batch * max_k", dict(total_draft=16 * 6 + 1), _lib.SV_ERR_CAPACITY),
    ]


def test_host_faults_enqueue_nothing(torch_mod, small):
    """Each host-checkable fault of spec_verify_run returns its code, sets the
    last error and leaves every output as it was."""
    import rejection_sampling_verify_06_amd as sv
    from rejection_sampling_verify_06_amd import _lib
    lib = _lib.load()
    b = make_random_batch(900, B=12, V=3000, kmax=6, dtype="f32", modes=ALL_MODES)
    d = gu.batch_to_device(b, torch_mod, 0)
    out = _sentinel_outputs(small, b.batch, b.total_draft, torch_mod)
    a = small.build_args(d["target"], d["draft"], d["draft_tokens"], d["num_draft"], d["temperature"], d["mode"],
                         d["seq_ids"], seed=b.seed, out=out, vocab=b.vocab)
    stream = ctypes.c_void_p(torch_mod.cuda.current_stream().cuda_stream)
    for name, change, code in _faults(a, lib, _lib, d):
        saved = {k: getattr(a, k) for k in change}
        for k, val in change.items():
            setattr(a, k, val)
        rc = lib.spec_verify_run(small._h, ctypes.byref(a), stream)
        msg = lib.spec_verify_last_error().decode()
        for k, val in saved.items():
            setattr(a, k, val)
        gu.log(f"[gpu] fault {name}: rc={rc} '{msg}'")
        assert rc == code, (name, rc, msg)
        assert msg, name
        assert _untouched(out, torch_mod), name
    # batch 0 is a no-op that succeeds
    a.batch = 0
    assert lib.spec_verify_run(small._h, ctypes.byref(a), stream) == _lib.SV_OK
    assert _untouched(out, torch_mod)
    a.batch = b.batch
    # the same arguments, all in order, run and match the oracle
    assert lib.spec_verify_run(small._h, ctypes.byref(a), stream) == _lib.SV_OK
    torch_mod.cuda.synchronize()
    got = {k: (None if t is None else t.cpu().numpy()) for k, t in out.items()}
    gu.assert_parity(gu.compare(gu.oracle_for(b, small.max_k), got))
    with pytest.raises(sv.VerifyError) as e:
        small.run(d["target"], d["draft"], d["draft_tokens"], d["num_draft"], d["temperature"], d["mode"],
                  d["seq_ids"], vocab=4001)
    assert e.value.code in (_lib.SV_ERR_INVALID, _lib.SV_ERR_CAPACITY)


def test_create_errors_on_device(torch_mod):
    from rejection_sampling_verify_06_amd import _lib
    lib = _lib.load()
    h = ctypes.c_void_p()
    ndev = torch_mod.cuda.device_count()
    for dev in (-1, ndev):
        assert lib.spec_verify_create(ctypes.byref(h), dev, 4, 4, 100) == _lib.SV_ERR_INVALID
        assert h.value is None
    assert lib.spec_verify_create(ctypes.byref(h), 0, 4, 4, 100) == _lib.SV_OK
    assert h.value
    lib.spec_verify_destroy(h)
    lib.spec_verify_destroy(None)


@pytest.mark.parametrize("want_pq,want_status", [(False, True), (True, False), (False, False)])
def test_optional_outputs_null(torch_mod, small, want_pq, want_status):
    """p/q at proposal and status may be NULL: the other outputs are unchanged."""
    for seed in (910, 911):
        b = make_random_batch(seed, B=16, V=3500, kmax=6, dtype="bf16", modes=ALL_MODES)
        out = gu.run_gpu(small, b, torch_mod, want_pq=want_pq, want_status=want_status)
        assert (out["p_at"] is None) != want_pq and (out["status"] is None) != want_status
        rep = gu.compare(gu.oracle_for(b, small.max_k), out)
        gu.log(f"[gpu] NULL outputs pq={want_pq} status={want_status} seed {seed}: {rep.summary()}")
        gu.assert_parity(rep)


def test_one_shot_verify_mixed_batches(torch_mod):
    """verify(): mixed modes, with and without filters, batch sizes that grow
    and shrink; one context per device, grown only when a call needs more."""
    import rejection_sampling_verify_06_amd as sv
    sv._SHARED.clear()
    sizes = [(5, 1200, 4), (16, 1200, 6), (3, 900, 2), (40, 2500, 8), (7, 2500, 3)]
    caps = []
    for i, (B, V, kmax) in enumerate(sizes):
        b = make_random_batch(920 + i, B=B, V=V, kmax=kmax, dtype="bf16" if i % 2 else "f32", modes=ALL_MODES)
        if i >= 3:
            rng = np.random.default_rng(i)
            b.top_k = rng.choice([0, 1, 5, 40], B).astype(np.int32)
            b.top_p = rng.choice([1.0, 0.9, 0.5], B).astype(np.float32)
        d = gu.batch_to_device(b, torch_mod, 0)
        o = sv.verify(d["target"], d["draft"], d["draft_tokens"], d["num_draft"], d["temperature"], d["mode"],
                      seed=b.seed, want_pq=bool(i % 2), seq_ids=d["seq_ids"], top_k=d["top_k"], top_p=d["top_p"])
        torch_mod.cuda.synchronize()
        got = {k: (None if t is None else t.cpu().numpy()) for k, t in o.items()}
        assert (got["p_at"] is None) == (i % 2 == 0)
        v = sv._SHARED[0]
        caps.append((v.max_batch, v.max_k, v.max_vocab))
        rep = gu.compare(gu.oracle_for(b, v.max_k), got)
        gu.log(f"[gpu] verify() {b.name} context {caps[-1]}: {rep.summary()}")
        gu.assert_parity(rep)
    assert len(sv._SHARED) == 1
    assert all(caps[i + 1][j] >= caps[i][j] for i in range(len(caps) - 1) for j in range(3))
    assert caps[2] == caps[1] and caps[4] == caps[3]          # smaller calls reuse the context


def test_row_stats_grid_in_two_dimensions(torch_mod):
    """1024 sequences with K = 32 over a one-chunk vocabulary: 66,560 row
    blocks, more than one grid dimension holds."""
    import rejection_sampling_verify_06_amd as sv
    b = make_random_batch(930, B=1024, V=600, kmax=32, k_min=32, dtype="bf16", modes=ALL_MODES)
    assert b.total_draft + b.batch + b.total_draft * (b.draft is not None) > 65535
    v = sv.Verifier(max_batch=1024, max_k=32, max_vocab=600, device=0)
    try:
        gu.check_batch(v, b, torch_mod, label="2-D row-statistics grid")
    finally:
        v.close()
