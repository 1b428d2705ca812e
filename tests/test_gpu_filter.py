"""GPU-vs-oracle parity of top-k / top-p filtered verification through the C
interface, under the usual rule (identical outputs except on flagged
near-ties; a top-p crossing within 1e-5 of a tie group may follow the
neighbouring threshold).  Covers every mode with per-sequence filters,
tie-heavy bf16 rows, thresholds on the largest and the smallest logits,
boundary bins larger than the filter's LDS buffer (refined by passes over
the row), filters that are off, the C3 workload with filters, and top-p
alone on flat rows that only the bracket search can decide."""
import numpy as np
import pytest

from workloads import (MODE_GREEDY, MODE_ONEHOT, MODE_SAMPLE, MODE_STRICT, Batch, bf16_round, bf16_widen,
                       make_config_batch, make_random_batch)

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
def verifier(torch_mod):
    import rejection_sampling_verify_06_amd as sv
    v = sv.Verifier(max_batch=4096, max_k=16, max_vocab=152064, device=0)
    yield v
    v.close()


def _with_filters(b: Batch, seed: int, ks, ps) -> Batch:
    rng = np.random.default_rng(seed)
    b.top_k = rng.choice(np.asarray(ks, np.int64), size=b.batch).astype(np.int32)
    b.top_p = rng.choice(np.asarray(ps, np.float64), size=b.batch).astype(np.float32)
    return b


FILTER_CASES = [
    # seed, B, V, kmax, dtype, ld_pad
    (0, 24, 7, 4, "f32", 0),
    (1, 24, 64, 6, "bf16", 0),
    (2, 32, 1000, 6, "f32", 3),       # unaligned rows
    (3, 32, 1000, 6, "bf16", 0),
    (4, 16, 20000, 8, "bf16", 0),
    (5, 12, 40000, 5, "f32", 0),
    (6, 6, 150000, 4, "bf16", 0),
]


@pytest.mark.parametrize("seed,B,V,kmax,dtype,ld_pad", FILTER_CASES)
def test_filtered_mixed(verifier, torch_mod, seed, B, V, kmax, dtype, ld_pad):
    b = make_random_batch(500 + seed, B=B, V=V, kmax=kmax, dtype=dtype, ld_pad=ld_pad, modes=ALL_MODES)
    ks = [0, 1, 2, 5, 50, V - 1, V, V + 3]
    ps = [1.0, 0.95, 0.9, 0.5, 0.1, 0.0, 2.0, float("nan")]
    _with_filters(b, seed, ks, ps)
    gu.check_batch(verifier, b, torch_mod, label=f"filters seed={seed}")


def test_filters_off_are_bitwise_unfiltered(verifier, torch_mod):
    b = make_random_batch(520, B=32, V=5000, kmax=6, dtype="bf16", modes=ALL_MODES)
    plain = gu.run_gpu(verifier, b, torch_mod)
    b.top_k = np.where(np.arange(b.batch) % 2 == 0, 0, b.vocab).astype(np.int32)
    b.top_p = np.where(np.arange(b.batch) % 3 == 0, 1.0, 3.0).astype(np.float32)
    filt = gu.run_gpu(verifier, b, torch_mod)
    for k in ("accepted_len", "emitted", "status"):
        assert np.array_equal(plain[k], filt[k]), k
    assert np.array_equal(plain["p_at"], filt["p_at"], equal_nan=True)


def _tie_batch(dtype: str, V: int, seed: int, flat: bool) -> Batch:
    """Rows on a coarse value grid (many equal logits); with ``flat`` most of
    the row shares one value, so the boundary bin holds more candidates than
    the filter's LDS buffer."""
    rng = np.random.default_rng(seed)
    B, K = 12, 3
    n = B * (K + 1)
    if flat:
        tgt = np.zeros((n, V), np.float32)
        tgt += (rng.random((n, V)) < 0.01) * np.round(rng.standard_normal((n, V)) * 4) / 4
    else:
        tgt = (np.round(rng.standard_normal((n, V)) * 2) / 2).astype(np.float32)
    modes = rng.choice(np.asarray([MODE_ONEHOT, MODE_STRICT], np.uint8), size=B)
    toks = rng.integers(0, V, size=B * K).astype(np.int32)
    store = bf16_round(tgt) if dtype == "bf16" else tgt
    return Batch(name=f"ties V={V} {dtype} flat={flat}", vocab=V, dtype=dtype, target=store, draft=None,
                 num_draft=np.full(B, K, np.int32), draft_tokens=toks,
                 temperature=rng.uniform(0.5, 1.5, B).astype(np.float32), mode=modes,
                 seq_ids=np.arange(B, dtype=np.uint32), seed=seed)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("flat", [False, True])
def test_ties_and_large_boundary_bins(verifier, torch_mod, dtype, flat):
    V = 30000
    b = _tie_batch(dtype, V, 600 + int(flat), flat)
    _with_filters(b, 7, [0, 1, 100, 5000, 15000, 29999], [1.0, 0.999, 0.9, 0.5, 0.3, 1e-4])
    gu.check_batch(verifier, b, torch_mod, label=f"ties {dtype} flat={flat}")


def test_c3_with_filters_bench_context(torch_mod):
    import rejection_sampling_verify_06_amd as sv
    v = sv.Verifier(max_batch=256, max_k=8, max_vocab=152064, device=0)
    try:
        for step, (k, p) in enumerate([(50, 0.9), (0, 0.95), (2000, 1.0)]):
            b = make_config_batch(3, step)
            b.top_k = np.full(b.batch, k, np.int32)
            b.top_p = np.full(b.batch, p, np.float32)
            gu.check_batch(v, b, torch_mod, label=f"C3 step {step} top_k={k} top_p={p}, bench context")
    finally:
        v.close()


@pytest.mark.parametrize("config", [2, 4])
def test_c2_c4_with_filters_full_size(torch_mod, config):
    """The same filters on the other benchmark shapes: float32 rows of
    128,256 tokens (C2: the bracket searches, the split final draw over
    eight blocks a sequence) and one-hot and greedy bf16 rows (C4: greedy
    ignores the filter, one-hot draws from the filtered p)."""
    import rejection_sampling_verify_06_amd as sv
    v = sv.Verifier(max_batch=128, max_k=8, max_vocab=128256, device=0)
    try:
        for step, (k, p) in enumerate([(50, 0.9), (0, 0.95), (2000, 1.0)]):
            b = make_config_batch(config, step)
            b.top_k = np.full(b.batch, k, np.int32)
            b.top_p = np.full(b.batch, p, np.float32)
            gu.check_batch(v, b, torch_mod, label=f"C{config} step {step} top_k={k} top_p={p}")
    finally:
        v.close()


def test_c3_strict_with_filters_full_size(torch_mod):
    """C3 in strict sample-match mode with the three filters: the filtered
    target rows' mass below the proposal (the strict draw's split) at the
    benchmark shape."""
    import rejection_sampling_verify_06_amd as sv
    v = sv.Verifier(max_batch=256, max_k=8, max_vocab=152064, device=0)
    try:
        for step, (k, p) in enumerate([(50, 0.9), (0, 0.95), (2000, 1.0)]):
            b = make_config_batch(3, step, strict=True)
            b.top_k = np.full(b.batch, k, np.int32)
            b.top_p = np.full(b.batch, p, np.float32)
            gu.check_batch(v, b, torch_mod, label=f"C3 strict step {step} top_k={k} top_p={p}")
    finally:
        v.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bounded_selection_edges(verifier, torch_mod, dtype):
    """Top-k at the edges of the bounded selection (1, 1023, 1024; 1025 takes
    the histogram path), with and without top-p, on rows that are not
    16-byte aligned; a second call gives bitwise the same outputs."""
    b = make_random_batch(540 + (dtype == "bf16"), B=16, V=40000, kmax=4, dtype=dtype, ld_pad=5,
                          modes=ALL_MODES)
    b.top_k = np.array([1, 1023, 1024, 1025, 300, 1024, 1, 1025] * 2, np.int32)
    b.top_p = np.array([1.0] * 8 + [0.9, 0.5, 0.99, 0.9, 0.0, 0.7, 0.95, 0.8], np.float32)
    _, out, _ = gu.check_batch(verifier, b, torch_mod, label=f"bounded selection edges {dtype}")
    again = gu.run_gpu(verifier, b, torch_mod)
    for k in ("accepted_len", "emitted", "status"):
        assert np.array_equal(out[k], again[k]), k
    assert np.array_equal(out["p_at"], again["p_at"], equal_nan=True)
    assert np.array_equal(out["q_at"], again["q_at"], equal_nan=True)


def _mask_rows(b: Batch, rng, frac: float):
    """-inf on a random fraction of every row's columns (a masked vocabulary),
    never on the row's largest logit."""
    from workloads import bf16_round
    neg = bf16_round(np.array([-np.inf], np.float32))[0] if b.dtype == "bf16" else np.float32(-np.inf)
    for arr in (b.target, b.draft):
        if arr is None:
            continue
        vals = arr[:, :b.vocab].view(np.uint16).astype(np.uint32) << 16 if b.dtype == "bf16" else arr[:, :b.vocab]
        vals = vals.view(np.float32) if b.dtype == "bf16" else vals
        keep = np.argmax(vals, axis=1)
        m = rng.random((arr.shape[0], b.vocab)) < frac
        m[np.arange(arr.shape[0]), keep] = False
        sub = arr[:, :b.vocab]
        sub[m] = neg
        arr[:, :b.vocab] = sub


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [5, 9, 4099, 50000])
def test_filter_special_values(verifier, torch_mod, dtype, V):
    """Filters on rows with a masked (-inf) part of the vocabulary, on
    vocabularies too small for one 16-byte vector round, on rows whose
    largest logit is tied, at temperatures from 0.05 to 5, on rows that are not
    16-byte aligned."""
    rng = np.random.default_rng(560 + V + (dtype == "bf16"))
    b = make_random_batch(560 + V, B=20, V=V, kmax=3, dtype=dtype, ld_pad=1, modes=ALL_MODES)
    _mask_rows(b, rng, 0.3)
    # ties at the largest logit in some target rows
    tgt = b.target if dtype == "f32" else None
    if tgt is not None and V >= 9:
        for r in range(0, b.target.shape[0], 4):
            row = b.target[r, :V]
            top = row.max()
            row[rng.choice(V, 3, replace=False)] = top
    b.temperature = rng.choice(np.array([0.05, 0.3, 1.0, 2.5, 5.0], np.float32), size=b.batch)
    ks = [0, 1, 2, 3, 50, 1024, 1025, V - 1]
    ps = [1.0, 0.95, 0.5, 0.0, 0.999]
    _with_filters(b, 9 + V, ks, ps)
    gu.check_batch(verifier, b, torch_mod, label=f"filter special values V={V} {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_topp_crossing_past_bracket_range(verifier, torch_mod, dtype):
    """Top-p alone whose crossing lies beyond 2^-32 of the largest weight (one
    logit 25 above a N(0, 1) row, p = 0.9999999): neither the bounded
    selection nor the bracket search can hold it, so the histogram path
    decides."""
    from workloads import bf16_round
    b = make_random_batch(580 + (dtype == "bf16"), B=6, V=60000, kmax=2, dtype=dtype, modes=ALL_MODES,
                          scale=(1.0, 1.0), noise=(0.0, 0.5), temp=(1.0, 1.0))
    rng = np.random.default_rng(581)
    for arr in (b.target, b.draft):
        if arr is None:
            continue
        cols = rng.integers(0, b.vocab, size=arr.shape[0])
        for r, col in enumerate(cols):
            arr[r, col] = bf16_round(np.array([25.0], np.float32))[0] if dtype == "bf16" else np.float32(25.0)
    b.top_k = np.zeros(b.batch, np.int32)
    b.top_p = np.full(b.batch, 0.9999999, np.float32)
    gu.check_batch(verifier, b, torch_mod, label=f"top-p past the bracket range {dtype}")


def _flat_batch(dtype: str, V: int, seed: int, grid: int) -> Batch:
    """Rows of N(0, sigma) logits, sigma in {0.5, 1, 2}, at temperatures 0.7
    to 3: with sigma / T <= 2 the 1024 largest of 100,000 weights carry at most
    about 37% of a row's mass (the upper 1% of a normal holds P(Z > 2.33 -
    sigma/T) of the exponential's mean), so every target row's top-p of 0.5 or
    more is left to the bracket search (draft rows, target plus noise, take
    either path).  With ``grid`` > 0 the logits sit on a grid of
    1/grid, so the crossing falls inside a tie group of thousands of tokens.
    Sample-mode sequences bring draft rows (filtered too); proposals are the
    target row's argmax or a random token."""
    rng = np.random.default_rng(seed)
    B, K = 8, 2
    sig_t = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), size=(B * (K + 1), 1))
    tgt = rng.standard_normal((B * (K + 1), V)).astype(np.float32) * sig_t
    dft = (tgt.reshape(B, K + 1, V)[:, :K].reshape(B * K, V)
           + 0.5 * rng.standard_normal((B * K, V)).astype(np.float32))
    if grid:
        tgt = np.round(tgt * grid) / grid
        dft = np.round(dft * grid) / grid
    temps = rng.choice(np.array([0.7, 1.0, 1.5, 3.0], np.float32), size=B)
    # sigma / T <= 2 on every row: scale down the rows of low-temperature sequences
    row_t = np.repeat(temps, K + 1)[:, None]
    tgt = np.where(sig_t / row_t > 2.0, tgt * (2.0 * row_t / sig_t), tgt).astype(np.float32)
    if grid:
        tgt = np.round(tgt * grid) / grid
    modes = rng.choice(np.asarray([MODE_SAMPLE, MODE_ONEHOT, MODE_STRICT], np.uint8), size=B)
    am = tgt.reshape(B, K + 1, V)[:, :K].argmax(axis=2).reshape(-1)
    toks = np.where(rng.random(B * K) < 0.5, am, rng.integers(0, V, size=B * K)).astype(np.int32)
    store = (lambda a: bf16_round(a)) if dtype == "bf16" else (lambda a: a)
    return Batch(name=f"flat rows V={V} {dtype} grid={grid}", vocab=V, dtype=dtype, target=store(tgt),
                 draft=store(dft.astype(np.float32)), num_draft=np.full(B, K, np.int32), draft_tokens=toks,
                 temperature=temps, mode=modes, seq_ids=np.arange(B, dtype=np.uint32), seed=seed,
                 top_k=np.zeros(B, np.int32),
                 top_p=rng.choice(np.array([0.5, 0.9, 0.95, 0.99, 0.999], np.float32), size=B))


@pytest.mark.parametrize("dtype,grid", [("bf16", 0), ("f32", 0), ("bf16", 4), ("f32", 8)])
def test_topp_bracket_search_flat_rows(verifier, torch_mod, dtype, grid):
    """Top-p alone on rows whose nucleus the thread maxima cannot carry: the
    bracket search's dense first pass, its binned passes and the f32 tie
    group past the last pass (grid 8); bf16 rows of N(0, sigma) take more
    distinct values than the value table holds and fall back to the bracket
    search, bf16 rows on a grid of 1/4 take the value table (strict-mode
    target rows take the bracket search either way); a second call gives
    bitwise the same outputs."""
    b = _flat_batch(dtype, 100_000, 610 + grid + (dtype == "bf16"), grid)
    _, out, _ = gu.check_batch(verifier, b, torch_mod, label=f"top-p bracket search, flat rows {dtype} grid={grid}")
    again = gu.run_gpu(verifier, b, torch_mod)
    for k in ("accepted_len", "emitted", "status"):
        assert np.array_equal(out[k], again[k]), k
    assert np.array_equal(out["p_at"], again["p_at"], equal_nan=True)


def _segment_elements(dtype: str, V: int, chunk: int, group: int) -> np.ndarray:
    """Element indices of one row-statistics segment: the elements that the
    8 lanes of `group` (of 32) load from 32 KB chunk `chunk`, 16-byte
    vectors handed out to 256 threads in turn."""
    vec = 8 if dtype == "bf16" else 4
    ce = 32768 // (2 if dtype == "bf16" else 4)
    e = np.arange(chunk * ce, min(V, (chunk + 1) * ce))
    thread = ((e - chunk * ce) // vec) % 256
    return e[thread // 8 == group]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_topk_heavy_tokens_in_one_segment(verifier, torch_mod, dtype):
    """Top-k whose largest logits all sit in one segment of the row statistics:
    the k-th largest segment maximum then lies far below the k-th largest
    logit, so the bound from the segment maxima admits many more tokens than
    k, and on every other row, where 1500 tokens tie just below the heavy
    ones, more than the candidate buffer holds (the histogram path then
    decides)."""
    rng = np.random.default_rng(640 + (dtype == "bf16"))
    V, B, K = 100_000, 6, 2
    b = make_random_batch(641, B=B, V=V, kmax=K, k_min=K, dtype=dtype, modes=ALL_MODES, scale=(0.5, 2.0))
    for arr in (b.target, b.draft):
        if arr is None:
            continue
        for r in range(arr.shape[0]):
            row = bf16_widen(arr[r, :V]) if dtype == "bf16" else arr[r, :V]
            top = float(row.max())
            if r % 2:                            # 1500 tokens tied just below: more candidates than the buffer
                tied = np.full(1500, top + 0.5, np.float32)
                arr[r, rng.choice(np.arange(3 * 32768 // 4, V), size=tied.size, replace=False)] = (
                    bf16_round(tied) if dtype == "bf16" else tied)
            heavy = (top + np.linspace(2.0, 1.0, 64)).astype(np.float32)   # the row's 64 largest
            seg = _segment_elements(dtype, V, int(rng.integers(0, 3)), int(rng.integers(0, 32)))
            cols = rng.choice(seg, size=heavy.size, replace=False)
            arr[r, cols] = bf16_round(heavy) if dtype == "bf16" else heavy
    b.top_k = rng.choice(np.array([10, 50, 64], np.int32), size=B)
    b.top_p = rng.choice(np.array([1.0, 0.9], np.float32), size=B)
    gu.check_batch(verifier, b, torch_mod, label=f"top-k, heavy tokens in one segment {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("where", ["tail", "last_vector", "many_segments"])
def test_bounded_read_of_the_bound_segments(torch_mod, dtype, where):
    """The bounded selection reads only the row-statistics segments whose
    maximum reaches its bound.  The row's largest logits placed in its last
    few elements (V not a multiple of a vector, rows on 16 bytes: read as
    single elements), in
    its last whole vector, or tied at the top across more segments than the
    list holds (V = 2,097,152: 4096 segments a bf16 row, 8192 a float32 one,
    the tie on about 600 of them, so the whole row is read); top-k 50 and top-p 0.9 per sequence as in the
    benchmark's filtered workload, every mode."""
    import rejection_sampling_verify_06_amd as sv
    rng = np.random.default_rng(660 + ["tail", "last_vector", "many_segments"].index(where) + (dtype == "f32"))
    # (the segment maxima bound top-k when there are at least 2k of them: 32 a 32 KB chunk)
    V = {"tail": 100_003, "last_vector": 163_840, "many_segments": 2_097_152}[where]
    B = 3 if where == "many_segments" else 8
    # rows on 16 bytes (the segment maxima exist only for such rows): V = 100,003 in rows 100,008 apart
    b = make_random_batch(661, B=B, V=V, kmax=2, k_min=1, dtype=dtype, modes=ALL_MODES, scale=(0.5, 2.0),
                          ld_pad=5 if where == "tail" else 0)
    vec = 8 if dtype == "bf16" else 4
    assert (b.target.shape[1] * (2 if dtype == "bf16" else 4)) % 16 == 0
    for arr in (b.target, b.draft):
        if arr is None:
            continue
        for r in range(arr.shape[0]):
            row = bf16_widen(arr[r, :V]) if dtype == "bf16" else arr[r, :V].copy()
            top = float(row.max())
            if where == "tail":
                cols = np.arange(V - (V % vec), V)              # the elements after the last whole vector
                vals = top + np.linspace(3.0, 2.0, cols.size)
            elif where == "last_vector":
                cols = np.arange(V - vec, V)
                vals = top + np.linspace(3.0, 2.0, cols.size)
            else:
                cols = rng.choice(V // 1024, size=600, replace=False) * 1024 + rng.integers(0, 1024, size=600)
                vals = np.full(cols.size, top + 2.0)
            arr[r, cols] = bf16_round(vals.astype(np.float32)) if dtype == "bf16" else vals.astype(np.float32)
    b.top_k = np.full(b.batch, 50, np.int32)
    b.top_p = np.full(b.batch, 0.9, np.float32)
    v = sv.Verifier(max_batch=16, max_k=4, max_vocab=V, device=0)
    try:
        gu.check_batch(v, b, torch_mod, label=f"bounded read of the bound's segments: {where} {dtype} V={V}")
    finally:
        v.close()


@pytest.mark.parametrize("dtype,V,ks", [("bf16", 152064, (1025, 2000, 5000)), ("f32", 40000, (1100, 3000, 30000)),
                                        ("bf16", 20000, (1500, 19999))])
def test_large_top_k_count_bracket(verifier, torch_mod, dtype, V, ks):
    """top-k above the bounded selection's 1024 tokens, alone: the value table
    (bf16 rows, its band around the k-th largest from a sample) or the count
    bracket search (f32 rows, strict-mode target rows, and bf16 rows with
    more distinct values than the table holds: a first pass split at 8, 32,
    128 log2 units below the maximum, then even or binned passes) finds the
    k-th largest logit; every mode, temperatures 0.3..1.5 (the k-th token far
    below the maximum at low temperature)."""
    b = make_random_batch(560 + V % 97, B=12, V=V, kmax=3, dtype=dtype, modes=ALL_MODES, temp=(0.3, 1.5))
    b.top_k = np.resize(np.asarray(ks, np.int32), b.batch).astype(np.int32)
    b.top_p = None
    gu.check_batch(verifier, b, torch_mod, label=f"large top-k {ks} {dtype}")


def test_large_top_k_on_tie_rows(verifier, torch_mod):
    """top-k 1500 and 3000 on bf16 rows on a coarse grid: the k-th value is
    shared by many tokens (the bracket ends as one value and keeps them all)."""
    b = _tie_batch("bf16", 30000, 571, flat=False)
    b.top_k = np.resize(np.asarray([1500, 3000, 1100], np.int32), b.batch).astype(np.int32)
    b.top_p = None
    gu.check_batch(verifier, b, torch_mod, label="large top-k on tie rows")
    b = _tie_batch("bf16", 30000, 572, flat=True)
    b.top_k = np.resize(np.asarray([2000, 1030], np.int32), b.batch).astype(np.int32)
    b.top_p = None
    gu.check_batch(verifier, b, torch_mod, label="large top-k on flat tie rows")


def _zipf_bf16_batch(seed: int, V: int, ld: int, B: int = 10) -> Batch:
    """Zipf-shaped bf16 rows as in the benchmark workloads: -1.1 ln(rank) +
    N(0, 1), randomly relabelled per row, draft = target + N(0, 0.7^2).  In
    bf16 such a row takes a few hundred distinct values, the ones near a
    top-p crossing shared by thousands of tokens.  K ~ U{1..3}, modes SAMPLE,
    ONEHOT, GREEDY and STRICT, T ~ U[0.3, 1.5]; SAMPLE proposals are the draft
    row's argmax or one of its 2000 largest tokens, the others the target
    row's argmax or a random token."""
    rng = np.random.default_rng(seed)
    K = rng.integers(1, 4, size=B).astype(np.int32)
    modes = rng.choice(np.asarray([MODE_SAMPLE, MODE_ONEHOT, MODE_GREEDY, MODE_STRICT], np.uint8), size=B)
    temps = rng.uniform(0.3, 1.5, size=B).astype(np.float32)
    base = (-1.1 * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)
    n_t, n_d = int(K.sum()) + B, int(K.sum())
    tgt = np.zeros((n_t, ld), np.float32)
    dft = np.zeros((n_d, ld), np.float32)
    toks = np.empty(n_d, np.int32)
    rt = rd = 0
    for s in range(B):
        for i in range(int(K[s]) + 1):
            t32 = bf16_widen(bf16_round(base[rng.permutation(V)] + rng.standard_normal(V).astype(np.float32)))
            tgt[rt, :V] = t32
            if i < K[s]:
                d32 = bf16_widen(bf16_round(t32 + 0.7 * rng.standard_normal(V).astype(np.float32)))
                dft[rd, :V] = d32
                src = d32 if modes[s] == MODE_SAMPLE else t32
                top = np.argpartition(-src, 2000)[:2000]
                toks[rd] = int(src.argmax()) if rng.random() < 0.5 else int(rng.choice(top))
                rd += 1
            rt += 1
    return Batch(name=f"zipf bf16 rows V={V} ld={ld}", vocab=V, dtype="bf16", target=bf16_round(tgt),
                 draft=bf16_round(dft), num_draft=K, draft_tokens=toks, temperature=temps, mode=modes,
                 seq_ids=np.arange(B, dtype=np.uint32), seed=seed, top_k=np.zeros(B, np.int32),
                 top_p=np.ones(B, np.float32))


@pytest.mark.parametrize("V,ld", [(152064, 152064), (100003, 100008)])
@pytest.mark.parametrize("which", ["top_p", "top_k"])
def test_value_table_zipf_rows(verifier, torch_mod, V, ld, which):
    """bf16 rows with few distinct values and large tie groups, one filter per
    sequence: the value table's sample, its band around the crossing, the
    full read's counts and the exact threshold (top-p 0.5 .. 0.99, top-k
    1025 .. 40000), the row tail past the last whole vector (V = 100003),
    strict-mode target rows on the other paths; a second call gives bitwise
    the same outputs."""
    b = _zipf_bf16_batch(700 + V % 7 + (which == "top_k"), V, ld)
    rng = np.random.default_rng(710 + V % 7)
    if which == "top_p":
        b.top_p = rng.choice(np.array([0.5, 0.9, 0.95, 0.99], np.float32), size=b.batch)
    else:
        b.top_k = rng.choice(np.array([1025, 2000, 5000, 40000], np.int32), size=b.batch)
    _, out, _ = gu.check_batch(verifier, b, torch_mod, label=f"value table, zipf bf16 V={V} {which}")
    again = gu.run_gpu(verifier, b, torch_mod)
    for k in ("accepted_len", "emitted", "status"):
        assert np.array_equal(out[k], again[k]), k


@pytest.mark.parametrize("V", [4104, 30000])
@pytest.mark.parametrize("which", ["top_p", "top_k"])
def test_value_table_signed_zero_and_masked_rows(verifier, torch_mod, V, which):
    """bf16 rows (16-byte aligned) built so that the crossing falls in a tie
    group of exact zeros stored half as +0 and half as -0 (two bit patterns,
    one value: the value table must keep or drop both together): a few
    positive tokens, about 40% zeros, the rest negative; a third of the rows
    also masked to -inf over 30% of the vocabulary; temperatures 0.05 to 5;
    V just above the table's smallest row and 30000."""
    rng = np.random.default_rng(730 + V % 11 + (which == "top_k"))
    b = make_random_batch(731 + V % 11, B=16, V=V, kmax=3, k_min=1, dtype="bf16", modes=ALL_MODES)
    n_pos = max(8, V // 50)
    for arr in (b.target, b.draft):
        if arr is None:
            continue
        for r in range(arr.shape[0]):
            row = np.empty(V, np.float32)
            perm = rng.permutation(V)
            n_zero = int(0.4 * V)
            row[perm[:n_pos]] = rng.uniform(0.5, 3.0, size=n_pos)
            zeros = perm[n_pos:n_pos + n_zero]
            row[zeros] = np.where(rng.random(n_zero) < 0.5, np.float32(0.0), np.float32(-0.0))
            rest = perm[n_pos + n_zero:]
            row[rest] = rng.uniform(-5.0, -1.0, size=rest.size)
            if r % 3 == 2:
                row[rng.choice(V, int(0.3 * V), replace=False)] = -np.inf
            arr[r, :V] = bf16_round(row)
    b.temperature = rng.choice(np.array([0.05, 0.3, 1.0, 2.5, 5.0], np.float32), size=b.batch)
    if which == "top_p":
        b.top_p = rng.choice(np.array([0.3, 0.5, 0.9, 0.999], np.float32), size=b.batch)
    else:
        b.top_k = rng.choice(np.array([n_pos + 10, n_pos + V // 8, V // 2, V - 1], np.int32), size=b.batch)
    neg_zero = int((b.target[:, :V] == 0x8000).sum())
    assert neg_zero > 0, "the rows must hold -0 patterns"
    gu.check_batch(verifier, b, torch_mod, label=f"value table, signed zeros and masked rows V={V} {which}")
