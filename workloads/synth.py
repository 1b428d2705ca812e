"""Seeded synthetic verify-step batches.

Layout of a batch (the packed ragged layout the library takes):

* ``num_draft[s] = K_s`` draft tokens for sequence ``s``.
* Target logits: ``sum_s (K_s + 1)`` rows.  Sequence ``s`` owns the rows
  ``off_t[s] .. off_t[s] + K_s`` with ``off_t[s] = sum_{j<s} (K_j + 1)``; its
  row ``i < K_s`` judges draft token ``i`` and its row ``K_s`` is the bonus
  distribution.
* Draft logits: ``sum_s K_s`` rows; sequence ``s`` owns rows
  ``off_d[s] .. off_d[s] + K_s - 1`` with ``off_d[s] = sum_{j<s} K_j``.
* ``draft_tokens``: ``sum_s K_s`` int32, packed like the draft rows.
* Rows are ``ld >= V`` elements apart; columns ``V .. ld-1`` are padding that
  must never be read (filled here with a large finite logit so a stray read
  changes the result).

Logits are float32, or bfloat16 stored as uint16 bit patterns.  bfloat16
values are produced by round-to-nearest-even on float32 bits.

Random numbers come from numpy's PCG64 seeded with ``(1000 + config, step)``
for the five benchmark workloads, so any step can be regenerated on its own.
The Philox seed that the verify step itself uses is ``step`` (base seed 0).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

# Per-sequence verify mode, as encoded in the library's ``mode`` input.
MODE_SAMPLE = 0   # probabilistic accept/correct against draft logits q
MODE_GREEDY = 1   # accept iff the proposed token is the target argmax
MODE_ONEHOT = 2   # deterministic proposal: q is one-hot on the proposed token
MODE_STRICT = 3   # sample match: accept iff the target's own sample equals the proposal

PAD_LOGIT = 30000.0  # value written into row padding (columns >= V)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_widen(u: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32, exact."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Batch:
    name: str
    vocab: int
    dtype: str                      # "f32" or "bf16"
    target: np.ndarray              # [sum(K+1), ld] float32 or uint16
    draft: Optional[np.ndarray]     # [sum(K), ld] same dtype, or None
    num_draft: np.ndarray           # int32 [B]
    draft_tokens: np.ndarray        # int32 [sum(K)]
    temperature: np.ndarray         # float32 [B]
    mode: np.ndarray                # uint8 [B]
    seq_ids: np.ndarray             # uint32 [B]
    seed: int                       # Philox key (64-bit)
    top_k: Optional[np.ndarray] = None   # int32 [B] (top-k filter; <= 0 off) or None
    top_p: Optional[np.ndarray] = None   # float32 [B] (nucleus filter; >= 1 off) or None

    @property
    def batch(self) -> int:
        return int(self.num_draft.shape[0])

    @property
    def total_draft(self) -> int:
        return int(self.num_draft.astype(np.int64).sum())

    @property
    def ld(self) -> int:
        return int(self.target.shape[1])

    @property
    def positions(self) -> int:
        """Verified positions in this batch: sum_s (K_s + 1)."""
        return self.total_draft + self.batch

    def nbytes_logits(self) -> int:
        n = self.target.nbytes
        if self.draft is not None:
            n += self.draft.nbytes
        return n


# ---------------------------------------------------------------------------
# row builders
# ---------------------------------------------------------------------------

def sequence_slice(b: "Batch", lo: int, hi: int, name: Optional[str] = None) -> "Batch":
    """Sequences lo..hi-1 of a batch, as the packed layout of their own (their
    target and draft rows, tokens and per-sequence values; seq_ids kept, so
    the Philox draws are those of the whole batch).  Pure data slicing."""
    K = b.num_draft.astype(np.int64)
    d0, d1 = int(K[:lo].sum()), int(K[:hi].sum())
    pick = lambda a: None if a is None else a[lo:hi].copy()
    return Batch(name=name or f"{b.name} [sequences {lo}..{hi - 1}]", vocab=b.vocab, dtype=b.dtype,
                 target=b.target[d0 + lo:d1 + hi].copy(), draft=None if b.draft is None else b.draft[d0:d1].copy(),
                 num_draft=b.num_draft[lo:hi].copy(), draft_tokens=b.draft_tokens[d0:d1].copy(),
                 temperature=b.temperature[lo:hi].copy(), mode=b.mode[lo:hi].copy(),
                 seq_ids=b.seq_ids[lo:hi].copy(), seed=b.seed, top_k=pick(b.top_k), top_p=pick(b.top_p))


def _zipf_base(V: int) -> np.ndarray:
    """Sorted Zipf-shaped base logits: -1.1 * ln(rank), rank = 1..V."""
    return (-1.1 * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)


class _ZipfRows:
    """Zipf-shaped logit rows: base[rank] + N(0,1), randomly relabelled.

    One uniformly random permutation of the vocabulary is drawn per batch;
    each row uses that permutation rotated by its own random offset, so every
    row's labelling is a uniformly random permutation (rows share structure
    only through the rotation, which does not change any row's statistics).
    """

    def __init__(self, rng: np.random.Generator, V: int):
        self.rng = rng
        self.V = V
        self.perm_base = _zipf_base(V)[rng.permutation(V)]

    def row(self) -> np.ndarray:
        off = int(self.rng.integers(self.V))
        r = np.roll(self.perm_base, off)
        r = r + self.rng.standard_normal(self.V, dtype=np.float32)
        return r.astype(np.float32, copy=False)


def _store(row_f32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(row_f32) if dtype == "bf16" else row_f32.astype(np.float32)


def _stored_as_f32(row: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_widen(row) if dtype == "bf16" else row


def _draw_from_logits(rng: np.random.Generator, logits_f32: np.ndarray, T: float) -> int:
    """Proposer stand-in: one token from softmax(logits / T) by the
    exponential-race (Gumbel-max) construction, argmax(l/T - ln E), E ~ Exp(1).
    Float32 throughout: the verify step treats the proposal as given input."""
    e = rng.standard_exponential(logits_f32.shape[0], dtype=np.float32)
    np.maximum(e, np.float32(1e-30), out=e)
    key = logits_f32 / np.float32(T) - np.log(e)
    return int(np.argmax(key))


def _near_argmax_token(rng: np.random.Generator, logits_f32: np.ndarray, p_hit: float) -> int:
    """N-gram/prompt-lookup style proposal stand-in: the row argmax with
    probability p_hit, else a uniformly random other token."""
    V = logits_f32.shape[0]
    am = int(np.argmax(logits_f32))
    if V == 1 or rng.random() < p_hit:
        return am
    j = int(rng.integers(V - 1))
    return j + (1 if j >= am else 0)


def _pad(rows: np.ndarray, ld: int, dtype: str) -> np.ndarray:
    n, V = rows.shape
    if ld == V:
        return rows
    out = np.empty((n, ld), dtype=rows.dtype)
    out[:, :V] = rows
    pad = np.float32(PAD_LOGIT)
    out[:, V:] = bf16_round(np.array([pad]))[0] if dtype == "bf16" else pad
    return out


# ---------------------------------------------------------------------------
# the five benchmark workloads
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    0: "C0: B=1 K=4 V=1000 fp32 gaussian, T=1",
    1: "C1: B=1 K=5 V=32000 bf16 zipf, T=1",
    2: "C2: B=32 K=5 V=128256 fp32 zipf+peak, T=0.7",
    3: "C3: B=256 K~U{1..8} V=152064 bf16 zipf, T~U[0.3,1.2]",
    4: "C4: B=128 K=5 V=128256 bf16 zipf, one-hot half + greedy half",
}
STRICT_SUFFIX = "; every sequence in strict sample-match mode, no draft logits"


def config_description(cfg: int) -> dict:
    """Static shape facts of a workload (no random draws)."""
    return {
        0: dict(batch=1, k="4", vocab=1000, dtype="f32"),
        1: dict(batch=1, k="5", vocab=32000, dtype="bf16"),
        2: dict(batch=32, k="5", vocab=128256, dtype="f32"),
        3: dict(batch=256, k="U{1..8}", vocab=152064, dtype="bf16"),
        4: dict(batch=128, k="5", vocab=128256, dtype="bf16"),
    }[cfg]


def make_config_batch(cfg: int, step: int = 0, ld_pad: int = 0,
                      interleave_modes: bool = False, strict: bool = False) -> Batch:
    """Batch ``step`` of benchmark workload ``cfg`` (0..4).

    C0  B=1, K=4, V=1000, fp32: target ~ N(0, 2^2) i.i.d.; draft = target +
        N(0, 0.5^2); T = 1.
    C1  B=1, K=5, V=32000, bf16: Zipf-shaped target; draft = target + N(0,1).
    C2  B=32, K=5, V=128256, fp32: Zipf-shaped target with one uniformly
        random token per row boosted by +6; draft = target + N(0, 0.7^2);
        T = 0.7.
    C3  B=256, V=152064, bf16: K_s ~ U{1..8}, T_s ~ U[0.3, 1.2],
        sigma_s ~ U[0.2, 2.0]; Zipf-shaped target; draft = target +
        N(0, sigma_s^2).
    C4  B=128, K=5, V=128256, bf16 target only: sequences 0..63 use the
        one-hot proposal, 64..127 strict greedy (``interleave_modes``
        alternates them instead); proposals are the target argmax with
        probability 0.7, else uniform over the other tokens; T = 1.

    SAMPLE-mode proposals are drawn from the stored draft logits at the
    sequence's temperature.
    """
    rng = np.random.default_rng(np.random.PCG64([1000 + cfg, step]))
    if cfg == 0:
        B, V, dtype = 1, 1000, "f32"
        K = np.full(B, 4, np.int32)
        T = np.full(B, 1.0, np.float32)
        modes = np.full(B, MODE_SAMPLE, np.uint8)
        sig = np.full(B, 0.5, np.float32)
    elif cfg == 1:
        B, V, dtype = 1, 32000, "bf16"
        K = np.full(B, 5, np.int32)
        T = np.full(B, 1.0, np.float32)
        modes = np.full(B, MODE_SAMPLE, np.uint8)
        sig = np.full(B, 1.0, np.float32)
    elif cfg == 2:
        B, V, dtype = 32, 128256, "f32"
        K = np.full(B, 5, np.int32)
        T = np.full(B, 0.7, np.float32)
        modes = np.full(B, MODE_SAMPLE, np.uint8)
        sig = np.full(B, 0.7, np.float32)
    elif cfg == 3:
        B, V, dtype = 256, 152064, "bf16"
        K = rng.integers(1, 9, size=B).astype(np.int32)
        T = rng.uniform(0.3, 1.2, size=B).astype(np.float32)
        modes = np.full(B, MODE_SAMPLE, np.uint8)
        sig = rng.uniform(0.2, 2.0, size=B).astype(np.float32)
    elif cfg == 4:
        B, V, dtype = 128, 128256, "bf16"
        K = np.full(B, 5, np.int32)
        T = np.full(B, 1.0, np.float32)
        if interleave_modes:
            modes = np.where(np.arange(B) % 2 == 0, MODE_ONEHOT, MODE_GREEDY).astype(np.uint8)
        else:
            modes = np.where(np.arange(B) < B // 2, MODE_ONEHOT, MODE_GREEDY).astype(np.uint8)
        sig = np.zeros(B, np.float32)
    else:
        raise ValueError(f"unknown workload {cfg}")

    n_t = int(K.sum()) + B
    n_d = int(K.sum())
    tgt = np.empty((n_t, V), dtype=np.uint16 if dtype == "bf16" else np.float32)
    has_draft = cfg != 4
    dft = np.empty((n_d, V), dtype=tgt.dtype) if has_draft else None
    toks = np.empty(n_d, np.int32)
    zipf = _ZipfRows(rng, V) if cfg != 0 else None

    rt = rd = 0
    for s in range(B):
        for i in range(int(K[s]) + 1):
            if cfg == 0:
                row = (2.0 * rng.standard_normal(V, dtype=np.float32)).astype(np.float32)
            else:
                row = zipf.row()
                if cfg == 2:
                    row[int(rng.integers(V))] += np.float32(6.0)
            tgt[rt] = _store(row, dtype)
            if i < K[s]:
                t32 = _stored_as_f32(tgt[rt], dtype)
                if has_draft:
                    d = t32 + np.float32(sig[s]) * rng.standard_normal(V, dtype=np.float32)
                    dft[rd] = _store(d.astype(np.float32), dtype)
                if modes[s] == MODE_SAMPLE:
                    toks[rd] = _draw_from_logits(rng, _stored_as_f32(dft[rd], dtype), float(T[s]))
                else:
                    toks[rd] = _near_argmax_token(rng, t32, 0.7)
                rd += 1
            rt += 1

    ld = V + ld_pad
    if strict:      # the same proposals, verified by sample match; the draft logits are not needed
        modes = np.full(B, MODE_STRICT, np.uint8)
        dft = None
    return Batch(
        name=CONFIG_NAMES[cfg] + (STRICT_SUFFIX if strict else ""), vocab=V, dtype=dtype,
        target=_pad(tgt, ld, dtype),
        draft=_pad(dft, ld, dtype) if dft is not None else None,
        num_draft=K, draft_tokens=toks, temperature=T, mode=modes,
        seq_ids=np.arange(B, dtype=np.uint32), seed=int(step),
    )


# ---------------------------------------------------------------------------
# small random batches for parity tests
# ---------------------------------------------------------------------------

def make_random_batch(seed: int, B: int, V: int, kmax: int, dtype: str = "f32",
                      modes: Sequence[int] = (MODE_SAMPLE, MODE_GREEDY, MODE_ONEHOT),
                      k_min: int = 0, ld_pad: int = 0, with_draft: Optional[bool] = None,
                      scale: tuple = (0.5, 3.0), noise: tuple = (0.0, 1.5),
                      temp: tuple = (0.3, 1.5), philox_seed: Optional[int] = None,
                      seq_id_base: int = 0, identical_draft: bool = False,
                      p_hit: float = 0.7) -> Batch:
    """A small mixed batch: per sequence K ~ U{k_min..kmax}, a random mode,
    T ~ U[temp], target rows ~ N(0, scale_s^2), draft = target + N(0, noise_s^2)
    (exactly the target rows when ``identical_draft``)."""
    rng = np.random.default_rng(np.random.PCG64([77, seed]))
    K = rng.integers(k_min, kmax + 1, size=B).astype(np.int32)
    mode = rng.choice(np.asarray(modes, np.uint8), size=B).astype(np.uint8)
    T = rng.uniform(temp[0], temp[1], size=B).astype(np.float32)
    sc = rng.uniform(scale[0], scale[1], size=B).astype(np.float32)
    ns = rng.uniform(noise[0], noise[1], size=B).astype(np.float32)
    if with_draft is None:
        with_draft = bool((mode == MODE_SAMPLE).any())
    n_t, n_d = int(K.sum()) + B, int(K.sum())
    sdt = np.uint16 if dtype == "bf16" else np.float32
    tgt = np.empty((n_t, V), sdt)
    dft = np.empty((n_d, V), sdt) if with_draft else None
    toks = np.empty(n_d, np.int32)
    rt = rd = 0
    for s in range(B):
        for i in range(int(K[s]) + 1):
            row = (sc[s] * rng.standard_normal(V, dtype=np.float32)).astype(np.float32)
            tgt[rt] = _store(row, dtype)
            if i < K[s]:
                t32 = _stored_as_f32(tgt[rt], dtype)
                if identical_draft:
                    d32 = t32.copy()
                else:
                    d32 = (t32 + ns[s] * rng.standard_normal(V, dtype=np.float32)).astype(np.float32)
                if with_draft:
                    dft[rd] = _store(d32, dtype)
                    d32 = _stored_as_f32(dft[rd], dtype)
                if mode[s] == MODE_SAMPLE:
                    toks[rd] = _draw_from_logits(rng, d32, float(T[s]))
                else:
                    toks[rd] = _near_argmax_token(rng, t32, p_hit)
                rd += 1
            rt += 1
    ld = V + ld_pad
    return Batch(
        name=f"random(seed={seed},B={B},V={V},kmax={kmax},{dtype})", vocab=V, dtype=dtype,
        target=_pad(tgt, ld, dtype),
        draft=_pad(dft, ld, dtype) if dft is not None else None,
        num_draft=K, draft_tokens=toks, temperature=T, mode=mode,
        seq_ids=(np.arange(B, dtype=np.uint64) + seq_id_base).astype(np.uint32),
        seed=int(seed if philox_seed is None else philox_seed),
    )


# ---------------------------------------------------------------------------
# token histories for the N-gram (prompt-lookup) proposer
# ---------------------------------------------------------------------------

@dataclass
class NgramBatch:
    name: str
    history: np.ndarray       # int32 [total_len]
    offsets: np.ndarray       # int64 [B + 1]
    min_n: int
    max_n: int
    max_tokens: int

    @property
    def batch(self) -> int:
        return len(self.offsets) - 1

    @property
    def total_len(self) -> int:
        return int(self.offsets[-1])


NGRAM_WORKLOAD = "NG: B=256 histories of U{1024..16384} tokens, V=152064 Zipf ids, half the output copied from the prompt; windows 2..4, 5 proposed tokens"


def _ngram_history(rng: np.random.Generator, L: int, vocab: int, ids: np.ndarray, p_tail_hit: float) -> np.ndarray:
    """A prompt of Zipf-distributed ids, then an output in which runs of
    fresh ids alternate with copies of 8..64-token spans of what came before;
    with probability p_tail_hit the history ends inside a copied span."""
    ranks = rng.zipf(1.2, size=L)
    h = ids[np.minimum(ranks - 1, vocab - 1)].astype(np.int32)
    pos = L // 2
    while pos < L:
        span = int(rng.integers(8, 65))
        if rng.random() < 0.5 and pos > span:
            src = int(rng.integers(0, pos - span))
            n = min(span, L - pos)
            h[pos:pos + n] = h[src:src + n]
        pos += span
    if rng.random() < p_tail_hit and L > 80:
        span = int(rng.integers(4, 16))
        src = int(rng.integers(0, L - 2 * span - 40))
        h[L - span:] = h[src:src + span]
    return h


def make_ngram_batch(seed: int, B: int = 256, min_len: int = 1024, max_len: int = 16384, vocab: int = 152064,
                     p_tail_hit: float = 0.7, min_n: int = 2, max_n: int = 4, max_tokens: int = 5,
                     lengths: Optional[Sequence[int]] = None, name: Optional[str] = None) -> NgramBatch:
    """Seeded ragged batch of histories (PCG64 seeded with (2000, seed))."""
    rng = np.random.default_rng(np.random.PCG64([2000, seed]))
    ids = rng.permutation(vocab).astype(np.int32)            # which id has which Zipf rank
    if lengths is None:
        lengths = rng.integers(min_len, max_len + 1, B)
    lengths = np.asarray(lengths, dtype=np.int64)
    parts = [_ngram_history(rng, int(L), vocab, ids, p_tail_hit) for L in lengths]
    offsets = np.concatenate(([0], np.cumsum(lengths))).astype(np.int64)
    hist = np.concatenate(parts).astype(np.int32) if len(parts) else np.zeros(0, np.int32)
    return NgramBatch(name=name or f"ngram(seed={seed},B={len(lengths)},L={min_len}..{max_len})", history=hist,
                      offsets=offsets, min_n=min_n, max_n=max_n, max_tokens=max_tokens)


def make_ngram_workload(step: int = 0) -> NgramBatch:
    return make_ngram_batch(step, name=NGRAM_WORKLOAD)


ROUNDS_WORKLOAD = ("ST: B=256 rounds per call, K ~ U{1..8}, each proposed token accepted with a per-sequence "
                   "probability beta_s ~ U[0.3, 0.95] up to the first rejection, 2% of rounds not verified; "
                   "statistics with max_k 8 and the sliding-window controller (window 100, 10 samples, target 0.7, "
                   "lengths 1..10)")


def make_rounds_workload(step: int = 0, B: int = 256, max_k: int = 8):
    """Verify-round outcomes (num_draft, accepted_len) shaped like the mixed
    C3 batch: the inputs of the acceptance statistics and the draft-length
    controllers.  A round's acceptances are drawn directly (independent
    per-position Bernoulli draws), not computed by a verify step."""
    rng = np.random.default_rng([3000, step])
    K = rng.integers(1, max_k + 1, B).astype(np.int32)
    beta = rng.uniform(0.3, 0.95, B)
    ok = rng.random((B, max_k)) < beta[:, None]
    first_no = np.where(ok.all(axis=1), max_k, np.argmin(ok, axis=1))
    A = np.minimum(first_no, K).astype(np.int32)
    A[rng.random(B) < 0.02] = -1
    return K, A
