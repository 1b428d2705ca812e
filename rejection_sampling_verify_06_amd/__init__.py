"""Batched speculative-decoding verify step on AMD MI355X (gfx950).

A thin Python face of the C library ``libspec_verify.so`` (include/spec_verify.h).
Everything the verify step computes runs in the library's HIP kernels; this
module only checks tensor shapes and passes device pointers and torch's
current stream.  PyTorch supplies device memory and streams.

    v = Verifier(max_batch=256, max_k=8, max_vocab=152064)
    out = v.run(target, draft, draft_tokens, num_draft, temperature, mode, seed=step)
    out["accepted_len"], out["emitted"], out["p_at"], out["q_at"], out["status"]

If the library has not been built, every entry point raises ``LibraryMissing``:
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
from typing import Optional

from . import _lib
from ._lib import (  # noqa: F401
    SV_F32, SV_BF16, SV_SAMPLE, SV_GREEDY, SV_ONEHOT, SV_STRICT,
    SV_ST_BAD_LAYOUT, SV_ST_K_TOO_LARGE, SV_ST_BAD_MODE, SV_ST_BAD_TEMPERATURE,
    SV_ST_NO_DRAFT_LOGITS, SV_ST_BAD_TOKEN, SV_ST_NONFINITE, SV_ST_ZERO_RESIDUAL,
    KERNEL_NAMES, LibraryMissing,
    SV_ADAPT_WINDOW, SV_ADAPT_MULTIPLICATIVE, SV_ADAPT_OPTIMAL_K, SV_ADAPT_COUNT_EMITTED, SV_ADAPT_COUNT_DRAFT_ONLY,
)

__all__ = ["Verifier", "VerifyError", "verify", "propose_ngram", "NgramProposer", "AcceptanceStats",
           "DraftLengthController", "LibraryMissing", "KERNEL_NAMES"]


class VerifyError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"spec_verify error {code}: {msg}")
        self.code = code


def _check(rc: int):
    if rc != 0:
        raise VerifyError(rc, _lib.last_error())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _logits_dtype(t, torch):
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _need(t, name, dtypes, torch, numel=None, device=None):
    if t is None:
        return
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")


class Verifier:
    """One library context (device scratch sized for the given maxima)."""

    def __init__(self, max_batch: int, max_k: int, max_vocab: int, device: Optional[int] = None):
        import torch
        self._torch = torch
        self._lib = _lib.load()
        self.device = torch.cuda.current_device() if device is None else int(device)
        self.max_batch, self.max_k, self.max_vocab = int(max_batch), int(max_k), int(max_vocab)
        h = ctypes.c_void_p()
        _check(self._lib.spec_verify_create(ctypes.byref(h), self.device, self.max_batch, self.max_k,
                                            self.max_vocab))
        self._h = h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.spec_verify_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- outputs ------------------------------------------------------------
    def make_outputs(self, batch: int, total_draft: int, want_pq: bool = True, want_status: bool = True) -> dict:
        torch = self._torch
        dev = torch.device("cuda", self.device)
        return {
            "accepted_len": torch.empty(batch, dtype=torch.int32, device=dev),
            "emitted": torch.empty(total_draft + batch, dtype=torch.int32, device=dev),
            "p_at": torch.empty(total_draft, dtype=torch.float32, device=dev) if want_pq else None,
            "q_at": torch.empty(total_draft, dtype=torch.float32, device=dev) if want_pq else None,
            "status": torch.empty(batch, dtype=torch.int32, device=dev) if want_status else None,
        }

    # -- the step -------------------------------------------------------------
    def build_args(self, target, draft, draft_tokens, num_draft, temperature=None, mode=None, seq_ids=None,
                   seed: int = 0, out: Optional[dict] = None, vocab: Optional[int] = None,
                   total_draft: Optional[int] = None, top_k=None, top_p=None) -> "_lib.SpecVerifyArgs":
        """Check shapes and pack the argument struct (no device work)."""
        torch = self._torch
        dev = torch.device("cuda", self.device)
        if target.dim() != 2 or target.stride(1) != 1:
            raise ValueError("target must be 2-D with unit column stride")
        B = int(num_draft.numel())
        T = int(draft_tokens.numel()) if total_draft is None else int(total_draft)
        V = int(target.shape[1]) if vocab is None else int(vocab)
        if target.shape[0] != T + B:
            raise ValueError(f"target has {target.shape[0]} rows, expected total_draft + B = {T + B}")
        if not target.is_cuda or target.device != dev:
            raise ValueError("target must be on the context's device")
        if draft is not None and draft.numel() == 0:
            draft = None
        if draft is not None:
            if draft.dim() != 2 or draft.stride(1) != 1 or draft.shape[0] != T or not draft.is_cuda:
                raise ValueError("draft must be a 2-D device tensor [total_draft, >= vocab] with unit column stride")
        _need(draft_tokens, "draft_tokens", (torch.int32,), torch, T, dev)
        _need(num_draft, "num_draft", (torch.int32,), torch, B, dev)
        _need(temperature, "temperature", (torch.float32,), torch, B, dev)
        _need(mode, "mode", (torch.uint8,), torch, B, dev)
        _need(seq_ids, "seq_ids", (torch.int32, getattr(torch, "uint32", torch.int32)), torch, B, dev)
        _need(top_k, "top_k", (torch.int32,), torch, B, dev)
        _need(top_p, "top_p", (torch.float32,), torch, B, dev)
        if out is None:
            raise ValueError("out is required (see make_outputs)")
        _need(out["accepted_len"], "accepted_len", (torch.int32,), torch, B, dev)
        _need(out["emitted"], "emitted", (torch.int32,), torch, T + B, dev)
        _need(out.get("p_at"), "p_at", (torch.float32,), torch, T, dev)
        _need(out.get("q_at"), "q_at", (torch.float32,), torch, T, dev)
        _need(out.get("status"), "status", (torch.int32,), torch, B, dev)
        a = _lib.SpecVerifyArgs()
        a.batch = B
        a.vocab = V
        a.total_draft = T
        a.target_dtype = _logits_dtype(target, torch)
        a.draft_dtype = _logits_dtype(draft, torch) if draft is not None else SV_F32
        a.target_logits = target.data_ptr()
        a.ld_target = target.stride(0)
        a.draft_logits = _ptr(draft)
        a.ld_draft = draft.stride(0) if draft is not None else 0
        a.draft_tokens = _ptr(draft_tokens) if T > 0 else None
        a.num_draft = num_draft.data_ptr()
        a.temperature = _ptr(temperature)
        a.mode = _ptr(mode)
        a.seq_ids = _ptr(seq_ids)
        a.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
        a.accepted_len = out["accepted_len"].data_ptr()
        a.emitted_tokens = out["emitted"].data_ptr()
        a.p_at_proposal = _ptr(out.get("p_at"))
        a.q_at_proposal = _ptr(out.get("q_at"))
        a.status = _ptr(out.get("status"))
        a.top_k = _ptr(top_k)
        a.top_p = _ptr(top_p)
        return a

    def run_args(self, args: "_lib.SpecVerifyArgs", stream=None):
        """Enqueue one step from a packed argument struct on ``stream``
        (default: torch's current stream on the context's device)."""
        s = self._torch.cuda.current_stream(self.device) if stream is None else stream
        _check(self._lib.spec_verify_run(self._h, ctypes.byref(args), ctypes.c_void_p(s.cuda_stream)))

    def run(self, target, draft, draft_tokens, num_draft, temperature=None, mode=None, seq_ids=None,
            seed: int = 0, out: Optional[dict] = None, want_pq: bool = True, want_status: bool = True,
            vocab: Optional[int] = None, total_draft: Optional[int] = None, stream=None,
            top_k=None, top_p=None) -> dict:
        if out is None:
            T = int(draft_tokens.numel()) if total_draft is None else int(total_draft)
            out = self.make_outputs(int(num_draft.numel()), T, want_pq, want_status)
        args = self.build_args(target, draft, draft_tokens, num_draft, temperature, mode, seq_ids, seed, out,
                               vocab, total_draft, top_k, top_p)
        self.run_args(args, stream)
        return out

    # -- measurement hooks ------------------------------------------------------
    def timing_enable(self, max_calls: int):
        _check(self._lib.spec_verify_timing_enable(self._h, int(max_calls)))

    def timing_read(self):
        calls = ctypes.c_int32()
        ms = (ctypes.c_double * _lib.SV_NUM_KERNELS)()
        _check(self._lib.spec_verify_timing_read(self._h, ctypes.byref(calls), ms))
        return int(calls.value), dict(zip(KERNEL_NAMES, list(ms)))


_SHARED: dict = {}


def _shared_verifier(dev: int, B: int, kmax: int, V: int) -> Verifier:
    """The one context per device that ``verify`` uses.  It only grows: a
    call beyond its sizes replaces it by one sized for the larger of the old
    and the new maxima (the batch rounded up to a power of two), so a serving
    loop with varying batch sizes holds one context, not one per size."""
    v = _SHARED.get(dev)
    if v is not None and B <= v.max_batch and kmax <= v.max_k and V <= v.max_vocab:
        return v
    nb = 1
    while nb < B:
        nb *= 2
    if v is not None:
        nb, kmax, V = max(nb, v.max_batch), max(kmax, v.max_k), max(V, v.max_vocab)
        import torch
        torch.cuda.synchronize(dev)      # work queued on the old context finishes before its scratch is freed
        v.close()
        del _SHARED[dev]
    v = _SHARED[dev] = Verifier(min(nb, 4096), kmax, V, dev)
    return v


def verify(target, draft, draft_tokens, num_draft, temperature=None, mode=None, seed: int = 0,
           want_pq: bool = False, seq_ids=None, top_k=None, top_p=None, want_status: bool = True) -> dict:
    """One-shot verify step on torch's current stream: allocates the outputs
    (``p_at``/``q_at`` only with ``want_pq``, ``status`` only with
    ``want_status``) and runs the library on a per-device context that is
    reused across calls.  ``top_k`` / ``top_p`` are optional per-sequence
    filters (int32 / float32 [B])."""
    import torch
    dev = target.device.index if target.device.index is not None else torch.cuda.current_device()
    B = int(num_draft.numel())
    T = int(draft_tokens.numel())
    kmax = max(1, min(128, T))          # K_s <= total_draft: the context holds any split of it
    v = _shared_verifier(dev, max(B, 1), kmax, int(target.shape[1]))
    return v.run(target, draft, draft_tokens, num_draft, temperature, mode, seq_ids, seed, want_pq=want_pq,
                 want_status=want_status, top_k=top_k, top_p=top_p)


class NgramProposer:
    """N-gram (prompt-lookup) proposals for a ragged batch of histories
    (spec_verify_ngram_propose).  Holds only its packed argument struct, so a
    caller that reuses the output tensors can re-run it cheaply."""

    def __init__(self):
        self._lib = _lib.load()

    def make_outputs(self, batch: int, max_tokens: int, device, want_match: bool = True) -> dict:
        import torch
        return {"draft_tokens": torch.empty((batch, max_tokens), dtype=torch.int32, device=device),
                "num_draft": torch.empty(batch, dtype=torch.int32, device=device),
                "match_n": torch.empty(batch, dtype=torch.int32, device=device) if want_match else None}

    def build_args(self, history, offsets, min_n: int, max_n: int, max_tokens: int, out: dict):
        import torch
        dev = offsets.device
        B = int(offsets.numel()) - 1
        if B < 0:
            raise ValueError("offsets needs batch + 1 entries")
        _need(offsets, "offsets", (torch.int64,), torch, device=dev)
        _need(history, "history", (torch.int32,), torch, device=dev)
        _need(out["draft_tokens"], "draft_tokens", (torch.int32,), torch, B * max_tokens, dev)
        _need(out["num_draft"], "num_draft", (torch.int32,), torch, B, dev)
        _need(out.get("match_n"), "match_n", (torch.int32,), torch, B, dev)
        a = _lib.SpecVerifyNgramArgs()
        a.batch = B
        a.history = _ptr(history) if history.numel() else None
        a.hist_offsets = _ptr(offsets)
        a.total_len = int(history.numel())
        a.min_n, a.max_n, a.max_tokens = int(min_n), int(max_n), int(max_tokens)
        a.draft_tokens = _ptr(out["draft_tokens"])
        a.num_draft = _ptr(out["num_draft"])
        a.match_n = _ptr(out.get("match_n"))
        return a

    def run_args(self, args, stream=None):
        import torch
        st = stream if stream is not None else torch.cuda.current_stream()
        _check(self._lib.spec_verify_ngram_propose(ctypes.byref(args), ctypes.c_void_p(st.cuda_stream)))

    def run(self, history, offsets, min_n: int = 2, max_n: int = 4, max_tokens: int = 5, stream=None) -> dict:
        B = int(offsets.numel()) - 1
        out = self.make_outputs(B, max_tokens, offsets.device)
        self.run_args(self.build_args(history, offsets, min_n, max_n, max_tokens, out), stream)
        return out


def propose_ngram(history, offsets, min_n: int = 2, max_n: int = 4, max_tokens: int = 5) -> dict:
    """One-shot N-gram proposals: draft_tokens [B, max_tokens] (-1 padded),
    num_draft [B], match_n [B] (0: no occurrence)."""
    return NgramProposer().run(history, offsets, min_n, max_n, max_tokens)


class AcceptanceStats:
    """Acceptance counters kept on the device (spec_verify_stats_accumulate /
    spec_verify_stats_summary).  `counters` is int64 storage for the C
    interface's uint64 words; `add` queues one call's rounds, `summary`
    queues the rates into a float64 tensor."""

    def __init__(self, max_k: int, device):
        import torch
        self._lib = _lib.load()
        self.max_k = int(max_k)
        self.counters = torch.zeros(_lib.stats_words(self.max_k), dtype=torch.int64, device=device)

    def reset(self):
        self.counters.zero_()

    def add(self, num_draft, accepted_len, stream=None):
        import torch
        B = int(num_draft.numel())
        _need(num_draft, "num_draft", (torch.int32,), torch, B, self.counters.device)
        _need(accepted_len, "accepted_len", (torch.int32,), torch, B, self.counters.device)
        st = stream if stream is not None else torch.cuda.current_stream()
        _check(self._lib.spec_verify_stats_accumulate(B, self.max_k, _ptr(num_draft), _ptr(accepted_len),
                                                      _ptr(self.counters), ctypes.c_void_p(st.cuda_stream)))

    def bind(self, num_draft, accepted_len, stream=None):
        """Check the arguments once and return a callable that only queues
        the accumulation (for a caller that reuses the same tensors)."""
        import torch
        B = int(num_draft.numel())
        _need(num_draft, "num_draft", (torch.int32,), torch, B, self.counters.device)
        _need(accepted_len, "accepted_len", (torch.int32,), torch, B, self.counters.device)
        st = ctypes.c_void_p((stream if stream is not None else torch.cuda.current_stream()).cuda_stream)
        f, a = self._lib.spec_verify_stats_accumulate, (B, self.max_k, _ptr(num_draft), _ptr(accepted_len),
                                                       _ptr(self.counters), st)
        return lambda: _check(f(*a))

    def summary(self, out=None, stream=None):
        import torch
        if out is None:
            out = torch.empty(_lib.stats_summary_words(self.max_k), dtype=torch.float64, device=self.counters.device)
        _need(out, "summary", (torch.float64,), torch, _lib.stats_summary_words(self.max_k), self.counters.device)
        st = stream if stream is not None else torch.cuda.current_stream()
        _check(self._lib.spec_verify_stats_summary(self.max_k, _ptr(self.counters), _ptr(out),
                                                   ctypes.c_void_p(st.cuda_stream)))
        return out


class DraftLengthController:
    """Per-sequence draft-length controllers on the device
    (spec_verify_adapt_reset / spec_verify_adapt).  `update` takes a round's
    num_draft and accepted_len and returns the next lengths (int32 [batch]).
    `count` picks the ratio: SV_ADAPT_COUNT_EMITTED (the pages' count,
    min(A + 1, K) / K) or SV_ADAPT_COUNT_DRAFT_ONLY (A / max(K, 1))."""

    def __init__(self, batch: int, kind: int = SV_ADAPT_WINDOW, *, min_k: int = 1, max_k: int = 10,
                 window: int = 100, min_samples: int = 10, target: float = 0.7, rate: float = 0.1,
                 init_k: int = 5, device=None, count: int = SV_ADAPT_COUNT_EMITTED):
        import torch
        self._lib = _lib.load()
        dev = torch.device("cuda", 0) if device is None else torch.device(device)
        self.batch = int(batch)
        nbytes = _lib.adapt_state_bytes(self.batch, window if kind == SV_ADAPT_WINDOW else 0)
        self.state = torch.empty(max(nbytes, 16) // 8 + 1, dtype=torch.int64, device=dev)
        self.next_k = torch.empty(self.batch, dtype=torch.int32, device=dev)
        a = _lib.SpecVerifyAdaptArgs()
        a.batch, a.kind, a.min_k, a.max_k = self.batch, int(kind), int(min_k), int(max_k)
        a.window, a.min_samples, a.target, a.rate = int(window), int(min_samples), float(target), float(rate)
        a.count = int(count)
        a.state, a.next_k = _ptr(self.state), _ptr(self.next_k)
        self._args = a
        self.reset(init_k)

    def reset(self, init_k: int, stream=None):
        import torch
        st = stream if stream is not None else torch.cuda.current_stream()
        _check(self._lib.spec_verify_adapt_reset(ctypes.byref(self._args), int(init_k),
                                                 ctypes.c_void_p(st.cuda_stream)))

    def bind(self, num_draft, accepted_len, stream=None):
        """Check the arguments once and return a callable that only queues
        the update (for a caller that reuses the same tensors)."""
        import torch
        _need(num_draft, "num_draft", (torch.int32,), torch, self.batch, self.next_k.device)
        _need(accepted_len, "accepted_len", (torch.int32,), torch, self.batch, self.next_k.device)
        a = _lib.SpecVerifyAdaptArgs()
        ctypes.pointer(a)[0] = self._args
        a.num_draft, a.accepted_len = _ptr(num_draft), _ptr(accepted_len)
        st = ctypes.c_void_p((stream if stream is not None else torch.cuda.current_stream()).cuda_stream)
        f, ref = self._lib.spec_verify_adapt, ctypes.byref(a)
        return lambda: _check(f(ref, st))

    def update(self, num_draft, accepted_len, stream=None):
        import torch
        _need(num_draft, "num_draft", (torch.int32,), torch, self.batch, self.next_k.device)
        _need(accepted_len, "accepted_len", (torch.int32,), torch, self.batch, self.next_k.device)
        self._args.num_draft, self._args.accepted_len = _ptr(num_draft), _ptr(accepted_len)
        st = stream if stream is not None else torch.cuda.current_stream()
        _check(self._lib.spec_verify_adapt(ctypes.byref(self._args), ctypes.c_void_p(st.cuda_stream)))
        return self.next_k


def library_loaded_path() -> str:
    """Path of the loaded library (raises LibraryMissing if not built)."""
    _lib.load()
    return _lib.library_path()
