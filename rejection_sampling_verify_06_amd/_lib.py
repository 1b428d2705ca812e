"""ctypes view of the C interface in include/spec_verify.h (marshalling only)."""
from __future__ import annotations

import ctypes
import os

from .build import library_path

# values from include/spec_verify.h
SV_F32, SV_BF16 = 0, 1
SV_SAMPLE, SV_GREEDY, SV_ONEHOT, SV_STRICT = 0, 1, 2, 3
SV_OK, SV_ERR_INVALID, SV_ERR_NOMEM, SV_ERR_HIP, SV_ERR_CAPACITY = 0, -1, -2, -3, -4
SV_ST_BAD_LAYOUT = 1
SV_ST_K_TOO_LARGE = 2
SV_ST_BAD_MODE = 4
SV_ST_BAD_TEMPERATURE = 8
SV_ST_NO_DRAFT_LOGITS = 16
SV_ST_BAD_TOKEN = 32
SV_ST_NONFINITE = 64
SV_ST_ZERO_RESIDUAL = 128
SV_NUM_KERNELS = 4
KERNEL_NAMES = ("row_stats", "filter", "final", "select")

SV_NGRAM_MAX_N = 16
SV_NGRAM_MAX_TOKENS = 128

SV_STATS_MAX_K = 128
SV_ADAPT_WINDOW, SV_ADAPT_MULTIPLICATIVE, SV_ADAPT_OPTIMAL_K = 0, 1, 2
SV_ADAPT_COUNT_EMITTED, SV_ADAPT_COUNT_DRAFT_ONLY = 0, 1
SV_ADAPT_MAX_WINDOW = 256
SV_ADAPT_MAX_LENGTH = 4096


def stats_words(max_k: int) -> int:
    return 8 + 3 * max_k


def stats_summary_words(max_k: int) -> int:
    return 4 + 2 * max_k


def adapt_state_bytes(batch: int, window: int) -> int:
    return batch * (16 + 8 * window)

EXPORTED = (
    "spec_verify_create", "spec_verify_run", "spec_verify_destroy", "spec_verify_last_error",
    "spec_verify_timing_enable", "spec_verify_timing_read", "spec_verify_version",
    "spec_verify_args_size", "spec_verify_ngram_propose", "spec_verify_ngram_args_size",
    "spec_verify_stats_accumulate", "spec_verify_stats_summary", "spec_verify_adapt_reset", "spec_verify_adapt",
    "spec_verify_adapt_args_size", "spec_verify_run_noalloc",
)
SV_NOALLOC_SCRATCH_BYTES = 67108864


class SpecVerifyArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("vocab", ctypes.c_int64),
        ("total_draft", ctypes.c_int64),
        ("target_dtype", ctypes.c_int32),
        ("draft_dtype", ctypes.c_int32),
        ("target_logits", ctypes.c_void_p),
        ("ld_target", ctypes.c_int64),
        ("draft_logits", ctypes.c_void_p),
        ("ld_draft", ctypes.c_int64),
        ("draft_tokens", ctypes.c_void_p),
        ("num_draft", ctypes.c_void_p),
        ("temperature", ctypes.c_void_p),
        ("mode", ctypes.c_void_p),
        ("seq_ids", ctypes.c_void_p),
        ("seed", ctypes.c_uint64),
        ("accepted_len", ctypes.c_void_p),
        ("emitted_tokens", ctypes.c_void_p),
        ("p_at_proposal", ctypes.c_void_p),
        ("q_at_proposal", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
        ("top_k", ctypes.c_void_p),
        ("top_p", ctypes.c_void_p),
    ]


class SpecVerifyNgramArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("history", ctypes.c_void_p),
        ("hist_offsets", ctypes.c_void_p),
        ("total_len", ctypes.c_int64),
        ("min_n", ctypes.c_int32),
        ("max_n", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32),
        ("draft_tokens", ctypes.c_void_p),
        ("num_draft", ctypes.c_void_p),
        ("match_n", ctypes.c_void_p),
    ]


class SpecVerifyAdaptArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("kind", ctypes.c_int32),
        ("min_k", ctypes.c_int32),
        ("max_k", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("min_samples", ctypes.c_int32),
        ("count", ctypes.c_int32),
        ("target", ctypes.c_double),
        ("rate", ctypes.c_double),
        ("num_draft", ctypes.c_void_p),
        ("accepted_len", ctypes.c_void_p),
        ("state", ctypes.c_void_p),
        ("next_k", ctypes.c_void_p),
    ]


_LIB = None


class LibraryMissing(RuntimeError):
    pass


def load() -> ctypes.CDLL:
    """Load libspec_verify.so.  torch is imported first so that the library
    binds to the HIP runtime torch already loaded (one runtime per process,
    so torch's stream handles are valid in the library)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    import torch  # noqa: F401  (loads torch's HIP runtime first)
    path = library_path()
    if not os.path.exists(path):
        raise LibraryMissing(f"{path} is not built; run __graft_entry__.build() (hipcc for gfx950)")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.spec_verify_create.argtypes = [ctypes.POINTER(P), ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64]
    lib.spec_verify_create.restype = ctypes.c_int
    lib.spec_verify_run.argtypes = [P, ctypes.POINTER(SpecVerifyArgs), P]
    lib.spec_verify_run.restype = ctypes.c_int
    lib.spec_verify_run_noalloc.argtypes = [ctypes.POINTER(SpecVerifyArgs), ctypes.c_int32, P]
    lib.spec_verify_run_noalloc.restype = ctypes.c_int
    lib.spec_verify_destroy.argtypes = [P]
    lib.spec_verify_destroy.restype = None
    lib.spec_verify_last_error.argtypes = []
    lib.spec_verify_last_error.restype = ctypes.c_char_p
    lib.spec_verify_timing_enable.argtypes = [P, ctypes.c_int32]
    lib.spec_verify_timing_enable.restype = ctypes.c_int
    lib.spec_verify_timing_read.argtypes = [P, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)]
    lib.spec_verify_timing_read.restype = ctypes.c_int
    lib.spec_verify_version.argtypes = []
    lib.spec_verify_version.restype = ctypes.c_char_p
    lib.spec_verify_args_size.argtypes = []
    lib.spec_verify_args_size.restype = ctypes.c_int64
    lib.spec_verify_ngram_propose.argtypes = [ctypes.POINTER(SpecVerifyNgramArgs), P]
    lib.spec_verify_ngram_propose.restype = ctypes.c_int
    lib.spec_verify_ngram_args_size.argtypes = []
    lib.spec_verify_ngram_args_size.restype = ctypes.c_int64
    lib.spec_verify_stats_accumulate.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P, P, P]
    lib.spec_verify_stats_accumulate.restype = ctypes.c_int
    lib.spec_verify_stats_summary.argtypes = [ctypes.c_int32, P, P, P]
    lib.spec_verify_stats_summary.restype = ctypes.c_int
    lib.spec_verify_adapt_reset.argtypes = [ctypes.POINTER(SpecVerifyAdaptArgs), ctypes.c_int32, P]
    lib.spec_verify_adapt_reset.restype = ctypes.c_int
    lib.spec_verify_adapt.argtypes = [ctypes.POINTER(SpecVerifyAdaptArgs), P]
    lib.spec_verify_adapt.restype = ctypes.c_int
    lib.spec_verify_adapt_args_size.argtypes = []
    lib.spec_verify_adapt_args_size.restype = ctypes.c_int64
    if lib.spec_verify_args_size() != ctypes.sizeof(SpecVerifyArgs):
        raise RuntimeError("spec_verify_args layout differs between the library and the binding")
    if lib.spec_verify_ngram_args_size() != ctypes.sizeof(SpecVerifyNgramArgs):
        raise RuntimeError("spec_verify_ngram_args layout differs between the library and the binding")
    if lib.spec_verify_adapt_args_size() != ctypes.sizeof(SpecVerifyAdaptArgs):
        raise RuntimeError("spec_verify_adapt_args layout differs between the library and the binding")
    _LIB = lib
    return lib


def last_error() -> str:
    return load().spec_verify_last_error().decode(errors="replace")
