"""CPU checks of the C-ABI library: it builds, loads next to torch's HIP
runtime, exports every function the header declares, and its struct layout
and constants match the binding.  No device calls."""
import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (torch's HIP runtime must be the first one loaded, as in the binding)

from rejection_sampling_verify_06_amd import build as svbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


def _ensure_built():
    if not os.path.exists(svbuild.library_path()):
        svbuild.build_library()
    return svbuild.library_path()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_verify_[a-z_]+)\s*\(", src)))


def _header_enums():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    out = {}
    for body in re.findall(r"enum\s*\{(.*?)\}", src, flags=re.S):
        for name, val in re.findall(r"(SV_[A-Z0-9_]+)\s*=\s*(-?\d+)", body):
            out[name] = int(val)
    for name, val in re.findall(r"#define\s+(SV_[A-Z_]+)\s+(\d+)\b", src):
        out[name] = int(val)
    return out


def test_header_declares_the_core_entry_points():
    names = _declared_functions()
    for n in ("spec_verify_create", "spec_verify_run", "spec_verify_destroy", "spec_verify_last_error"):
        assert n in names


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(_ensure_built())
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_knows_every_export():
    from rejection_sampling_verify_06_amd import _lib
    assert sorted(_lib.EXPORTED) == _declared_functions()


def test_struct_layout_and_single_hip_runtime():
    _ensure_built()
    from rejection_sampling_verify_06_amd import _lib
    lib = _lib.load()                       # checks sizeof(spec_verify_args) against the binding
    assert lib.spec_verify_args_size() == ctypes.sizeof(_lib.SpecVerifyArgs) == 168   # with the two filter pointers
    assert lib.spec_verify_adapt_args_size() == ctypes.sizeof(_lib.SpecVerifyAdaptArgs) == 80
    assert b"gfx950" in lib.spec_verify_version()
    maps = open("/proc/self/maps").read()
    hip = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(hip) == 1, hip


def test_constants_match_header():
    from rejection_sampling_verify_06_amd import _lib
    import oracle
    enums = _header_enums()
    for name, val in enums.items():
        if hasattr(_lib, name):
            assert getattr(_lib, name) == val, name
    # the oracle's own copies of the interface encoding
    assert (oracle.SAMPLE, oracle.GREEDY, oracle.ONEHOT) == (enums["SV_SAMPLE"], enums["SV_GREEDY"], enums["SV_ONEHOT"])
    for o, h in (("ST_BAD_LAYOUT", "SV_ST_BAD_LAYOUT"), ("ST_K_TOO_LARGE", "SV_ST_K_TOO_LARGE"),
                 ("ST_BAD_MODE", "SV_ST_BAD_MODE"), ("ST_BAD_TEMPERATURE", "SV_ST_BAD_TEMPERATURE"),
                 ("ST_NO_DRAFT_LOGITS", "SV_ST_NO_DRAFT_LOGITS"), ("ST_BAD_TOKEN", "SV_ST_BAD_TOKEN"),
                 ("ST_NONFINITE", "SV_ST_NONFINITE"), ("ST_ZERO_RESIDUAL", "SV_ST_ZERO_RESIDUAL")):
        assert getattr(oracle, o) == enums[h], o


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from rejection_sampling_verify_06_amd import _lib
    monkeypatch.setattr(_lib, "_LIB", None)
    monkeypatch.setattr(_lib, "library_path", lambda: str(tmp_path / "nope.so"))
    with pytest.raises(_lib.LibraryMissing):
        _lib.load()


def test_package_does_not_import_the_oracle():
    """The product package never reaches for the CPU oracle."""
    pkg = os.path.join(ROOT, "rejection_sampling_verify_06_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h", ".hpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", src, flags=re.M), f
                assert "workloads" not in src or f.endswith(".md"), f


# ---- host-side argument checks that return before any HIP call (no device needed) ----

def _lib_loaded():
    _ensure_built()
    from rejection_sampling_verify_06_amd import _lib
    return _lib, _lib.load()


def test_destroy_null_and_run_without_context():
    _lib, lib = _lib_loaded()
    lib.spec_verify_destroy(None)                       # NULL is accepted
    a = _lib.SpecVerifyArgs()
    assert lib.spec_verify_run(None, ctypes.byref(a), None) == _lib.SV_ERR_INVALID
    assert b"NULL" in lib.spec_verify_last_error()
    assert lib.spec_verify_run(None, None, None) == _lib.SV_ERR_INVALID
    assert lib.spec_verify_timing_enable(None, 4) == _lib.SV_ERR_INVALID
    calls = ctypes.c_int32()
    ms = (ctypes.c_double * _lib.SV_NUM_KERNELS)()
    assert lib.spec_verify_timing_read(None, ctypes.byref(calls), ms) == _lib.SV_ERR_INVALID


@pytest.mark.parametrize("max_batch,max_k,max_vocab", [(0, 8, 1000), (4097, 8, 1000), (4, 0, 1000), (4, 129, 1000),
                                                        (4, 8, 0), (4, 8, 2097153)])
def test_create_rejects_bad_sizes(max_batch, max_k, max_vocab):
    _lib, lib = _lib_loaded()
    h = ctypes.c_void_p(12345)
    assert lib.spec_verify_create(ctypes.byref(h), 0, max_batch, max_k, max_vocab) == _lib.SV_ERR_INVALID
    assert h.value is None                              # *out is cleared on failure
    assert lib.spec_verify_last_error()
    assert lib.spec_verify_create(None, 0, 4, 8, 1000) == _lib.SV_ERR_INVALID


def test_side_entry_points_reject_bad_arguments():
    _lib, lib = _lib_loaded()
    assert lib.spec_verify_ngram_propose(None, None) == _lib.SV_ERR_INVALID
    g = _lib.SpecVerifyNgramArgs()
    g.batch, g.min_n, g.max_n, g.max_tokens = 2, 3, 2, 5       # min_n > max_n
    assert lib.spec_verify_ngram_propose(ctypes.byref(g), None) == _lib.SV_ERR_INVALID
    g.min_n, g.max_n, g.max_tokens = 1, 17, 5                   # window past the limit
    assert lib.spec_verify_ngram_propose(ctypes.byref(g), None) == _lib.SV_ERR_INVALID
    g.max_n, g.max_tokens = 4, 129
    assert lib.spec_verify_ngram_propose(ctypes.byref(g), None) == _lib.SV_ERR_INVALID
    assert lib.spec_verify_stats_accumulate(4, 0, None, None, None, None) == _lib.SV_ERR_INVALID
    assert lib.spec_verify_stats_accumulate(4, 8, None, None, None, None) == _lib.SV_ERR_INVALID
    assert lib.spec_verify_stats_summary(129, None, None, None) == _lib.SV_ERR_INVALID
    ad = _lib.SpecVerifyAdaptArgs()
    ad.batch, ad.kind, ad.min_k, ad.max_k, ad.window, ad.min_samples, ad.target, ad.rate = 0, 0, 1, 5, 10, 1, 0.7, 0.1
    ad.count = 2                                                # unknown count
    assert lib.spec_verify_adapt(ctypes.byref(ad), None) == _lib.SV_ERR_INVALID
    assert b"count" in lib.spec_verify_last_error()
    ad.count, ad.kind = 0, 3                                    # unknown kind
    assert lib.spec_verify_adapt(ctypes.byref(ad), None) == _lib.SV_ERR_INVALID
    ad.kind, ad.target = 0, 1.5
    assert lib.spec_verify_adapt_reset(ctypes.byref(ad), 5, None) == _lib.SV_ERR_INVALID
    ad.target = 0.7
    assert lib.spec_verify_adapt_reset(ctypes.byref(ad), 0, None) == _lib.SV_ERR_INVALID   # init_k
    assert lib.spec_verify_adapt(ctypes.byref(ad), None) == _lib.SV_OK                     # batch 0: nothing to do
