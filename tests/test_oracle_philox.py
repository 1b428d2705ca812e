"""Pins of the oracle's Philox4x32-10 and of the 24-bit uniforms built on it."""
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle.philox import (philox4x32_10, philox4x32_10_np, u24, verify_uniform,
                           verify_uniforms_np, PURPOSE_ACCEPT, PURPOSE_SAMPLE)

HERE = os.path.dirname(os.path.abspath(__file__))


def _kat_rows():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                w = [int(x, 16) for x in line.split()]
                rows.append((tuple(w[0:4]), tuple(w[4:6]), tuple(w[6:10])))
    return rows


def test_known_answer_vectors():
    rows = _kat_rows()
    assert len(rows) == 3
    for ctr, key, want in rows:
        assert philox4x32_10(ctr, key) == want


def test_numpy_form_matches_scalar_form():
    rng = np.random.default_rng(5)
    c = rng.integers(0, 2**32, size=(6, 500), dtype=np.uint64)
    out = philox4x32_10_np(*c)
    for j in range(500):
        want = philox4x32_10(c[0:4, j], c[4:6, j])
        assert tuple(int(o[j]) for o in out) == want


def _torch_header():
    try:
        import torch
    except Exception:
        return None
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    return inc if os.path.exists(os.path.join(inc, "ATen", "core", "PhiloxRNGEngine.h")) else None


@pytest.mark.skipif(shutil.which("g++") is None or _torch_header() is None,
                    reason="needs g++ and PyTorch's Philox header")
def test_against_pytorch_philox_engine(tmp_path):
    """An independent implementation: PyTorch's open-source at::philox_engine,
    compiled here with g++ from its header."""
    exe = tmp_path / "tp"
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", _torch_header(),
                    os.path.join(HERE, "philox_ref", "torch_philox_dump.cpp"), "-o", str(exe)],
                   check=True, capture_output=True)
    rng = np.random.default_rng(11)
    c = rng.integers(0, 2**32, size=(2000, 6), dtype=np.uint64)
    c[:50, 0] = 0xFFFFFFFF            # counter-word carries inside the engine's offset math
    c[50:100, 0:2] = 0
    inp = "\n".join(" ".join(str(int(v)) for v in row) for row in c) + "\n"
    out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
    for row, line in zip(c, out):
        got = tuple(int(x) for x in line.split())
        assert got == philox4x32_10(row[0:4], row[4:6])


def test_verify_uniform_layout():
    """The uniform at (seed, seq, position, purpose) is word 0 of the block
    with counter (position, purpose, seq, 0) and key (seed lo, seed hi)."""
    seed = 0x0123456789ABCDEF
    w = philox4x32_10((7, PURPOSE_SAMPLE, 42, 0), (0x89ABCDEF, 0x01234567))[0]
    assert verify_uniform(seed, 42, 7, PURPOSE_SAMPLE) == (w >> 8) / 2**24
    got = verify_uniforms_np(seed, np.array([42, 43]), np.array([7, 7]), PURPOSE_SAMPLE)
    assert got[0] == verify_uniform(seed, 42, 7, PURPOSE_SAMPLE)
    assert got[1] == verify_uniform(seed, 43, 7, PURPOSE_SAMPLE)
    assert verify_uniform(seed, 42, 7, PURPOSE_ACCEPT) != verify_uniform(seed, 42, 7, PURPOSE_SAMPLE)


def test_u24_grid():
    assert u24(0) == 0.0
    assert u24(0xFFFFFFFF) == 1.0 - 2.0 ** -24
    assert u24(0x00000100) == 2.0 ** -24
    u = verify_uniforms_np(3, np.arange(10000), 0, PURPOSE_ACCEPT)
    assert ((u * 2**24) == np.floor(u * 2**24)).all()
    assert (u >= 0).all() and (u < 1).all()
    assert (u.astype(np.float32).astype(np.float64) == u).all()   # exact in float32


def test_u24_uniformity_chi_square():
    u = verify_uniforms_np(0, np.arange(1_000_000) % 4096, np.arange(1_000_000) // 4096, PURPOSE_ACCEPT)
    counts = np.bincount((u * 256).astype(np.int64), minlength=256)
    assert stats.chisquare(counts).pvalue > 1e-4
    # serial pairs: consecutive positions of one sequence are independent
    pairs = (u[:-1] * 16).astype(int) * 16 + (u[1:] * 16).astype(int)
    assert stats.chisquare(np.bincount(pairs, minlength=256)).pvalue > 1e-4
