"""Philox4x32-10, written from its published definition.

Source: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3", SC'11, section 3 (the Philox S-box).  One round
maps the counter (x0, x1, x2, x3) and key (k0, k1) to

    (hi(M1*x2) ^ x1 ^ k0,  lo(M1*x2),  hi(M0*x0) ^ x3 ^ k1,  lo(M0*x0))

with the 32x32->64 bit products split into high and low words, and between
rounds the key is bumped by the Weyl constants (W0, W1).  Philox4x32-10 runs
ten rounds; the first uses the key as given.

Test infrastructure: part of the CPU oracle.  Python integers throughout,
plus a numpy (uint64) form for many counters at once.
"""
from __future__ import annotations

import numpy as np

MASK32 = 0xFFFFFFFF
M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9   # golden ratio, 32-bit
W1 = 0xBB67AE85   # sqrt(3) - 1, 32-bit

PURPOSE_ACCEPT = 0   # counter word 1 for the uniforms of the acceptance test
PURPOSE_SAMPLE = 1   # counter word 1 for the uniform of the final-token draw


def philox4x32_10(counter, key, rounds: int = 10):
    """One Philox4x32 block: returns the four 32-bit output words."""
    x0, x1, x2, x3 = (int(c) & MASK32 for c in counter)
    k0, k1 = (int(k) & MASK32 for k in key)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
        a = M0 * x0
        b = M1 * x2
        x0, x1, x2, x3 = ((b >> 32) ^ x1 ^ k0, b & MASK32, (a >> 32) ^ x3 ^ k1, a & MASK32)
    return x0, x1, x2, x3


def philox4x32_10_np(c0, c1, c2, c3, k0, k1, rounds: int = 10):
    """Vectorised Philox4x32-10 over numpy arrays of 32-bit values."""
    m = np.uint64(MASK32)
    x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) & m for c in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64) & m
    k1 = np.asarray(k1, dtype=np.uint64) & m
    s32 = np.uint64(32)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + np.uint64(W0)) & m
            k1 = (k1 + np.uint64(W1)) & m
        a = np.uint64(M0) * x0
        b = np.uint64(M1) * x2
        x0, x1, x2, x3 = ((b >> s32) ^ x1 ^ k0, b & m, (a >> s32) ^ x3 ^ k1, a & m)
    return x0, x1, x2, x3


def u24(word) -> float:
    """Top 24 bits of a 32-bit word as a uniform in [0, 1): exact in float32."""
    return float((int(word) >> 8)) * 2.0 ** -24


def verify_uniform(seed: int, seq_id: int, position: int, purpose: int) -> float:
    """The uniform the verify step uses at (sequence, position, purpose):
    counter = (position, purpose, seq_id, 0), key = (seed low, seed high)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    w = philox4x32_10((position, purpose, seq_id, 0), (seed & MASK32, seed >> 32))
    return u24(w[0])


def verify_uniforms_np(seed: int, seq_ids, positions, purpose: int) -> np.ndarray:
    """Vectorised ``verify_uniform`` (float64 array)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    seq_ids = np.asarray(seq_ids, dtype=np.uint64)
    positions = np.asarray(positions, dtype=np.uint64)
    shape = np.broadcast(seq_ids, positions).shape
    z = np.zeros(shape, np.uint64)
    w0, _, _, _ = philox4x32_10_np(positions + z, np.uint64(purpose) + z, seq_ids + z, z,
                                   np.uint64(seed & MASK32) + z, np.uint64(seed >> 32) + z)
    return (w0 >> np.uint64(8)).astype(np.float64) * 2.0 ** -24
