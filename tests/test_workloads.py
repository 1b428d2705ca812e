"""CPU checks of the seeded input generators' data helpers (no method
arithmetic): a sequence slice keeps each sequence's rows, tokens and
per-sequence values, and the oracle gives the slice's sequences the same
outputs as in the whole batch (their seq_ids, hence their draws, are kept)."""
import numpy as np

import oracle
from workloads import make_random_batch, sequence_slice


def test_sequence_slice_layout_and_outputs():
    b = make_random_batch(90, B=12, V=40, kmax=5, dtype="bf16", modes=(0, 1, 2, 3))
    K = b.num_draft.astype(np.int64)
    off_d = np.concatenate(([0], np.cumsum(K)[:-1]))
    off_t = off_d + np.arange(b.batch)
    full = oracle.verify_batch_from(b)
    for lo, hi in ((0, 12), (0, 5), (5, 12), (3, 4), (7, 7)):
        s = sequence_slice(b, lo, hi)
        assert s.batch == hi - lo
        assert np.array_equal(s.seq_ids, b.seq_ids[lo:hi]) and s.seed == b.seed
        for j, q in enumerate(range(lo, hi)):
            ks = int(K[q])
            so_t = int(np.sum(s.num_draft[:j])) + j
            so_d = int(np.sum(s.num_draft[:j]))
            assert np.array_equal(s.target[so_t:so_t + ks + 1], b.target[off_t[q]:off_t[q] + ks + 1])
            assert np.array_equal(s.draft[so_d:so_d + ks], b.draft[off_d[q]:off_d[q] + ks])
            assert np.array_equal(s.draft_tokens[so_d:so_d + ks], b.draft_tokens[off_d[q]:off_d[q] + ks])
        if hi > lo:
            part = oracle.verify_batch_from(s)
            assert np.array_equal(part.accepted_len, full.accepted_len[lo:hi])
            e0, e1 = off_t[lo], (off_t[hi - 1] + K[hi - 1] + 1)
            assert np.array_equal(part.emitted, full.emitted[e0:e1])
