"""Parity of the five workloads at full size, at the planned depth: C0 1000
steps, C1 10^4, C2 50, C3 20, C4 50, each through a context sized the way
bench.py sizes it (max_batch = B, max_k = max(8, K), max_vocab = V), so the
launch shapes are the ones it times.  Every step's outputs must be identical
to the oracle's, or matched through a flagged 1e-5 near-tie; no step may
need a degenerate-input flag.  Input generation and the oracle run in a pool
of spawned CPU processes while the device runs the steps."""
import multiprocessing as mp
import os
import time

import numpy as np
import pytest

from . import gpu_util as gu
from . import parity_jobs

pytestmark = pytest.mark.gpu

DEPTH = {0: 1000, 1: 10000, 2: 50, 3: 20, 4: 50}
WORKERS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def pool():
    with mp.get_context("spawn").Pool(WORKERS) as p:
        yield p


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_full_depth_parity(torch_mod, pool, cfg):
    import rejection_sampling_verify_06_amd as sv
    from workloads import config_description
    steps = DEPTH[cfg]
    desc = config_description(cfg)
    kmax = 8 if cfg == 3 else int(desc["k"])
    v = sv.Verifier(max_batch=desc["batch"], max_k=max(8, kmax), max_vocab=desc["vocab"], device=0)
    gu.log(f"[gpu] C{cfg}: {steps} steps, context ({desc['batch']}, {v.max_k}, {desc['vocab']}), {WORKERS} CPU workers")
    t0 = time.time()
    chunk = max(1, min(64, steps // (4 * WORKERS)))
    pending = []
    try:
        for b in pool.imap(parity_jobs.gen, [(cfg, s) for s in range(steps)], chunksize=chunk):
            out = gu.run_gpu(v, b, torch_mod)
            pending.append(pool.apply_async(parity_jobs.compare, ((cfg, len(pending), v.max_k, out),)))
            if len(pending) % max(1, steps // 10) == 0:
                gu.log(f"      device: {len(pending)} / {steps} steps ({time.time() - t0:.0f} s)")
    finally:
        v.close()
    tot = {"n_seq": 0, "n_exact": 0, "n_exempt": 0, "n_degenerate": 0, "n_mismatch": 0, "n_oracle_flagged": 0}
    max_pq, msgs = 0.0, []
    for i, p in enumerate(pending):
        r = p.get(timeout=600)
        for k in tot:
            tot[k] += r[k]
        max_pq = max(max_pq, r["max_pq_err"])
        msgs += r["messages"]
        if (i + 1) % max(1, steps // 5) == 0:
            gu.log(f"      oracle: {i + 1} / {steps} steps compared ({time.time() - t0:.0f} s)")
    gu.log(f"[gpu] C{cfg} x{steps}: seqs={tot['n_seq']} exact={tot['n_exact']} exempt={tot['n_exempt']} "
           f"degenerate={tot['n_degenerate']} mismatch={tot['n_mismatch']} flagged={tot['n_oracle_flagged']} "
           f"max|dp,dq|={max_pq:.3g} ({time.time() - t0:.0f} s)")
    assert tot["n_mismatch"] == 0, "\n".join(msgs[:20])
    assert tot["n_degenerate"] == 0
    assert tot["n_seq"] == steps * desc["batch"]
    assert max_pq <= 1e-5

