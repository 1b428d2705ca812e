"""CPU worker functions of the full-depth parity tests.  They run in spawned
processes that never touch the GPU: one regenerates a workload step from its
seed (the inputs the device is given), the other regenerates it again and
compares the device outputs of that step with the oracle."""
from __future__ import annotations

import oracle
from workloads import make_config_batch


def gen(job):
    cfg, step = job
    return make_config_batch(cfg, step)


def compare(job):
    cfg, step, max_k, out = job
    b = make_config_batch(cfg, step)
    ref = oracle.verify_batch_from(b, max_k=max_k)
    rep = oracle.compare(ref, out["accepted_len"], out["emitted"], out["p_at"], out["q_at"], out["status"])
    return {"step": step, "n_seq": rep.n_seq, "n_exact": rep.n_exact, "n_exempt": rep.n_exempt,
            "n_degenerate": rep.n_degenerate, "n_mismatch": rep.n_mismatch, "n_status_z": rep.n_status_z,
            "n_oracle_flagged": rep.n_oracle_flagged, "max_pq_err": rep.max_pq_err,
            "messages": [f"step {step}: {m}" for m in rep.messages[:5]]}
