"""Helpers for the GPU tests: move a host batch to the device, run the
library through its C interface, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def logits_to_device(a, dtype: str, torch, dev, offset_elems: int = 0):
    """Copy a [rows, ld] host logits array to the device; with offset_elems > 0
    the device rows start that many elements into a larger buffer (so the base
    pointer is not 16-byte aligned)."""
    if a is None:
        return None
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if offset_elems:
        flat = torch.empty(t.numel() + offset_elems, dtype=t.dtype)
        flat[offset_elems:] = t.reshape(-1)
        d = flat.to(dev)
        return d[offset_elems:].view(t.shape)
    return t.to(dev)


def batch_to_device(batch, torch, dev=0, offset_elems: int = 0, draft_as=None):
    dev = torch.device("cuda", dev)
    draft = batch.draft
    ddtype = batch.dtype
    if draft is not None and draft_as is not None and draft_as != batch.dtype:
        from workloads import bf16_widen, bf16_round
        draft = bf16_widen(draft) if batch.dtype == "bf16" else bf16_round(draft)
        ddtype = draft_as
    return dict(
        target=logits_to_device(batch.target, batch.dtype, torch, dev, offset_elems),
        draft=logits_to_device(draft, ddtype, torch, dev, offset_elems),
        draft_tokens=torch.from_numpy(np.ascontiguousarray(batch.draft_tokens, np.int32)).to(dev),
        num_draft=torch.from_numpy(np.ascontiguousarray(batch.num_draft, np.int32)).to(dev),
        temperature=torch.from_numpy(np.ascontiguousarray(batch.temperature, np.float32)).to(dev),
        mode=torch.from_numpy(np.ascontiguousarray(batch.mode, np.uint8)).to(dev),
        seq_ids=torch.from_numpy(np.ascontiguousarray(batch.seq_ids, np.uint32).view(np.int32)).to(dev),
        top_k=None if batch.top_k is None else torch.from_numpy(np.ascontiguousarray(batch.top_k, np.int32)).to(dev),
        top_p=None if batch.top_p is None else torch.from_numpy(np.ascontiguousarray(batch.top_p, np.float32)).to(dev),
    )


def run_gpu(verifier, batch, torch, d=None, want_pq=True, seed=None, total_draft=None, **kw):
    d = d or batch_to_device(batch, torch, verifier.device)
    kw.setdefault("top_k", d.get("top_k"))
    kw.setdefault("top_p", d.get("top_p"))
    out = verifier.run(d["target"], d["draft"], d["draft_tokens"], d["num_draft"], d["temperature"], d["mode"],
                       d["seq_ids"], seed=batch.seed if seed is None else seed, vocab=batch.vocab,
                       want_pq=want_pq, total_draft=total_draft, **kw)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in out.items()}


def oracle_for(batch, max_k, draft=None, dtype=None, total_draft=None):
    return oracle.verify_batch(target=batch.target, draft=batch.draft if draft is None else draft,
                               dtype=dtype or batch.dtype, vocab=batch.vocab, num_draft=batch.num_draft,
                               draft_tokens=batch.draft_tokens, temperature=batch.temperature,
                               mode=batch.mode, seq_ids=batch.seq_ids, seed=batch.seed, max_k=max_k,
                               total_draft=total_draft, top_k=batch.top_k, top_p=batch.top_p)


def compare(ref, out):
    return oracle.compare(ref, out["accepted_len"], out["emitted"], out.get("p_at"), out.get("q_at"),
                          out.get("status"))


def assert_parity(rep, allow_degenerate=False):
    """The parity bar: every sequence identical to the oracle, or matched
    through a flagged 1e-5 near-tie; matches through a degenerate-input flag
    (q(x) < 1e-30, residual mass < 1e-6) only where a test asks for them."""
    assert rep.ok, "\n".join(rep.messages)
    if not allow_degenerate:
        assert rep.n_degenerate == 0, f"{rep.n_degenerate} sequences matched only through a degenerate-input flag"


def add_reports(tot, rep):
    """Accumulate compare reports (tot None: start from rep)."""
    if tot is None:
        return rep
    for f in ("n_seq", "n_exact", "n_exempt", "n_degenerate", "n_mismatch", "n_oracle_flagged", "n_status_z"):
        setattr(tot, f, getattr(tot, f) + getattr(rep, f))
    tot.max_pq_err = max(tot.max_pq_err, rep.max_pq_err)
    tot.messages.extend(rep.messages[:max(0, 20 - len(tot.messages))])
    return tot


def check_batch(verifier, batch, torch, label="", allow_degenerate=False, **kw):
    log(f"[gpu] {label} {batch.name}")
    out = run_gpu(verifier, batch, torch, **kw)
    ref = oracle_for(batch, verifier.max_k)
    rep = compare(ref, out)
    log(f"      {rep.summary()}")
    assert_parity(rep, allow_degenerate)
    return rep, out, ref
