"""Throughput of the batched speculative-decoding verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS] [--workload C3]

A step is one call of the library's verify step (row statistics, then the
acceptance scan and final draw) over one batch of a synthetic workload whose
inputs are already resident in HBM.  R distinct input sets rotate so that the 256 MB
last-level cache cannot serve repeated reads.  Prints one JSON line:

  value       verified positions per second, sum_s (K_s + 1) per step, from
              the K timed steps, run without per-kernel events after the W
              warm-up steps and an untimed settle of --settle-ms (the chip's
              clocks rise over tens of milliseconds of sustained load);
              ``warmup_ms_per_step`` is the W warm-up steps' own rate, on a
              cold chip and with the first calls' costs
  roofline    the row-statistics kernel (the dominant one): algorithmic
              bytes per launch (every streamed logit row read once) over its
              mean duration from HIP events recorded around each kernel on
              the library's stream during K further steps, against 8 TB/s;
              ``traffic`` is the HBM bytes per launch measured by rocprofv3
              FETCH_SIZE + WRITE_SIZE when a counter summary for the current
              kernel source is committed
  cpu_baseline  the float64 CPU oracle on a bounded sample of the same
              workload, single process
  configs     the other target workloads (C2 and C4 after the default C3),
              each measured the same way: its own step time, positions per
              second, row-statistics roofline and step bytes
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified positions/sec (B·(K+1) over V) + achieved HBM GB/s vs peak"
PEAK_HBM_GBPS = 8000.0
WORKLOADS = {"C0": 0, "C1": 1, "C2": 2, "C3": 3, "C4": 4, "C3S": 3, "C3F": 3, "C3P": 3, "C3K": 3, "C3D8": 3}
STRICT_WORKLOADS = {"C3S"}       # the same batches, every sequence in strict sample-match mode
# one GPU's share when the batch is split across N GPUs by sequence: the
# first B/N sequences, with their global seq_ids
SHARD_WORKLOADS = {"C3D8": 8}
# the same batches with top-k / top-p on every sequence (top-k 0: off)
FILTER_WORKLOADS = {"C3F": (50, 0.9), "C3P": (0, 0.95), "C3K": (2000, 1.0)}
NGRAM_ROTATE = 32          # 32 x ~8.6 MB of histories: more than the 256 MB last-level cache
ROTATE = {0: 64, 1: 64, 2: 6, 3: 2, 4: 6}
SETTLE_SEED0 = 1 << 30     # seeds of the untimed settle steps: apart from the warm-up's and the timed steps'
COUNTERS_FILE = os.path.join(ROOT, "profiles", "row_stats_counters.json")
NGRAM_COUNTERS_FILE = os.path.join(ROOT, "profiles", "ngram_counters.json")
KERNEL_SOURCE = os.path.join(ROOT, "rejection_sampling_verify_06_amd", "csrc", "sv_kernels.hip")
NGRAM_SOURCE = os.path.join(ROOT, "rejection_sampling_verify_06_amd", "csrc", "sv_ngram.hip")
FILTER_COUNTERS_FILE = os.path.join(ROOT, "profiles", "filter_counters.json")
FILTER_SOURCE = os.path.join(ROOT, "rejection_sampling_verify_06_amd", "csrc", "sv_filter.hip")


def kernel_source_sha(path: str = KERNEL_SOURCE) -> str:
    """Hash of a kernel source's code: comments and blank lines are left out,
    so that counters stay attached to the code they were taken on."""
    with open(path) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    lines = [re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines()]
    code = "\n".join(ln for ln in lines if ln)
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def settle(step, k0: int, torch, min_ms: float, chunk: int = 10):
    """Untimed steps after the warm-up until at least ``min_ms`` of wall time
    has passed, synchronised every ``chunk`` steps so the queue stays short.
    The GPU's clocks rise over some tens of milliseconds of sustained load and
    fall again after a few milliseconds idle; a handful of warm-up steps
    leaves a short timed region on a chip that is still ramping up, which a
    serving loop running steps back to back never sees.  Returns (steps run,
    wall ms)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(chunk):
            step(k0 + n)
            n += 1
        torch.cuda.synchronize()
    return n, round((time.perf_counter() - t0) * 1e3, 2)


def timed_warmup(step, w: int, torch):
    """The W warm-up steps, timed on their own (first calls and a cold chip
    included): ms per step, or None for W = 0."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(w):
        step(i)
    torch.cuda.synchronize()
    return round((time.perf_counter() - t0) * 1e3 / w, 5) if w else None


def make_workload_batch(workload: str, step: int):
    from workloads import make_config_batch
    b = make_config_batch(WORKLOADS[workload], step, strict=workload in STRICT_WORKLOADS)
    if workload in SHARD_WORKLOADS:
        from workloads import sequence_slice
        n = SHARD_WORKLOADS[workload]
        b = sequence_slice(b, 0, b.batch // n,
                           name=f"{b.name}; one GPU's share of {n}: sequences 0..{b.batch // n - 1}")
    if workload in FILTER_WORKLOADS:
        k, p = FILTER_WORKLOADS[workload]
        b.top_k = np.full(b.batch, k, np.int32)
        b.top_p = np.full(b.batch, p, np.float32)
        b.name += (f"; top-p {p} on every sequence" if not k else
                   (f"; top-k {k} on every sequence" if p >= 1.0 else f"; top-k {k} and top-p {p} on every sequence"))
    return b


def row_bytes(batch) -> dict:
    """Algorithmic bytes of one step: every target row, and every draft row of
    a SAMPLE sequence, read once by the row-statistics kernel; plus the final
    draw's re-read (computed from the outputs)."""
    bt = 2 if batch.dtype == "bf16" else 4
    V = batch.vocab
    K = batch.num_draft.astype(np.int64)
    sample = batch.mode == 0
    stats = int(V * bt * ((K + 1).sum() + (K[sample]).sum() * (batch.draft is not None)))
    return {"row_stats": stats}


def final_bytes(batch, accepted_len) -> dict:
    """Bytes of the final draw, from each sequence's outcome.

    read:    what this library reads — both rows at a SAMPLE rejection; one
             32 KB chunk of the target row for a bonus or one-hot draw (its
             chunk sums come from the row statistics); nothing for GREEDY.
    formula: the method's own count (the whole target row for a bonus or
             one-hot draw as well), for context.
    early_exit: a sequential scan that stops at the first rejection reads
             target rows 0..A and draft rows 0..min(A, K-1), plus the final
             rows; the dense single pass reads every row."""
    bt = 2 if batch.dtype == "bf16" else 4
    bd = bt if batch.draft is not None else 0
    V = batch.vocab
    read = formula = early = 0
    for s in range(batch.batch):
        m = int(batch.mode[s])
        A, K = int(accepted_len[s]), int(batch.num_draft[s])
        if A < 0:
            continue
        early += V * (A + 1) * bt + (V * min(A + 1, K) * bd if m == 0 else 0)
        if m == 1:
            continue
        residual = m == 0 and A < K
        read += V * (bt + bd) if residual else min(32768, V * bt)
        formula += V * bt * (2 if residual else 1)
    return {"read": read, "formula": formula, "early_exit": early + read}


def to_device(batch, torch):
    dev = torch.device("cuda", 0)

    def logits(a):
        if a is None:
            return None
        if batch.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)
    return dict(
        target=logits(batch.target), draft=logits(batch.draft),
        draft_tokens=torch.from_numpy(batch.draft_tokens).to(dev),
        num_draft=torch.from_numpy(batch.num_draft).to(dev),
        temperature=torch.from_numpy(batch.temperature).to(dev),
        mode=torch.from_numpy(batch.mode).to(dev),
        seq_ids=torch.from_numpy(batch.seq_ids.view(np.int32)).to(dev),
        top_k=None if batch.top_k is None else torch.from_numpy(batch.top_k).to(dev),
        top_p=None if batch.top_p is None else torch.from_numpy(batch.top_p).to(dev),
    )


def cpu_baseline(workload: str, budget_s: float) -> dict:
    """The CPU oracle as it stands, single process, on the sequences of step 0
    of the same workload, pass after pass with Philox seeds 0, 1, 2, ... (the
    logits stay, the draws change) until about ``budget_s`` seconds are spent."""
    import oracle
    b = make_workload_batch(workload, 0)
    off_d = np.concatenate(([0], np.cumsum(b.num_draft)[:-1])).astype(np.int64)
    off_t = off_d + np.arange(b.batch)
    done_pos = 0
    nseq = 0
    passes = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        for s in range(b.batch):
            K = int(b.num_draft[s])
            sl_t = slice(int(off_t[s]), int(off_t[s]) + K + 1)
            sl_d = slice(int(off_d[s]), int(off_d[s]) + K)
            oracle.verify_batch(target=b.target[sl_t], draft=None if b.draft is None else b.draft[sl_d],
                                dtype=b.dtype, vocab=b.vocab, num_draft=b.num_draft[s:s + 1],
                                draft_tokens=b.draft_tokens[sl_d], temperature=b.temperature[s:s + 1],
                                mode=b.mode[s:s + 1], seq_ids=b.seq_ids[s:s + 1], seed=passes,
                                top_k=None if b.top_k is None else b.top_k[s:s + 1],
                                top_p=None if b.top_p is None else b.top_p[s:s + 1])
            done_pos += K + 1
            nseq += 1
            if time.perf_counter() - t0 > budget_s:
                break
        passes += 1
    dt = time.perf_counter() - t0
    return {"value": round(done_pos / dt, 3), "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"{nseq} sequences ({done_pos} positions) in {passes} pass(es) over the {b.batch} "
                      f"sequences of step 0 with seeds 0..{passes - 1}, {dt:.1f} s, numpy float64, one process"}


def step_traffic(workload: str, ms_step: float):
    """HBM bytes of a whole step (every kernel) from the committed counter
    summary, over the step time: the metric's own GB/s; None when the
    counters were taken on another kernel source."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    with open(COUNTERS_FILE) as f:
        c = json.load(f)
    w = c.get("workloads", {}).get(workload)
    if c.get("kernel_source_sha") != kernel_source_sha() or w is None or "step_hbm_bytes" not in w:
        return None
    gbps = w["step_hbm_bytes"] / (ms_step * 1e-3) / 1e9
    return {"hbm_bytes": w["step_hbm_bytes"], "GBps": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4)}


def cpu_baseline_parallel(workload: str, budget_s: float, workers: int) -> dict:
    """The same oracle over `workers` processes, each taking every
    workers-th sequence of step 0 pass after pass until the budget is spent.
    Runs in a child interpreter that never touches the GPU."""
    import multiprocessing as mp
    with mp.get_context("fork").Pool(workers) as pool:
        res = pool.starmap(_oracle_worker, [(workload, budget_s, w, workers) for w in range(workers)])
    pos = sum(r[0] for r in res)
    wall = max(r[1] for r in res)
    return {"value": round(pos / wall, 3), "unit": "positions/s", "cores": workers, "kind": "oracle",
            "sample": f"{pos} positions of step 0 (sequences split over {workers} processes, passes with new seeds), "
                      f"{wall:.1f} s, numpy float64"}


def _oracle_worker(workload, budget_s, w, n):
    import oracle
    b = make_workload_batch(workload, 0)
    off_d = np.concatenate(([0], np.cumsum(b.num_draft)[:-1])).astype(np.int64)
    off_t = off_d + np.arange(b.batch)
    mine = list(range(w, b.batch, n)) or [w % b.batch]
    done = passes = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        for s in mine:
            K = int(b.num_draft[s])
            sl_t = slice(int(off_t[s]), int(off_t[s]) + K + 1)
            sl_d = slice(int(off_d[s]), int(off_d[s]) + K)
            oracle.verify_batch(target=b.target[sl_t], draft=None if b.draft is None else b.draft[sl_d],
                                dtype=b.dtype, vocab=b.vocab, num_draft=b.num_draft[s:s + 1],
                                draft_tokens=b.draft_tokens[sl_d], temperature=b.temperature[s:s + 1],
                                mode=b.mode[s:s + 1], seq_ids=b.seq_ids[s:s + 1], seed=passes,
                                top_k=None if b.top_k is None else b.top_k[s:s + 1],
                                top_p=None if b.top_p is None else b.top_p[s:s + 1])
            done += K + 1
            if time.perf_counter() - t0 > budget_s:
                break
        passes += 1
    return done, time.perf_counter() - t0


def run_parallel_baseline_child(workload: str, budget_s: float, workers: int):
    import subprocess
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-parallel-child", workload,
                        "--cpu-budget", str(budget_s), "--cpu-workers", str(workers)],
                       capture_output=True, text=True, timeout=budget_s * 4 + 120)
    if r.returncode != 0:
        return {"error": (r.stderr or "")[-300:]}
    return json.loads(r.stdout.strip().splitlines()[-1])


def ngram_scan_bytes(b, match_n) -> int:
    """Bytes a scan from the end of each history must read to decide, from
    the window lengths the proposer returned: when the longest window a
    history allows matched, everything from the most recent valid occurrence
    of that window up to the end; otherwise the whole history (4 bytes per
    token id)."""
    total = 0
    for i in range(b.batch):
        h = b.history[b.offsets[i]:b.offsets[i + 1]]
        L = len(h)
        nmax = min(b.max_n, (L - 1) // 2)
        n = int(match_n[i])
        if n >= 1 and n == nmax:
            last = L - 2 * n - 1                  # largest start leaving a token before the tail
            ok = np.ones(last + 1, dtype=bool)
            for j in range(n):
                ok &= h[j:j + last + 1] == h[L - n + j]
            total += 4 * (L - int(np.nonzero(ok)[0][-1]))
        else:
            total += 4 * L
    return total


def copy_calibration(torch):
    """Five plain device copies of 1 GiB: the reference kernel that scales
    the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def bench_ngram(args):
    import torch
    import rejection_sampling_verify_06_amd as sv
    from workloads import make_ngram_workload, NGRAM_WORKLOAD
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sv.library_loaded_path()
    dev = torch.device("cuda", 0)
    R = args.rotate or NGRAM_ROTATE
    t_gen = time.perf_counter()
    batches = [make_ngram_workload(i) for i in range(R)]
    gen_s = time.perf_counter() - t_gen
    prop = sv.NgramProposer()
    packed, outs = [], []
    for b in batches:
        h = torch.from_numpy(b.history).to(dev)
        o = torch.from_numpy(b.offsets).to(dev)
        out = prop.make_outputs(b.batch, b.max_tokens, dev)
        outs.append((h, o, out))
        packed.append(prop.build_args(h, o, b.min_n, b.max_n, b.max_tokens, out))

    def step(i):
        prop.run_args(packed[i % R])

    warm_ms = timed_warmup(step, args.warmup, torch)
    settled = settle(step, SETTLE_SEED0, torch, args.settle_ms)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    sets = [(args.warmup + i) % R for i in range(args.steps)]
    seqs = np.mean([batches[r].batch for r in sets])
    toks = np.mean([batches[r].total_len for r in sets])
    ms_step = elapsed * 1e3 / args.steps
    # per-launch duration: K more launches back to back between two HIP events on the stream the
    # kernel runs on (events between single launches would add their own gaps to each)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(args.steps):
        step(args.warmup + args.steps + i)
    e1.record(st)
    torch.cuda.synchronize()
    launch_ms = e0.elapsed_time(e1) / args.steps
    ev_sets = sorted(set((args.warmup + args.steps + i) % R for i in range(args.steps)))
    scan = {r: ngram_scan_bytes(batches[r], outs[r][2]["match_n"].cpu().numpy()) for r in ev_sets}
    scan_bytes = np.mean([scan[(args.warmup + args.steps + i) % R] for i in range(args.steps)])
    hist_bytes = np.mean([4 * batches[(args.warmup + args.steps + i) % R].total_len for i in range(args.steps)])
    ach = scan_bytes / (launch_ms * 1e-3) / 1e9
    if args.copy_calibration:
        copy_calibration(torch)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        b = batches[0]
        t1 = time.perf_counter()
        done = 0
        while time.perf_counter() - t1 < args.cpu_budget:
            oracle.ngram_propose_batch(b.history, b.offsets, b.min_n, b.max_n, b.max_tokens)
            done += 1
        dt = time.perf_counter() - t1
        cpu = {"value": round(done * b.batch / dt, 1), "unit": "histories/s", "cores": 1, "kind": "oracle",
               "sample": f"{done} passes over the {b.batch} histories of set 0 ({b.total_len} tokens), {dt:.1f} s, "
                         f"numpy, one process"}
    line = {
        "metric": "N-gram proposals/sec (histories searched per second)", "value": round(float(seqs / (ms_step * 1e-3)), 1),
        "unit": "histories/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int32", "data": "synthetic", "warmup_ms_per_step": warm_ms,
        "settle": {"steps": settled[0], "ms": settled[1]},
        "config": {"workload": NGRAM_WORKLOAD, "histories": int(seqs), "tokens_per_step": int(toks),
                   "rotating_input_sets": R},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(ach / PEAK_HBM_GBPS, 4),
                     "traffic": load_traffic("NG", NGRAM_COUNTERS_FILE, NGRAM_SOURCE), "kernel": "k_ngram",
                     "algorithmic_bytes_per_launch": int(scan_bytes), "history_bytes_per_launch": int(hist_bytes),
                     "mean_launch_ms": round(launch_ms, 5)},
        "cpu_baseline": cpu,
        "tokens_per_s": round(float(toks / (ms_step * 1e-3)), 1),
        "input_generation_s": round(gen_s, 1),
    }
    print(json.dumps(line), flush=True)


def bench_stats(args):
    """Acceptance statistics + sliding-window controller on C3-shaped rounds:
    one step adds a call's 256 rounds to the counters and updates every
    sequence's controller (window 100, filled before timing)."""
    import torch
    import rejection_sampling_verify_06_amd as sv
    from workloads import make_rounds_workload, ROUNDS_WORKLOAD
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sv.library_loaded_path()
    R = args.rotate or 32
    max_k, window = 8, 100
    sets = [make_rounds_workload(i) for i in range(R)]
    B = len(sets[0][0])
    dev_sets = [(torch.from_numpy(K).cuda(), torch.from_numpy(A).cuda()) for K, A in sets]
    stats = sv.AcceptanceStats(max_k, "cuda")
    ctl = sv.DraftLengthController(B, sv.SV_ADAPT_WINDOW, min_k=1, max_k=10, window=window, min_samples=10,
                                   target=0.7, init_k=5, device="cuda")

    bound = [(stats.bind(K, A), ctl.bind(K, A)) for K, A in dev_sets]

    def step(i):
        add, update = bound[i % R]
        add()
        update()

    for i in range(window):                          # fill the windows, then warm up
        step(i)
    warm_ms = timed_warmup(lambda i: step(window + i), args.warmup, torch)
    settled = settle(step, 0, torch, args.settle_ms)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    st = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        add, update = bound[i % R]
        ev[i][0].record(st)
        add()
        ev[i][1].record(st)
        update()
        ev[i][2].record(st)
    torch.cuda.synchronize()
    stats_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    adapt_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))
    valid = float(np.mean([(A >= 0).sum() for _, A in sets]))
    # algorithmic bytes: stats reads (K, A) per round and reads + writes its counters; the controller reads
    # (K, A), its header and the window entries it sums, and writes the new entry, the header and next_k
    stats_bytes = 8 * B + 2 * 8 * (8 + 3 * max_k)
    adapt_bytes = 8 * B + valid * (16 + 8 * (window - 1) + 8 + 16) + 4 * B
    ach = adapt_bytes / (adapt_ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        t1 = time.perf_counter()
        done = 0
        states = [oracle.Controller(5) for _ in range(B)]
        c = np.zeros(8 + 3 * max_k, np.uint64)
        while time.perf_counter() - t1 < args.cpu_budget:
            K, A = sets[done % R]
            oracle.acceptance_counters(K, A, max_k, into=c)
            oracle.adapt_batch(states, K, A, oracle.WINDOW, min_k=1, max_k=10, window=window, min_samples=10,
                               target=0.7)
            done += 1
        dt = time.perf_counter() - t1
        cpu = {"value": round(done * B / dt, 1), "unit": "rounds/s", "cores": 1, "kind": "oracle",
               "sample": f"{done} calls of {B} rounds (counters + window controller, windows filling from empty), "
                         f"{dt:.1f} s, numpy/Python, one process"}
    line = {
        "metric": "verify rounds/sec through acceptance statistics + draft-length controller",
        "value": round(B / (ms_step * 1e-3), 1), "unit": "rounds/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic", "warmup_ms_per_step": warm_ms,
        "settle": {"steps": settled[0], "ms": settled[1]},
        "config": {"workload": ROUNDS_WORKLOAD, "rounds_per_call": B, "rotating_input_sets": R},
        "roofline": {"bound": "hbm", "achieved": round(ach, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(ach / PEAK_HBM_GBPS, 6), "traffic": None, "kernel": "k_adapt",
                     "algorithmic_bytes_per_launch": int(adapt_bytes), "mean_launch_ms": round(adapt_ms, 5)},
        "cpu_baseline": cpu,
        "kernel_ms": {"stats_accumulate": round(stats_ms, 5), "adapt": round(adapt_ms, 5)},
        "stats_bytes_per_launch": int(stats_bytes),
    }
    print(json.dumps(line), flush=True)


def load_traffic(workload: str, path: str = COUNTERS_FILE, source: str = KERNEL_SOURCE):
    """HBM bytes per launch of the dominant kernel from a committed counter
    summary, or None when it was taken on another kernel source or another
    workload."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("kernel_source_sha") != kernel_source_sha(source):
        return None
    w = c.get("workloads", {}).get(workload)
    return None if w is None else w.get("hbm_bytes_per_launch")


def measure_verify(workload: str, args, torch, sv) -> dict:
    """Run one verify-step workload: warm up, time K steps without per-kernel
    events (five repetitions for the median), then K more steps with each
    kernel timed by the events its own dispatch records.  Returns the
    measurement fields of the JSON line and frees the workload's memory."""
    from workloads import config_description
    cfg = WORKLOADS[workload]
    # a GPU's share is an eighth of C3's bytes: enough input sets to exceed the 256 MB last-level cache
    R = args.rotate or (12 if workload in SHARD_WORKLOADS else ROTATE[cfg])

    t_gen = time.perf_counter()
    batches = [make_workload_batch(workload, i) for i in range(R)]
    dev_in = [to_device(b, torch) for b in batches]
    gen_s = time.perf_counter() - t_gen
    desc = dict(config_description(cfg))
    if workload in SHARD_WORKLOADS:
        desc["batch"] //= SHARD_WORKLOADS[workload]
    maxk = max(8, int(max(b.num_draft.max() for b in batches)))
    v = sv.Verifier(max_batch=desc["batch"], max_k=maxk, max_vocab=desc["vocab"], device=0)
    outs = [v.make_outputs(b.batch, b.total_draft, want_pq=True, want_status=True) for b in batches]
    packed = [v.build_args(d["target"], d["draft"], d["draft_tokens"], d["num_draft"], d["temperature"],
                           d["mode"], d["seq_ids"], seed=b.seed, out=o, vocab=b.vocab, top_k=d["top_k"],
                           top_p=d["top_p"])
              for b, d, o in zip(batches, dev_in, outs)]

    def step(i):
        packed[i % R].seed = i
        v.run_args(packed[i % R])

    warm_ms = timed_warmup(step, args.warmup, torch)
    settled = settle(step, SETTLE_SEED0, torch, args.settle_ms)

    def timed(k0):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(k0 + i)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    # the timed region: K steps right after the warm-up and the settle, no per-kernel events (they add gaps)
    elapsed = timed(args.warmup)
    # four more repetitions of the same K steps, for the median
    reps_ms = [timed(args.warmup + args.steps * (r + 1)) * 1e3 / args.steps for r in range(4)]

    # final-draw bytes depend on the outcome; measured on each rotating set's latest outputs (read back only
    # now, so that no host work sits between the warm-up and the timed steps)
    fin_b = []
    for r in range(R):
        fin_b.append(final_bytes(batches[r], outs[r]["accepted_len"].cpu().numpy()))
        st = outs[r]["status"].cpu().numpy()
        if (st & 127).any():
            raise RuntimeError(f"{workload} input set {r}: unexpected status bits {np.unique(st)}")
    sets_used = [(args.warmup + i) % R for i in range(args.steps)]
    pos = np.mean([batches[r].positions for r in sets_used])
    stats_bytes = np.mean([row_bytes(batches[r])["row_stats"] for r in sets_used])
    fin_bytes = np.mean([fin_b[r]["read"] for r in sets_used])
    fin_formula = np.mean([fin_b[r]["formula"] for r in sets_used])
    early_bytes = np.mean([fin_b[r]["early_exit"] for r in sets_used])
    ms_step = elapsed * 1e3 / args.steps
    value = pos * args.steps / elapsed
    reps = [ms_step] + reps_ms

    # per-kernel HIP events on the library's stream, K more steps
    events = not args.no_kernel_events
    kern = {}
    ev_ms_step = None
    if events:
        k0 = args.warmup + 5 * args.steps
        v.timing_enable(args.steps)
        ev_ms_step = timed(k0) * 1e3 / args.steps
        n, ms = v.timing_read()
        kern = {k: ms[k] / max(n, 1) for k in ms}
        v.timing_enable(0)
        ev_sets = [(k0 + i) % R for i in range(args.steps)]
        ev_stats_bytes = np.mean([row_bytes(batches[r])["row_stats"] for r in ev_sets])

    roofline = None
    if events and kern.get("row_stats", 0) > 0:
        ach = ev_stats_bytes / (kern["row_stats"] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": load_traffic(workload),
                    "kernel": "k_row_stats", "algorithmic_bytes_per_launch": int(ev_stats_bytes),
                    "mean_launch_ms": round(kern["row_stats"], 5)}

    filter_roofline = None
    if events and workload in FILTER_WORKLOADS and kern.get("filter", 0) > 0:
        # The filter's bytes depend on the rows: the bounded selection reads only
        # the segments whose maximum reaches its bound, the value table a 1/16
        # sample and the row once, the bracket search the row several times.
        # So its HBM rate comes from the counter-measured bytes per launch (when
        # the committed counters were taken on this filter source), and the
        # rate at which a filter reading each filtered row once would have to
        # stream to take the same time is reported beside it (above 8 TB/s when
        # the filter reads less than that).
        t_f = kern["filter"] * 1e-3
        traffic = load_traffic(workload, FILTER_COUNTERS_FILE, FILTER_SOURCE)
        ach = None if traffic is None else traffic / t_f / 1e9
        filter_roofline = {"bound": "hbm", "achieved": None if ach is None else round(ach, 1), "peak": PEAK_HBM_GBPS,
                           "unit": "GB/s", "frac": None if ach is None else round(ach / PEAK_HBM_GBPS, 4),
                           "traffic": traffic, "kernel": "k_filter",
                           "one_pass_bytes_per_launch": int(ev_stats_bytes),
                           "one_pass_equivalent_GBps": round(ev_stats_bytes / t_f / 1e9, 1),
                           "mean_launch_ms": round(kern["filter"], 5)}
    step_gbps = (stats_bytes + fin_bytes) / (ms_step * 1e-3) / 1e9
    res = {
        "workload": batches[0].name, "value": round(float(value), 1), "ms_per_step": round(ms_step, 5),
        "ms_per_step_median_of_5": round(float(np.median(reps)), 5),
        "warmup_ms_per_step": warm_ms,
        "settle": {"steps": settled[0], "ms": settled[1]},
        "config": {"workload": batches[0].name, "batch": desc["batch"], "k": desc["k"],
                   "vocab": desc["vocab"], "logits": desc["dtype"], "rotating_input_sets": R,
                   "positions_per_step": round(float(pos), 2)},
        "roofline": roofline,
        "step_bytes": {"row_stats": int(stats_bytes), "final_draw": int(fin_bytes),
                       "final_draw_formula": int(fin_formula), "early_exit_lower_bound": int(early_bytes),
                       "step_GBps": round(step_gbps, 1), "step_frac_of_peak": round(step_gbps / PEAK_HBM_GBPS, 4)},
        "step_traffic": step_traffic(workload, ms_step),
        "kernel_ms": {k: round(x, 5) for k, x in kern.items()},
        "filter_roofline": filter_roofline,
        "kernel_events_ms_per_step": None if ev_ms_step is None else round(ev_ms_step, 5),
        "input_generation_s": round(gen_s, 1),
    }
    v.close()
    del packed, outs, dev_in, batches
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed steps after the W warm-up steps for at least this many ms, so the timed "
                         "steps run at the clocks of sustained load (0: none)")
    ap.add_argument("--workload", default="C3", choices=sorted(WORKLOADS) + ["NG", "ST"],
                    help="C0..C4: the verify step; C3S: C3 in strict sample-match mode; C3F: C3 with top-k 50 "
                         "and top-p 0.9; C3P: C3 with top-p 0.95; C3K: C3 with top-k 2000; C3D8: one GPU's share of C3 split by sequence over 8 GPUs; "
                         "NG: the N-gram proposer; ST: acceptance statistics and the draft-length "
                         "controller")
    ap.add_argument("--also", default=None,
                    help="comma-separated verify workloads measured after the main one and reported under "
                         "'configs' (default: C2,C4 with the default C3 workload, none otherwise; '' for none)")
    ap.add_argument("--rotate", type=int, default=None, help="input sets kept resident and cycled")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=min(16, os.cpu_count() or 1),
                    help="processes for the parallel oracle baseline (0: skip it)")
    ap.add_argument("--cpu-parallel-child", default=None, help=argparse.SUPPRESS)
    ap.add_argument("--no-kernel-events", action="store_true", help="time without per-kernel HIP events")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 5 plain device copies of 1 GiB (the reference kernel for counter scaling)")
    args = ap.parse_args()
    if args.cpu_parallel_child is not None:      # child interpreter: CPU only
        print(json.dumps(cpu_baseline_parallel(args.cpu_parallel_child, args.cpu_budget, args.cpu_workers)))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus}, WORLD_SIZE {world} requested): the verify "
              f"step of a sequence-sharded batch needs no communication, so a multi-GPU run would just repeat "
              f"this line per device.", file=sys.stderr)
        sys.exit(2)

    if args.workload == "NG":
        return bench_ngram(args)
    if args.workload == "ST":
        return bench_stats(args)

    import torch
    import rejection_sampling_verify_06_amd as sv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sv.library_loaded_path()
    also = (["C2", "C4"] if args.workload == "C3" else []) if args.also is None else \
        [w for w in args.also.split(",") if w]
    for w in also:
        if w not in WORKLOADS:
            raise SystemExit(f"--also: unknown workload {w}")

    main_res = measure_verify(args.workload, args, torch, sv)
    sub = {}
    for w in also:
        r = measure_verify(w, args, torch, sv)
        sub[w] = {k: r[k] for k in ("workload", "value", "ms_per_step", "ms_per_step_median_of_5",
                                    "warmup_ms_per_step", "settle", "roofline", "step_bytes", "kernel_ms")}
        sub[w]["unit"] = "positions/s"
        sub[w]["positions_per_step"] = r["config"]["positions_per_step"]

    if args.copy_calibration:
        copy_calibration(torch)

    cpu = None if args.no_cpu_baseline else cpu_baseline(args.workload, args.cpu_budget)
    cpu_par = None if (args.no_cpu_baseline or args.cpu_workers < 1) else \
        run_parallel_baseline_child(args.workload, args.cpu_budget, args.cpu_workers)
    line = {
        "metric": METRIC, "value": main_res["value"], "unit": "positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": main_res["config"],
        "roofline": main_res["roofline"],
        "cpu_baseline": cpu,
        "ms_per_step_median_of_5": main_res["ms_per_step_median_of_5"],
        "warmup_ms_per_step": main_res["warmup_ms_per_step"],
        "settle": main_res["settle"],
        "step_bytes": main_res["step_bytes"],
        "step_traffic": main_res["step_traffic"],
        "cpu_baseline_parallel": cpu_par,
        "kernel_ms": main_res["kernel_ms"],
        "filter_roofline": main_res["filter_roofline"],
        "kernel_events_ms_per_step": main_res["kernel_events_ms_per_step"],
        "input_generation_s": main_res["input_generation_s"],
        "configs": sub,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
