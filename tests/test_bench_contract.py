"""Host-side parts of bench.py's contract, checked without a GPU: the refusal
of multi-GPU runs, the algorithmic byte counts the roofline divides by, and
the gate that detaches committed counter traffic from changed kernel code."""
import json
import os
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env=e, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("workload,B,K,V,bt,draft_rows", [
    ("C2", 32, 5, 128256, 4, True),     # every sequence SAMPLE: K draft rows each
    ("C4", 128, 5, 128256, 2, False),   # one-hot and greedy: target rows only
])
def test_row_statistics_bytes_are_one_read_of_every_row(workload, B, K, V, bt, draft_rows):
    b = bench.make_workload_batch(workload, 0)
    assert (b.batch, b.vocab) == (B, V)
    assert (b.num_draft == K).all()
    rows = B * (K + 1) + (B * K if draft_rows else 0)
    assert bench.row_bytes(b)["row_stats"] == rows * V * bt
    assert bench.row_bytes(b)["row_stats"] == {"C2": 180_584_448, "C4": 197_001_216}[workload]


def test_row_statistics_bytes_ragged():
    # ragged K, mixed modes: draft rows are counted for SAMPLE sequences only
    b = types.SimpleNamespace(dtype="bf16", vocab=1000, num_draft=np.array([3, 0, 5, 2]),
                              mode=np.array([0, 1, 0, 2]), draft=object())
    assert bench.row_bytes(b)["row_stats"] == 1000 * 2 * ((4 + 1 + 6 + 3) + (3 + 5))
    b.draft = None                      # no draft logits: target rows only
    assert bench.row_bytes(b)["row_stats"] == 1000 * 2 * (4 + 1 + 6 + 3)


def test_final_draw_bytes_per_outcome():
    V = 100_000
    b = types.SimpleNamespace(dtype="f32", vocab=V, batch=6, draft=object(),
                              num_draft=np.array([4, 4, 4, 4, 4, 4]),
                              mode=np.array([0, 0, 2, 2, 1, 0]))
    A = np.array([1, 4, 2, 4, 3, -1])   # SAMPLE reject, SAMPLE bonus, one-hot reject, one-hot bonus, greedy, failed
    fb = bench.final_bytes(b, A)
    chunk = 32768                       # one 32 KB chunk of the target row
    assert fb["read"] == V * 8 + chunk + chunk + chunk
    assert fb["formula"] == 2 * V * 4 + V * 4 + V * 4 + V * 4
    # a sequential scan reads target rows 0..A and, for SAMPLE, draft rows 0..min(A, K-1)
    early = (V * 2 * 4 + V * 2 * 4) + (V * 5 * 4 + V * 4 * 4) + V * 3 * 4 + V * 5 * 4 + V * 4 * 4
    assert fb["early_exit"] == early + fb["read"]


def test_counter_traffic_is_dropped_for_changed_kernel_code(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("// a kernel\n__global__ void k() {\n  int x = 1;  // one\n}\n")
    same = tmp_path / "k2.hip"
    same.write_text("/* other words */\n__global__ void k() {\n\n  int x = 1;\n}\n")
    other = tmp_path / "k3.hip"
    other.write_text("__global__ void k() {\n  int x = 2;\n}\n")
    sha = bench.kernel_source_sha(str(src))
    assert bench.kernel_source_sha(str(same)) == sha          # comments and blank lines do not count
    assert bench.kernel_source_sha(str(other)) != sha
    cnt = tmp_path / "c.json"
    cnt.write_text(json.dumps({"kernel_source_sha": sha, "workloads": {"C3": {"hbm_bytes_per_launch": 123}}}))
    assert bench.load_traffic("C3", str(cnt), str(src)) == 123
    assert bench.load_traffic("C3", str(cnt), str(same)) == 123
    assert bench.load_traffic("C3", str(cnt), str(other)) is None
    assert bench.load_traffic("C2", str(cnt), str(src)) is None
    assert bench.load_traffic("C3", str(tmp_path / "missing.json"), str(src)) is None

