"""Build the HIP library (libspec_verify.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libspec_verify.so"
SOURCES = ["csrc/sv_kernels.hip", "csrc/sv_ngram.hip", "csrc/sv_stats.hip", "csrc/sv_filter.hip", "csrc/sv_noalloc.hip",
           "csrc/sv_api.cpp"]
ARCH = "gfx950"


def library_path() -> str:
    return os.path.join(HERE, LIB_NAME)


def hipcc_command(out: str) -> list:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return [
        hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 instructions are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # no implicit a*b+c fusion: the softmax merge relies on round(m*c) being
        # the same value wherever it is formed; fusion is written out as fmaf
        "-ffp-contract=off",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
        *[os.path.join(HERE, s) for s in SOURCES],
        "-o", out,
    ]


def build_library(verbose: bool = False) -> str:
    """Compile the library; returns its path.  Writes to a temporary name and
    renames, so a concurrent loader never sees a half-written file."""
    out = library_path()
    tmp = out + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = [l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
