"""Build libdspark.so for gfx950 with hipcc (in-tree, no JIT cache).

Usage: python -m semi_ar_draft_amd.build   (or call build()).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libdspark.so")
SOURCES = ["api.hip", "sweep.hip", "verify.hip", "confidence.hip", "schedule.hip", "gru.hip", "sts.hip",
           "stream.hip"]
ARCH = os.environ.get("DSPARK_OFFLOAD_ARCH", "gfx950")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 arithmetic in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [ln for ln in p.stdout.splitlines() if "packed-fp32-ops" not in ln]
    return p.returncode, "\n".join(lines)


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source for gfx950 and link libdspark.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [hipcc, *COMMON_FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
        jobs.append((src, obj, cmd))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        results = list(ex.map(lambda j: (j[0], *_run(j[2])), jobs))
    for src, rc, out in results:
        if verbose and out.strip():
            print(out)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    tmp = LIB_PATH + ".tmp"
    rc, out = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC",
                    *[j[1] for j in jobs], "-ldl", "-o", tmp])
    if rc != 0:
        raise RuntimeError(f"link failed:\n{out}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
