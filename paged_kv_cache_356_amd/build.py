"""Build libpa.so: every HIP/C++ source under csrc/ compiled for gfx950 with hipcc, then linked.

Run as ``python -m paged_kv_cache_356_amd.build`` (or through ``__graft_entry__.build()``).  Objects
go to ``_build/``; the shared library is written next to this file, where the binding loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libpa.so")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    f"--offload-arch={ARCH}",
    "-I", INCLUDE, "-I", CSRC,
    # No packed-fp32 instructions; IEEE-correct fp32 division (the fp8 encoder divides by scale).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
]


# Per-file options.  The prefill runs with the hardware's IEEE mode off (a float maximum is then
# one instruction; IEEE mode makes the compiler quiet each operand first); clang accepts that only
# with relaxed NaN handling.  The prefill tests no value for NaN (see prefill_mfma.hip).
EXTRA = {"prefill_mfma.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = ["hipcc", *COMMON, *EXTRA.get(os.path.basename(src), []), *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(8, len(srcs))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else None))
