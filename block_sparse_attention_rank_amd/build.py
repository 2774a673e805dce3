"""Build libsparsp.so (the C-ABI library with its gfx950 kernels) in-tree with hipcc.

    python -m block_sparse_attention_rank_amd.build [--verbose]

Each HIP translation unit is compiled to an object under ``_build/`` in parallel, then linked into
``block_sparse_attention_rank_amd/libsparsp.so``.  Always rebuilds.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsparsp.so")
SOURCES = ["api.hip", "union_compact.hip", "pack.hip", "attention.hip", "merge.hip", "permute.hip", "accounting.hip",
           "materialize.hip", "measure.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
    # packed fp32 VALU forms stay disabled: only plain scalar fp32 arithmetic is emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr).strip()
    # the host pass does not know the packed-fp32 feature name; that warning is expected
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    flags = COMMON_FLAGS + list(extra_flags or [])
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(len(jobs)) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv)
    print(path)
