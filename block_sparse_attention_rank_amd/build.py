"""Build libsparsp.so (the C-ABI library with its gfx950 kernels) in-tree with hipcc.

    python -m block_sparse_attention_rank_amd.build [--verbose] [--no-asan]

Each HIP translation unit is compiled to an object under ``_build/`` in parallel, then linked into
``block_sparse_attention_rank_amd/libsparsp.so``.  A second copy whose host code is built with
AddressSanitizer (the device code is not instrumented) goes to ``_build/asan/libsparsp_asan.so``; the CPU
tests load it into a child process to check the host-side calls.  Always rebuilds.
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
ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libsparsp_asan.so")
# host code only: every sanitizer flag is scoped to the host pass
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g", "-O1"]
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


def build_asan(verbose: bool = False) -> str:
    """The library with AddressSanitizer on its host code (argument checks, the host calls)."""
    cc = hipcc()
    os.makedirs(ASAN_DIR, exist_ok=True)
    flags = [f for f in COMMON_FLAGS if f != "-O3"] + ASAN_FLAGS
    objs, jobs = [], []
    for src in SOURCES:
        obj = os.path.join(ASAN_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(len(jobs)) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    tmp = ASAN_LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address", "-o", tmp, *objs],
         verbose)
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


def asan_runtime() -> str | None:
    """Path of the compiler's AddressSanitizer runtime (to preload into a process that loads ASAN_LIB)."""
    for cand in ("/opt/rocm/llvm/bin/clang", shutil.which("clang") or ""):
        if cand and os.path.exists(cand):
            res = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            path = res.stdout.strip()
            if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    return None


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv)
    print(path)
    if "--no-asan" not in sys.argv:
        print(build_asan(verbose="--verbose" in sys.argv))
