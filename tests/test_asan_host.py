"""The library's host code under AddressSanitizer (CPU only): a child process preloads the sanitizer runtime,
loads the sanitized build of the library (its device code is not instrumented) and drives every host-side call
and the argument checks of the device calls (tests/asan_host_calls.py).  Any out-of-bounds access, use after
free or double free in the host code aborts the child with a sanitizer report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_calls_under_address_sanitizer():
    from block_sparse_attention_rank_amd import build
    if not os.path.exists(build.ASAN_LIB):
        pytest.skip("the sanitized library is not built (python -m block_sparse_attention_rank_amd.build)")
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime found")
    env = dict(os.environ, LD_PRELOAD=rt, SPARSP_LIB=build.ASAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "asan_host_calls.py")], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "asan host calls ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
    assert "AddressSanitizer" not in r.stderr
