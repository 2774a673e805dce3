"""Child-process driver for tests/test_asan_host.py: exercises every host-side call of the library and the
argument checks of the device calls (none of which reaches a launch) against the AddressSanitizer build.
Run with LD_PRELOAD set to the sanitizer runtime and SPARSP_LIB pointing at the sanitized library."""
import ctypes
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import block_sparse_attention_rank_amd as bsa  # noqa: E402
from block_sparse_attention_rank_amd import _lib  # noqa: E402

lib = bsa.load()
assert lib.sparsp_abi_version() == 7
for st in (0, 1, 2, 3, 99):
    assert lib.sparsp_status_string(st)
rng = np.random.default_rng(5)
i32p = ctypes.POINTER(ctypes.c_int32)

# local set, permutation, accounting and chunk plan on random placements
for nb, G in ((1, 1), (16, 4), (929, 8), (3072, 8), (5000, 64)):
    P = rng.integers(0, G, nb).astype(np.int32)
    for r in (0, G - 1):
        q = bsa.local_query_blocks(P, G, r)
        assert np.array_equal(q, np.flatnonzero(P == r))
    pos, offs = bsa.placement_permutation(P, G)
    assert sorted(pos.tolist()) == list(range(nb)) and offs[-1] == nb
    H = 3
    W = -(-nb // 64)
    words = rng.integers(0, 2 ** 63, size=(G, H, W), dtype=np.int64).view(np.uint64)
    v = bsa.comm_volume(words, P, G)
    assert v["direct"].shape == (G, G)
    seg = np.concatenate([[0], np.cumsum(rng.integers(0, 5, G * H))]).astype(np.int32)
    counts = rng.integers(0, 9, (H, nb)).astype(np.int32)
    for steady, drain in ((1, 1), (2, 3), (7, 99)):
        plan = bsa.chunk_plan(seg, counts, P, G, 0, steady, drain)
        assert sum(c["slot_hi"] - c["slot_lo"] for c in plan) == int(seg[-1])

# error paths of the host calls: too small capacities, bad values, NULLs
P = np.array([0, 1, 2, 5], np.int32)
out = np.zeros(4, np.int32)
n = ctypes.c_int32(0)
assert lib.sparsp_local_query_blocks(P.ctypes.data_as(i32p), 4, 4, 0, out.ctypes.data_as(i32p), 4, ctypes.byref(n)) != 0
P = np.array([0, 0, 0, 1], np.int32)
assert lib.sparsp_local_query_blocks(P.ctypes.data_as(i32p), 4, 2, 0, out.ctypes.data_as(i32p), 2, ctypes.byref(n)) != 0
buf = (_lib.Chunk * 1)()
seg = np.array([0, 1, 2, 3, 4], np.int32)
cnt = np.ones((2, 4), np.int32)
assert lib.sparsp_chunk_plan(seg.ctypes.data_as(i32p), cnt.ctypes.data_as(i32p), P.ctypes.data_as(i32p), 2, 2, 4, 0,
                             1, 4, buf, 1, ctypes.byref(n)) != 0
assert lib.sparsp_last_error()

# device calls refused before any launch
FAKE = 0x1000
g = _lib.Geometry(2, 128, 128, 1000, 4, 0, 2)
gp = ctypes.byref(g)
assert lib.sparsp_demand_union(gp, FAKE, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) != 0
assert lib.sparsp_pack_kv(gp, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None) != 0
assert lib.sparsp_block_sparse_attn(gp, FAKE, FAKE, 64, FAKE, FAKE, 4, float("nan"), FAKE, FAKE, None) != 0
assert lib.sparsp_block_sparse_attn_chunk_accumulate(gp, FAKE, FAKE, 64, FAKE, FAKE, 0, 4, 2, 1, 0.1, FAKE, FAKE,
                                                     None) != 0
assert lib.sparsp_materialize_mask(gp, FAKE, FAKE, 0.1, 1.5, 0, FAKE, 64, None) != 0
assert lib.sparsp_clock_sampler(None, 4, 10, None) != 0
print("asan host calls ok")
