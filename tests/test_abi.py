"""The C ABI without a GPU: the library loads, exports every symbol include/sparsp.h declares, and the
host-side logic (status strings, the local-set call, argument checks) behaves as documented.  No call
here reaches a kernel launch: every device entry point is called with arguments it must reject first."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_attention_rank_amd as bsa
import oracle as O
from block_sparse_attention_rank_amd import _lib
from workloads import placement_contiguous, placement_periodic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparsp.h")


MEASURE_HEADER = os.path.join(ROOT, "include", "sparsp_measure.h")


def _declared_symbols(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparsp_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = bsa.load()
    declared = _declared_symbols()
    assert set(declared) == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    measure = _declared_symbols(MEASURE_HEADER)
    assert set(measure) == set(_lib.MEASURE_EXPORTS)
    for name in measure:
        assert hasattr(lib, name), name


def test_measure_argument_checks():
    lib = bsa.load()
    E = _lib.SPARSP_ERR_INVALID
    assert lib.sparsp_clock_sampler(None, 4, 10, None) == E
    assert lib.sparsp_clock_sampler(FAKE, 1, 10, None) == E
    assert lib.sparsp_clock_sampler(FAKE, 4, 0, None) == E
    assert lib.sparsp_clock_sampler(FAKE, 1 << 20, 1 << 20, None) == E                 # unbounded run time
    assert lib.sparsp_wall_timestamp(None, None) == E
    assert lib.sparsp_wall_clock_khz(None) == E


def test_version_and_status_strings():
    lib = bsa.load()
    assert lib.sparsp_abi_version() == 7
    assert lib.sparsp_status_string(0) == b"ok"
    assert lib.sparsp_status_string(1) == b"invalid argument"
    assert lib.sparsp_status_string(2) == b"unsupported configuration"
    assert lib.sparsp_status_string(3) == b"HIP runtime error"
    assert lib.sparsp_status_string(99) == b"unknown status"


@pytest.mark.parametrize("placement", [placement_contiguous(929, 8), placement_periodic(929, 128, 3600, 8),
                                       placement_periodic(3072, 64, 6144, 8)])
def test_local_query_blocks_matches_oracle(placement):
    G = int(placement.max()) + 1
    for r in range(G):
        assert np.array_equal(bsa.local_query_blocks(placement, G, r), O.local_query_blocks(placement, r))


def test_local_query_blocks_errors():
    lib = bsa.load()
    i32p = ctypes.POINTER(ctypes.c_int32)
    P = np.array([0, 1, 2, 5], np.int32)                 # 5 is outside [0, G) for G = 4
    out = np.zeros(4, np.int32)
    n = ctypes.c_int32(-1)
    st = lib.sparsp_local_query_blocks(P.ctypes.data_as(i32p), 4, 4, 0, out.ctypes.data_as(i32p), 4, ctypes.byref(n))
    assert st == _lib.SPARSP_ERR_INVALID and b"placement" in lib.sparsp_last_error()
    P = np.array([0, 0, 0, 1], np.int32)
    st = lib.sparsp_local_query_blocks(P.ctypes.data_as(i32p), 4, 2, 0, out.ctypes.data_as(i32p), 2, ctypes.byref(n))
    assert st == _lib.SPARSP_ERR_INVALID and n.value == 3         # needed size reported
    st = lib.sparsp_local_query_blocks(P.ctypes.data_as(i32p), 4, 2, 2, out.ctypes.data_as(i32p), 4, ctypes.byref(n))
    assert st == _lib.SPARSP_ERR_INVALID


FAKE = 0x1000  # never dereferenced: every call below fails its argument check first


def _geom(**kw):
    base = dict(H=2, d=128, b=128, N=1000, G=4, r=0, Lq=2)
    base.update(kw)
    return _lib.Geometry(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(H=0), _lib.SPARSP_ERR_INVALID),
    (dict(N=0), _lib.SPARSP_ERR_INVALID),
    (dict(r=4), _lib.SPARSP_ERR_INVALID),
    (dict(r=-1), _lib.SPARSP_ERR_INVALID),
    (dict(Lq=9), _lib.SPARSP_ERR_INVALID),          # nb = 8
    (dict(d=96), _lib.SPARSP_ERR_UNSUPPORTED),
    (dict(b=32), _lib.SPARSP_ERR_UNSUPPORTED),
    (dict(G=65, r=0), _lib.SPARSP_ERR_UNSUPPORTED),
    (dict(N=128 * 16385, Lq=1), _lib.SPARSP_ERR_UNSUPPORTED),
])
def test_geometry_checks(kw, status):
    lib = bsa.load()
    g = _geom(**kw)
    assert lib.sparsp_demand_union(ctypes.byref(g), FAKE, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == status
    assert lib.sparsp_pack_kv(ctypes.byref(g), FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, None) == status
    assert lib.sparsp_block_sparse_attn(ctypes.byref(g), FAKE, FAKE, 64, FAKE, FAKE, 4, 0.1, FAKE, FAKE, None) == status
    assert lib.sparsp_last_error() != b""


def test_argument_checks():
    lib = bsa.load()
    g = _geom()
    gp = ctypes.byref(g)
    E = _lib.SPARSP_ERR_INVALID
    assert lib.sparsp_demand_union(None, FAKE, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == E
    assert lib.sparsp_demand_union(gp, FAKE, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == E      # pitch < nb
    assert lib.sparsp_demand_union(gp, FAKE, 24, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == E     # not 16-aligned
    assert lib.sparsp_demand_union(gp, FAKE + 8, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == E  # misaligned
    assert lib.sparsp_demand_union(gp, FAKE, 64, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == E
    assert lib.sparsp_pack_kv(gp, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None) == E                  # capacity
    assert lib.sparsp_pack_kv(gp, FAKE + 2, FAKE, FAKE, FAKE, FAKE, 4, FAKE, None) == E              # alignment
    assert lib.sparsp_pack_kv(gp, FAKE, None, FAKE, FAKE, FAKE, 4, FAKE, None) == E
    assert lib.sparsp_block_sparse_attn(gp, FAKE, FAKE, 64, FAKE, FAKE, 4, float("nan"), FAKE, FAKE, None) == E
    assert lib.sparsp_block_sparse_attn(gp, FAKE, FAKE, 64, FAKE, FAKE, 4, 0.0, FAKE, FAKE, None) == E
    assert lib.sparsp_block_sparse_attn(gp, FAKE, FAKE, 64, FAKE, FAKE, 4, -0.1, FAKE, FAKE, None) == E
    assert lib.sparsp_block_sparse_attn(gp, None, FAKE, 64, FAKE, FAKE, 4, 0.1, FAKE, FAKE, None) == E
    assert lib.sparsp_block_sparse_attn(gp, FAKE, FAKE, 64, FAKE, FAKE, -1, 0.1, FAKE, FAKE, None) == E
    assert b"slot_capacity" in lib.sparsp_last_error()


def test_segment_and_merge_argument_checks():
    lib = bsa.load()
    g = _geom()
    gp = ctypes.byref(g)
    E, U = _lib.SPARSP_ERR_INVALID, _lib.SPARSP_ERR_UNSUPPORTED
    for fn in (lib.sparsp_block_sparse_attn_segment, lib.sparsp_block_sparse_attn_segment_accumulate):
        assert fn(gp, FAKE, FAKE, 64, FAKE, FAKE, -1, 4, 0.1, FAKE, FAKE, None) == E          # slot_lo < 0
        assert b"slot_lo" in lib.sparsp_last_error()
        assert fn(gp, FAKE, FAKE, 64, FAKE, FAKE, 5, 4, 0.1, FAKE, FAKE, None) == E           # hi < lo
        assert fn(gp, None, FAKE, 64, FAKE, FAKE, 0, 4, 0.1, FAKE, FAKE, None) == E
        assert fn(gp, FAKE, FAKE, 64, FAKE, FAKE, 0, 4, float("inf"), FAKE, FAKE, None) == E
        assert fn(gp, FAKE, FAKE, 64, FAKE, FAKE, 0, 4, 0.1, FAKE + 4, FAKE, None) == E       # O misaligned
        assert fn(gp, FAKE, FAKE, 8, FAKE, FAKE, 0, 4, 0.1, FAKE, FAKE, None) == E            # pitch < nb
        assert fn(ctypes.byref(_geom(d=96)), FAKE, FAKE, 64, FAKE, FAKE, 0, 4, 0.1, FAKE, FAKE, None) == U
        assert fn(None, FAKE, FAKE, 64, FAKE, FAKE, 0, 4, 0.1, FAKE, FAKE, None) == E
    mp = lib.sparsp_merge_partial
    assert mp(None, FAKE, FAKE, FAKE, FAKE, None) == E
    assert mp(gp, None, FAKE, FAKE, FAKE, None) == E
    assert mp(gp, FAKE, FAKE, FAKE, None, None) == E
    assert mp(gp, FAKE, FAKE, FAKE + 8, FAKE, None) == E                                       # O_part misaligned
    assert b"aligned" in lib.sparsp_last_error()
    assert mp(ctypes.byref(_geom(b=32)), FAKE, FAKE, FAKE, FAKE, None) == U


def test_compaction_lds_limit():
    """A geometry whose compaction tables exceed 64 KiB of LDS is refused, not launched."""
    lib = bsa.load()
    g = _geom(H=64, G=64, r=0, b=64, N=64 * 16384, Lq=1)       # W = 256: 64*256*12 bytes > 64 KiB
    pitch = 16384
    assert lib.sparsp_demand_union(ctypes.byref(g), FAKE, pitch, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None) == _lib.SPARSP_ERR_UNSUPPORTED


@pytest.mark.parametrize("placement,G", [(placement_contiguous(929, 8), 8), (placement_periodic(929, 128, 3600, 8), 8),
                                         (placement_periodic(3072, 64, 6144, 8), 8),
                                         (np.random.default_rng(3).integers(0, 5, 200).astype(np.int32), 5),
                                         (np.zeros(1, np.int32), 1)])
def test_placement_permutation_matches_oracle(placement, G):
    pos, offs = bsa.placement_permutation(placement, G)
    opos, ooffs = O.placement_permutation(placement, G)
    assert np.array_equal(pos, opos) and np.array_equal(offs, ooffs)


def test_permutation_argument_checks():
    lib = bsa.load()
    i32p = ctypes.POINTER(ctypes.c_int32)
    E = _lib.SPARSP_ERR_INVALID
    P = np.array([0, 1, 3], np.int32)
    pos = np.full(3, -7, np.int32)
    offs = np.zeros(4, np.int32)
    assert lib.sparsp_placement_permutation(P.ctypes.data_as(i32p), 3, 3, pos.ctypes.data_as(i32p),
                                            offs.ctypes.data_as(i32p)) == E
    assert pos.tolist() == [-7, -7, -7]                 # nothing written on error
    assert lib.sparsp_placement_permutation(None, 3, 3, pos.ctypes.data_as(i32p), offs.ctypes.data_as(i32p)) == E
    assert lib.sparsp_placement_permutation(P.ctypes.data_as(i32p), 0, 3, pos.ctypes.data_as(i32p),
                                            offs.ctypes.data_as(i32p)) == E
    # device call: every case fails its check before a launch
    assert lib.sparsp_permute_blocks(FAKE, FAKE + 4096, 1, 4, 24, FAKE, 0, None) == E      # not a multiple of 16
    assert lib.sparsp_permute_blocks(FAKE, FAKE + 4096, 1, 4, 0, FAKE, 0, None) == E
    assert lib.sparsp_permute_blocks(FAKE, FAKE + 4096, -1, 4, 32, FAKE, 0, None) == E
    assert lib.sparsp_permute_blocks(FAKE, FAKE + 4096, 1, 0, 32, FAKE, 0, None) == E
    assert lib.sparsp_permute_blocks(FAKE + 8, FAKE + 4096, 1, 4, 32, FAKE, 0, None) == E  # misaligned
    assert lib.sparsp_permute_blocks(FAKE, FAKE, 1, 4, 32, FAKE, 0, None) == E             # in place
    assert lib.sparsp_permute_blocks(None, FAKE, 1, 4, 32, FAKE, 0, None) == E
    assert lib.sparsp_permute_blocks(FAKE, FAKE + 4096, 1, 4, 32, None, 0, None) == E
    assert lib.sparsp_permute_blocks(FAKE, FAKE + 4096, 1 << 30, 4, 32, FAKE, 0, None) == _lib.SPARSP_ERR_UNSUPPORTED
    assert lib.sparsp_permute_blocks(None, None, 0, 4, 32, None, 0, None) == _lib.SPARSP_OK  # empty: no launch


def _unions_all(mask_all, P, G, nb):
    U = np.zeros((G, mask_all.shape[0], nb), dtype=bool)
    for c in range(G):
        U[c] = O.demand_union(mask_all[:, O.local_query_blocks(P, c), :], nb)
    return U


@pytest.mark.parametrize("H,nb,G,p,seed", [(1, 16, 4, 0.2, 0), (3, 130, 8, 0.05, 1), (2, 64, 5, 0.5, 2),
                                           (2, 65, 1, 0.3, 3), (4, 200, 16, 0.02, 4)])
def test_comm_volume_matches_oracle(H, nb, G, p, seed):
    """The host accounting call against the oracle's loops, on demand words the oracle built."""
    rng = np.random.default_rng(seed)
    P = rng.integers(0, G, nb).astype(np.int32)
    mask_all = np.zeros((H, nb, 64 * (-(-nb // 64))), np.uint8)
    mask_all[:, :, :nb] = rng.random((H, nb, nb)) < p
    U = _unions_all(mask_all, P, G, nb)
    words = np.stack([O.demand_words(U[c]) for c in range(G)])
    got = bsa.comm_volume(words, P, G)
    want = O.comm_volume(U, P, G)
    for key in ("direct", "relay", "dense"):
        assert np.array_equal(got[key], want[key]), key


def test_accounting_argument_checks():
    lib = bsa.load()
    E = _lib.SPARSP_ERR_INVALID
    g = _geom()
    assert lib.sparsp_demand_counts(ctypes.byref(g), FAKE, 64, None, None) == E
    assert lib.sparsp_demand_counts(ctypes.byref(g), FAKE, 8, FAKE, None) == E          # pitch < nb
    assert lib.sparsp_demand_counts(ctypes.byref(_geom(d=96)), FAKE, 64, FAKE, None) == _lib.SPARSP_ERR_UNSUPPORTED
    i32p = ctypes.POINTER(ctypes.c_int32)
    P = np.array([0, 1, 2], np.int32)
    words = np.zeros((2, 1, 1), np.uint64)
    out = np.zeros(64, np.int64)
    args = (words.ctypes.data, 2, 1, 3, P.ctypes.data_as(i32p), out.ctypes.data, out.ctypes.data, out.ctypes.data)
    assert lib.sparsp_comm_volume(*args) == E                                            # P = 2 outside [0, 2)
    assert b"placement" in lib.sparsp_last_error()
    assert lib.sparsp_comm_volume(None, *args[1:]) == E
    assert lib.sparsp_comm_volume(words.ctypes.data, 65, 1, 3, P.ctypes.data_as(i32p), out.ctypes.data,
                                  out.ctypes.data, out.ctypes.data) == E


def test_materialize_argument_checks():
    lib = bsa.load()
    E, U = _lib.SPARSP_ERR_INVALID, _lib.SPARSP_ERR_UNSUPPORTED
    g = _geom()
    gp = ctypes.byref(g)
    assert lib.sparsp_pool_blocks(gp, FAKE, 9, None, FAKE, None) == E                 # n_blocks > nb = 8
    assert lib.sparsp_pool_blocks(gp, FAKE, -1, None, FAKE, None) == E
    assert lib.sparsp_pool_blocks(gp, None, 2, None, FAKE, None) == E
    assert lib.sparsp_pool_blocks(gp, FAKE + 4, 2, None, FAKE, None) == E              # misaligned
    assert lib.sparsp_pool_blocks(gp, None, 0, None, None, None) == _lib.SPARSP_OK      # nothing to do
    assert lib.sparsp_pool_blocks(ctypes.byref(_geom(H=70000, Lq=1)), FAKE, 2, None, FAKE, None) == U
    mm = lib.sparsp_materialize_mask
    assert mm(gp, FAKE, FAKE, 0.1, 1.5, 0, FAKE, 64, None) == E                          # tau > 1
    assert mm(gp, FAKE, FAKE, 0.1, -0.1, 0, FAKE, 64, None) == E
    assert mm(gp, FAKE, FAKE, 0.1, float("nan"), 0, FAKE, 64, None) == E
    assert mm(gp, FAKE, FAKE, 0.1, 0.5, -1, FAKE, 64, None) == E                         # k_min < 0
    assert mm(gp, FAKE, FAKE, 0.0, 0.5, 1, FAKE, 64, None) == E                          # scale
    assert mm(gp, FAKE, FAKE, 0.1, 0.5, 1, FAKE, 8, None) == E                           # pitch < nb
    assert mm(gp, None, FAKE, 0.1, 0.5, 1, FAKE, 64, None) == E
    assert mm(gp, FAKE + 4, FAKE, 0.1, 0.5, 1, FAKE, 64, None) == E                      # misaligned
    big = _geom(b=64, N=64 * 16385, Lq=1)
    assert mm(ctypes.byref(big), FAKE, FAKE, 0.1, 0.5, 1, FAKE, 16448, None) == U         # nb > 16384


def test_product_path_never_touches_the_oracle():
    """The HIP library's sources and the Python binding name nothing under oracle/ (the oracle is test
    infrastructure; the product path has no CPU fallback)."""
    pkg = os.path.join(ROOT, "block_sparse_attention_rank_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), fn
                assert "sparsp_oracle" not in text, fn
    assert "oracle" not in open(HEADER).read().lower()


def test_binding_fails_loudly_without_the_library(tmp_path):
    """With the library path pointing at nothing, loading raises instead of falling back."""
    import subprocess
    import sys
    code = ("import block_sparse_attention_rank_amd as b\n"
            "try:\n    b.load()\nexcept RuntimeError as e:\n    print('raised', 'missing' in str(e))\n")
    env = dict(os.environ, SPARSP_LIB=str(tmp_path / "nope.so"))
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True)
    assert out.stdout.strip() == "raised True", out.stdout + out.stderr


@pytest.mark.parametrize("w_kw", [dict(H=3, d=64, b=64, T=3, HW=320, G=3, r=1, density=0.5),
                                  dict(H=4, d=128, b=128, T=2, HW=700, G=4, r=2, placement="periodic", density=0.6),
                                  dict(H=7, d=64, b=64, T=4, HW=256, G=8, r=5, density_range=(0.02, 0.5)),
                                  dict(H=1, d=64, b=64, T=2, HW=192, G=1, r=0, density=0.4)])
@pytest.mark.parametrize("steady,drain", [(1, 1), (1, 2), (2, 4), (5, 99)])
def test_chunk_plan_matches_oracle(w_kw, steady, drain):
    """The host schedule call against the oracle's plan, on the oracle's compaction and access counts."""
    from workloads import custom, make_inputs
    w = custom(**w_kw)
    inp = make_inputs(w, with_qkv=False)
    U = O.demand_union(inp["mask"], w.nb)
    c = O.compact(U, inp["placement"], w.G)
    counts = O.access_counts(inp["mask"], w.nb).astype(np.int32)
    got = bsa.chunk_plan(c["seg_offsets"], counts, inp["placement"], w.G, w.r, steady, drain)
    want = O.chunk_plan(c["seg_offsets"], O.segment_tiles(inp["mask"], inp["placement"], w.G, w.nb), w.G, w.H, w.r,
                        steady, drain)
    assert got == want


def test_chunk_plan_argument_checks():
    lib = bsa.load()
    i32p = ctypes.POINTER(ctypes.c_int32)
    E = _lib.SPARSP_ERR_INVALID
    H, G, nb = 2, 2, 4
    seg = np.array([0, 1, 2, 3, 4], np.int32)
    cnt = np.ones((H, nb), np.int32)
    P = np.array([0, 0, 1, 1], np.int32)
    n = ctypes.c_int32(-1)
    buf = (_lib.Chunk * 8)()
    args = lambda **kw: dict(dict(seg=seg, cnt=cnt, P=P, G=G, H=H, nb=nb, r=0, s=1, d=2, cap=8), **kw)  # noqa: E731

    def call(a):
        return lib.sparsp_chunk_plan(a["seg"].ctypes.data_as(i32p), a["cnt"].ctypes.data_as(i32p),
                                     a["P"].ctypes.data_as(i32p), a["G"], a["H"], a["nb"], a["r"], a["s"], a["d"], buf,
                                     a["cap"], ctypes.byref(n))
    assert call(args()) == _lib.SPARSP_OK and n.value == 3        # local whole + drain of 2
    assert call(args(r=2)) == E
    assert call(args(s=0)) == E
    assert call(args(d=0)) == E
    assert call(args(G=65)) == E
    assert call(args(P=np.array([0, 0, 2, 1], np.int32))) == E and b"placement" in lib.sparsp_last_error()
    assert call(args(seg=np.array([0, 2, 1, 3, 4], np.int32))) == E
    assert call(args(cap=2)) == E and n.value == 3                  # needed size reported
    assert lib.sparsp_chunk_plan(None, cnt.ctypes.data_as(i32p), P.ctypes.data_as(i32p), G, H, nb, 0, 1, 1, buf, 8,
                                 ctypes.byref(n)) == E
    g = _geom()
    fn = lib.sparsp_block_sparse_attn_chunk_accumulate
    assert fn(ctypes.byref(g), FAKE, FAKE, 64, FAKE, FAKE, 0, 4, -1, 1, 0.1, FAKE, FAKE, None) == E   # h_lo < 0
    assert fn(ctypes.byref(g), FAKE, FAKE, 64, FAKE, FAKE, 0, 4, 1, 3, 0.1, FAKE, FAKE, None) == E    # h_hi > H
    assert b"h_lo" in lib.sparsp_last_error()
    assert fn(ctypes.byref(g), FAKE, FAKE, 64, FAKE, FAKE, 0, 4, 2, 1, 0.1, FAKE, FAKE, None) == E    # hi < lo
    assert fn(ctypes.byref(g), FAKE, FAKE, 64, FAKE, FAKE, 4, 3, 0, 1, 0.1, FAKE, FAKE, None) == E    # slots


def test_binding_checks_shapes_before_any_launch():
    """Wrong shapes of the tensors a kernel reads or writes are refused by the binding (ValueError) before the
    library is called; on this CPU-only host every tensor is a host tensor, so a shape error must come first."""
    import torch
    g = bsa.geometry(H=2, d=64, b=64, N=1000, G=4, r=1, Lq=3)       # nb = 16
    bf, f32, u8, i32 = torch.bfloat16, torch.float32, torch.uint8, torch.int32
    Q = torch.zeros((2, 3 * 64, 64), dtype=bf)
    mask = torch.zeros((2, 3, 16), dtype=u8)
    slot_of = torch.zeros((2, 16), dtype=i32)
    packed = torch.zeros((4, 2, 64 * 64), dtype=bf)
    O_ = torch.zeros((2, 3 * 64, 64), dtype=f32)
    lse = torch.zeros((2, 3 * 64), dtype=f32)

    def shape_error(fn, *a, **kw):
        with pytest.raises(ValueError, match="shape|must be \\[|pitch|slots"):
            fn(*a, **kw)

    shape_error(bsa.block_sparse_attn, g, Q, torch.zeros((2, 2, 16), dtype=u8), slot_of, packed)        # Lq rows
    shape_error(bsa.block_sparse_attn, g, Q, torch.zeros((2, 3, 8), dtype=u8), slot_of, packed)         # pitch < nb
    shape_error(bsa.block_sparse_attn, g, Q, torch.zeros((2, 3, 24), dtype=u8), slot_of, packed)        # pitch % 16
    shape_error(bsa.block_sparse_attn, g, Q, mask, slot_of, torch.zeros((4, 2, 64 * 32), dtype=bf))     # slot size
    shape_error(bsa.block_sparse_attn, g, Q, mask, slot_of, torch.zeros((4, 64 * 64), dtype=bf))        # dims
    shape_error(bsa.block_sparse_attn, g, Q, mask, slot_of, packed, out=(O_[:, :64], lse))              # O rows
    shape_error(bsa.block_sparse_attn, g, Q, mask, slot_of, packed, out=(O_, lse[:1]))                  # lse
    shape_error(bsa.block_sparse_attn_segment, g, Q, mask, slot_of, packed, 0, 5)                       # > slots
    shape_error(bsa.block_sparse_attn_segment_accumulate, g, Q, mask, slot_of, packed, 0, 2, O_[:1], lse)
    shape_error(bsa.block_sparse_attn_chunk_accumulate, g, Q, mask, slot_of, packed,
                dict(slot_lo=0, slot_hi=9, h_lo=0, h_hi=1), O_, lse)
    u = bsa.UnionResult(demand=torch.zeros((2, 1), dtype=torch.int64), seg_offsets=torch.zeros(9, dtype=i32),
                        slot_block=torch.zeros(32, dtype=i32), slot_head=torch.zeros(32, dtype=i32),
                        slot_of=slot_of)
    K = torch.zeros((2, 16 * 64, 64), dtype=bf)
    shape_error(bsa.pack_kv, g, K, K, u, out=torch.zeros((4, 2, 100), dtype=bf))
    bad_u = bsa.UnionResult(demand=u.demand, seg_offsets=torch.zeros(8, dtype=i32), slot_block=u.slot_block,
                            slot_head=u.slot_head, slot_of=slot_of)
    shape_error(bsa.pack_kv, g, K, K, bad_u)
    shape_error(bsa.demand_union, g, torch.zeros((2, 3, 8), dtype=u8), torch.zeros(16, dtype=i32))
    shape_error(bsa.demand_union, g, mask, torch.zeros(16, dtype=i32), out=bad_u)
    shape_error(bsa.demand_counts, g, torch.zeros((1, 3, 16), dtype=u8))
    shape_error(bsa.materialize_mask, g, torch.zeros((2, 3, 64), dtype=f32), torch.zeros((2, 16, 64), dtype=f32),
                0.9, 1, out=torch.zeros((2, 3, 8), dtype=u8))
    # the right shapes pass the shape checks and stop at the device check
    with pytest.raises(ValueError, match="device"):
        bsa.block_sparse_attn(g, Q, mask, slot_of, packed, out=(O_, lse))
