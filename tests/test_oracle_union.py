"""Pins for the oracle's demand union, compaction and pack (CPU only).

Each check compares the oracle with something other than itself: brute-force enumeration, special cases
whose answer is known in closed form, the half-width bound of the periodic placement, and the worked
example of the demand-directed routing figure.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O
from workloads import custom, make_inputs, placement_contiguous, placement_periodic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_mask(rng, H, Lq, nb, p):
    pitch = 64 * (-(-nb // 64))
    m = np.zeros((H, Lq, pitch), np.uint8)
    m[:, :, :nb] = rng.random((H, Lq, nb)) < p
    return m


# ---------------------------------------------------------------------------------------------- union


@settings(max_examples=60, deadline=None)
@given(H=st.integers(1, 3), Lq=st.integers(0, 9), nb=st.integers(1, 150), p=st.floats(0, 1),
       seed=st.integers(0, 2**31 - 1))
def test_union_matches_bruteforce(H, Lq, nb, p, seed):
    rng = np.random.default_rng(seed)
    mask = _random_mask(rng, H, Lq, nb, p)
    U = O.demand_union(mask, nb)
    sets = O.demand_union_sets(mask, nb)
    for h in range(H):
        assert set(np.flatnonzero(U[h]).tolist()) == sets[h]
    words = O.demand_words(U)
    for h in range(H):
        for j in range(nb):
            assert bool((int(words[h, j // 64]) >> (j % 64)) & 1) == (j in sets[h])
        # bits past nb are zero
        if nb % 64:
            assert int(words[h, -1]) >> (nb % 64) == 0


def test_union_is_per_head_not_across_heads():
    """Section 5.2: demand is kept per head.  Two heads with disjoint selections keep disjoint unions."""
    nb = 8
    mask = np.zeros((2, 1, 64), np.uint8)
    mask[0, 0, [0, 1]] = 1
    mask[1, 0, [6, 7]] = 1
    U = O.demand_union(mask, nb)
    assert np.flatnonzero(U[0]).tolist() == [0, 1]
    assert np.flatnonzero(U[1]).tolist() == [6, 7]


def test_union_ignores_pitch_padding():
    nb = 10
    mask = np.zeros((1, 2, 64), np.uint8)
    mask[0, 0, 3] = 1
    mask[0, 1, 40] = 1          # past nb: not a block
    assert np.flatnonzero(O.demand_union(mask, nb)[0]).tolist() == [3]


# ---------------------------------------------------------------------------------------------- compaction


@settings(max_examples=60, deadline=None)
@given(H=st.integers(1, 3), Lq=st.integers(0, 6), nb=st.integers(1, 100), G=st.integers(1, 8),
       p=st.floats(0, 1), periodic=st.booleans(), seed=st.integers(0, 2**31 - 1))
def test_compaction_matches_bruteforce(H, Lq, nb, G, p, periodic, seed):
    rng = np.random.default_rng(seed)
    mask = _random_mask(rng, H, Lq, nb, p)
    P = placement_periodic(nb, 64, 64 * max(1, nb // 3), G) if periodic else placement_contiguous(nb, G)
    U = O.demand_union(mask, nb)
    c = O.compact(U, P, G)
    cb = O.compact_bruteforce(O.demand_union_sets(mask, nb), P, G, nb)
    for key in ("seg_offsets", "slot_block", "slot_head", "slot_of"):
        assert np.array_equal(c[key], cb[key]), key
    _check_compaction_invariants(c, U, P, G)


def _check_compaction_invariants(c, U, P, G):
    H, nb = U.shape
    seg, sb, sh, so = c["seg_offsets"], c["slot_block"], c["slot_head"], c["slot_of"]
    assert seg[0] == 0 and seg[-1] == c["S"] == int(U.sum())
    assert np.all(np.diff(seg) >= 0)
    for p in range(G):
        for h in range(H):
            lo, hi = seg[p * H + h], seg[p * H + h + 1]
            assert np.all(sh[lo:hi] == h)
            assert np.all(P[sb[lo:hi]] == p)
            assert np.all(np.diff(sb[lo:hi]) > 0)
            assert hi - lo == int((U[h] & (P == p)).sum())
    if c["S"]:
        assert np.array_equal(so[sh, sb], np.arange(c["S"]))
    assert int((so >= 0).sum()) == c["S"]
    assert np.all(so[~U] == -1)


@pytest.mark.parametrize("kind", ["ones", "identity", "zeros"])
def test_compaction_special_cases(kind):
    """All-ones: every block demanded, S = H*nb.  Identity: only the rank's own blocks, so every segment
    of another source rank is empty.  All-zero: nothing demanded."""
    w = custom(H=3, T=4, HW=256, b=64, G=4, r=1, mask_kind=kind)
    inp = make_inputs(w, with_qkv=False)
    U = O.demand_union(inp["mask"], w.nb)
    c = O.compact(U, inp["placement"], w.G)
    seg = c["seg_offsets"]
    if kind == "ones":
        assert c["S"] == w.H * w.nb
    elif kind == "identity":
        for h in range(w.H):
            assert np.flatnonzero(U[h]).tolist() == inp["q_blocks"].tolist()
        for p in range(w.G):
            lo, hi = O.segment_range(seg, w.H, p)
            assert (hi - lo == 0) == (p != w.r)
    else:
        assert c["S"] == 0 and np.all(c["slot_of"] == -1)
    _check_compaction_invariants(c, U, inp["placement"], w.G)


def test_local_query_blocks():
    P = placement_periodic(929, 128, 3600, 8)
    q = O.local_query_blocks(P, 0)
    assert len(q) == 121 and np.all(np.diff(q) > 0) and np.all(P[q] == 0)
    assert sum(len(O.local_query_blocks(P, r)) for r in range(8)) == 929


def _multidiagonal_demand(P, G, T, B, r, delta):
    """Remote demand of rank r under a pure multi-diagonal mask: query (t, s) selects every (t', s')
    with |s - s'| <= delta, in every frame t'."""
    nb = T * B
    q = O.local_query_blocks(P, r)
    s_of = np.arange(nb) % B
    mask = np.zeros((1, len(q), 64 * (-(-nb // 64))), np.uint8)
    mask[0, :, :nb] = np.abs(s_of[q][:, None] - s_of[None, :]) <= delta
    U = O.demand_union(mask, nb)
    c = O.compact(U, P, G)
    lo, hi = O.segment_range(c["seg_offsets"], 1, r)
    return c["S"] - (hi - lo), len(q)


@pytest.mark.parametrize("delta", [1, 2, 3])
def test_periodic_placement_halo_bound(delta):
    """Section 4.3: with B/G spatial positions per rank, replicated over T frames, a rank's remote
    demand under the multi-diagonal model is the 2*delta*T halo (delta*T for the two end ranks, whose
    interval touches the frame edge).  The contiguous partition of the same mask, whose ranks each
    cover every spatial position, needs every block it does not own."""
    T, B, G, b = 6, 24, 4, 64
    nb = T * B
    Pp = placement_periodic(nb, b, B * b, G)
    Pc = placement_contiguous(nb, G)
    for r in range(G):
        remote, _ = _multidiagonal_demand(Pp, G, T, B, r, delta)
        assert remote == (delta * T if r in (0, G - 1) else 2 * delta * T)
        remote_c, Lq = _multidiagonal_demand(Pc, G, T, B, r, delta)
        assert remote_c == nb - Lq


def test_fig9_direct_delivery_golden():
    g = json.load(open(os.path.join(GOLDEN, "fig9_direct_delivery.json")))
    G, nb = g["G"], g["nb"]
    P = placement_contiguous(nb, G)
    assert O.local_query_blocks(P, 0).tolist() == [g["block_names"][n] for n in "ABCD"]
    sent = 0
    for consumer, names in g["demand_from_rank0"].items():
        r = int(consumer)
        q = O.local_query_blocks(P, r)
        mask = np.zeros((1, len(q), 64), np.uint8)
        mask[0, np.arange(len(q)), q] = 1                 # own diagonal blocks
        for n in names:
            mask[0, 0, g["block_names"][n]] = 1           # the first local row selects the named block
        c = O.compact(O.demand_union(mask, nb), P, G)
        lo, hi = O.segment_range(c["seg_offsets"], 1, 0)
        assert c["slot_block"][lo:hi].tolist() == g["expected_segment_p0_blocks"][consumer]
        sent += hi - lo
    assert sent == g["expected_blocks_sent_by_rank0"]


def test_compaction_invariants_full_configs():
    for name in ("hunyuan", "wan", "ltx"):
        inp = make_inputs(name, with_qkv=False)
        w = inp["workload"]
        U = O.demand_union(inp["mask"], w.nb)
        c = O.compact(U, inp["placement"], w.G)
        _check_compaction_invariants(c, U, inp["placement"], w.G)


# ---------------------------------------------------------------------------------------------- pack


def test_pack_matches_block_view():
    w = custom(H=2, d=64, T=3, HW=160, b=64, G=3, density=0.5)
    inp = make_inputs(w)
    U = O.demand_union(inp["mask"], w.nb)
    c = O.compact(U, inp["placement"], w.G)
    packed = O.pack(inp["K"], inp["V"], c["slot_block"], c["slot_head"], w.b)
    Kb = inp["K"].reshape(w.H, w.nb, w.b, w.d)
    Vb = inp["V"].reshape(w.H, w.nb, w.b, w.d)
    expect_k = Kb[c["slot_head"], c["slot_block"]].reshape(c["S"], -1)
    expect_v = np.swapaxes(Vb[c["slot_head"], c["slot_block"]], 1, 2).reshape(c["S"], -1)
    assert np.array_equal(packed[:, 0], expect_k)
    assert np.array_equal(packed[:, 1], expect_v)
    # the zero tail of the padded last block travels as zeros
    last = np.flatnonzero(c["slot_block"] == w.nb - 1)
    valid = w.N - (w.nb - 1) * w.b
    for s in last:
        assert not packed[s, 0].reshape(w.b, w.d)[valid:].any()
        assert not packed[s, 1].reshape(w.d, w.b)[:, valid:].any()


def test_bf16_decode_known_values():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x7F80, 0x0001], np.uint16)
    vals = O.bf16_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[2] == 0.0
    assert np.signbit(vals[3]) and vals[3] == 0.0
    assert vals[4] == 3.140625 and np.isinf(vals[5])
    assert vals[6] == 2.0 ** -133
