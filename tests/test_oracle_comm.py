"""Pins for the oracle's communication-volume accounting: access counts (Figure 4's sharing metric),
demand-directed delivery versus the relayed ring (section 3.3, section 5.1 and Figure 9) and the dense
ring.  Checked against the worked example of Figure 9, the two-rank identity of section 3.3, closed
forms for all-ones, identity and multi-diagonal masks, and a hop-by-hop ring simulation written with
sets."""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O
from workloads import placement_contiguous, placement_periodic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _all_unions(mask_all, P, G, nb):
    """U_all [G][H][nb]: each consumer's union over its own rows of a mask given for every logical row."""
    H = mask_all.shape[0]
    U = np.zeros((G, H, nb), dtype=bool)
    for c in range(G):
        q = O.local_query_blocks(P, c)
        U[c] = O.demand_union(mask_all[:, q, :], nb)
    return U


def _simulate_ring(U_all, P, G):
    """Ring Attention with selective forwarding, hop by hop with Python sets: the shard of producer p
    leaves p holding every block some other rank selected; at each hop the receiver takes what it needs
    and the rest moves on only if a rank further along still needs it."""
    Gc, H, nb = U_all.shape
    hops = np.zeros((G, G), dtype=np.int64)
    for p in range(G):
        carried = {(h, j) for h in range(H) for j in range(nb)
                   if P[j] == p and any(U_all[c, h, j] for c in range(G) if c != p)}
        for k in range(1, G):
            hops[p, k] = len(carried)
            still = set()
            for (h, j) in carried:
                if any(U_all[(p + kk) % G, h, j] for kk in range(k + 1, G)):
                    still.add((h, j))
            carried = still
    return hops


def test_fig9_golden():
    g = json.load(open(os.path.join(GOLDEN, "fig9_ring_relay.json")))
    G, nb = g["G"], g["nb"]
    P = placement_contiguous(nb, G)
    mask_all = np.zeros((1, nb, 64), np.uint8)
    mask_all[0, np.arange(nb), np.arange(nb)] = 1
    for consumer, names in g["demand_from_rank0"].items():
        first_row = int(O.local_query_blocks(P, int(consumer))[0])
        for n in names:
            mask_all[0, first_row, g["block_names"][n]] = 1
    v = O.comm_volume(_all_unions(mask_all, P, G, nb), P, G)
    assert v["relay"][0].tolist() == g["expected_relay_hops_rank0"]
    assert int(v["relay"][0].sum()) == g["expected_relay_total_rank0"]
    assert v["direct"][:, 0].tolist() == g["expected_direct_to_consumers_from_rank0"]
    assert int(v["direct"][:, 0].sum()) == g["expected_direct_total_rank0"]
    assert int(v["dense"][0]) == g["expected_dense_ring_rank0"]
    assert v["direct"][:, 1:].sum() == 0 and v["relay"][1:].sum() == 0


def _random_all(rng, H, nb, p):
    m = np.zeros((H, nb, 64 * (-(-nb // 64))), np.uint8)
    m[:, :, :nb] = rng.random((H, nb, nb)) < p
    return m


@settings(max_examples=50, deadline=None)
@given(H=st.integers(1, 3), nb=st.integers(1, 40), G=st.integers(1, 7), p=st.floats(0, 1),
       periodic=st.booleans(), seed=st.integers(0, 2**31 - 1))
def test_relay_matches_hop_simulation_and_bounds(H, nb, G, p, periodic, seed):
    rng = np.random.default_rng(seed)
    P = placement_periodic(nb, 64, 64 * max(1, nb // 3), G) if periodic else placement_contiguous(nb, G)
    U = _all_unions(_random_all(rng, H, nb, p), P, G, nb)
    v = O.comm_volume(U, P, G)
    assert np.array_equal(v["relay"], _simulate_ring(U, P, G))
    assert np.all(np.diff(v["relay"][:, 1:], axis=1) <= 0)          # hops carry less and less
    assert v["direct"].sum() <= v["relay"].sum() <= v["dense"].sum()
    assert np.all(np.diag(v["direct"]) == 0)
    for c in range(G):                                              # direct = the remote part of Eq. 2
        for q in range(G):
            if q != c:
                assert v["direct"][c, q] == sum(int(U[c, h, j]) for h in range(H) for j in range(nb) if P[j] == q)
    if G == 2:                                                      # section 3.3: one hop, no relay
        assert v["relay"].sum() == v["direct"].sum()


def test_all_ones_and_identity():
    H, nb, G = 2, 24, 4
    P = placement_periodic(nb, 64, 64 * 8, G)
    n = np.bincount(P, minlength=G)
    ones = np.ones((H, nb, 64), np.uint8)
    v = O.comm_volume(_all_unions(ones, P, G, nb), P, G)
    for c in range(G):
        for p in range(G):
            assert v["direct"][c, p] == (0 if c == p else H * n[p])
    assert np.array_equal(v["relay"][:, 1:], np.repeat((H * n)[:, None], G - 1, axis=1))
    assert np.array_equal(v["relay"].sum(1), v["dense"])
    eye = np.zeros((H, nb, 64), np.uint8)
    eye[:, np.arange(nb), np.arange(nb)] = 1
    v = O.comm_volume(_all_unions(eye, P, G, nb), P, G)
    assert v["direct"].sum() == 0 and v["relay"].sum() == 0


@pytest.mark.parametrize("delta", [1, 2])
def test_multidiagonal_direct_volume_closed_form(delta):
    """Section 4.3: under periodic placement a consumer's remote demand is the 2*delta*T halo (delta*T at
    the two end ranks); under the contiguous partition it is every block it does not own."""
    T, B, G, b = 5, 16, 4, 64
    nb = T * B
    s = np.arange(nb) % B
    mask_all = np.zeros((1, nb, 128), np.uint8)
    mask_all[0, :, :nb] = np.abs(s[:, None] - s[None, :]) <= delta
    Pp = placement_periodic(nb, b, B * b, G)
    v = O.comm_volume(_all_unions(mask_all, Pp, G, nb), Pp, G)
    for c in range(G):
        assert v["direct"][c].sum() == (delta * T if c in (0, G - 1) else 2 * delta * T)
    Pc = placement_contiguous(nb, G)
    v = O.comm_volume(_all_unions(mask_all, Pc, G, nb), Pc, G)
    n = np.bincount(Pc, minlength=G)
    for c in range(G):
        assert v["direct"][c].sum() == nb - n[c]


@settings(max_examples=40, deadline=None)
@given(H=st.integers(1, 3), Lq=st.integers(0, 9), nb=st.integers(1, 90), p=st.floats(0, 1),
       seed=st.integers(0, 2**31 - 1))
def test_access_counts(H, Lq, nb, p, seed):
    rng = np.random.default_rng(seed)
    m = np.zeros((H, Lq, 64 * (-(-nb // 64))), np.uint8)
    m[:, :, :nb] = (rng.random((H, Lq, nb)) < p) * rng.integers(1, 256, (H, Lq, nb))   # any nonzero byte selects
    m[:, :, nb:] = 1                                                                 # pitch padding is ignored
    cnt = O.access_counts(m, nb)
    assert np.array_equal(cnt, (m[:, :, :nb] != 0).sum(1))
    assert np.array_equal(cnt > 0, O.demand_union(m, nb))
    assert cnt.sum() == int((m[:, :, :nb] != 0).sum())


def test_sharing_fractions_small_case():
    """Four local rows; remote block 5 is selected by one of them, remote block 6 by all four, own block 0
    by three: the two received remote blocks are shared by 1/4 and 4/4 of the local query blocks."""
    P = np.array([0, 0, 0, 0, 1, 1, 1, 1], np.int32)
    m = np.zeros((1, 4, 64), np.uint8)
    m[0, 0, 5] = 1
    m[0, :, 6] = 1
    m[0, :3, 0] = 1
    f = O.sharing_fractions(O.access_counts(m, 8), P, 0, 4)
    assert f.tolist() == [0.25, 1.0]
