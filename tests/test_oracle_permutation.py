"""Pins for the oracle's placement permutation (section 4.3: logical blocks are permuted to (rank, offset)
order before the distributed region and restored afterwards; whole blocks move, their contents do not).

The checks compare the oracle with closed forms (contiguous placement = identity; the periodic placement
of Eq. 4 on frame-aligned blocks), with an independent sort, with the sequence-parallel split it must
produce, and with the permutation equivariance of attention.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O
from workloads import placement_contiguous, placement_periodic


@settings(max_examples=80, deadline=None)
@given(nb=st.integers(1, 300), G=st.integers(1, 16), kind=st.sampled_from(["contiguous", "periodic", "random"]),
       seed=st.integers(0, 2**31 - 1))
def test_permutation_is_rank_major_sort(nb, G, kind, seed):
    if kind == "contiguous":
        P = placement_contiguous(nb, G)
    elif kind == "periodic":
        P = placement_periodic(nb, 64, 64 * max(1, nb // 4 + 1), G)
    else:
        P = np.random.default_rng(seed).integers(0, G, nb).astype(np.int32)
    pos, offs = O.placement_permutation(P, G)
    # a bijection onto 0..nb-1
    assert sorted(pos.tolist()) == list(range(nb))
    # the same order as an independent sort by (rank, logical index)
    order = sorted(range(nb), key=lambda j: (int(P[j]), j))
    assert [int(pos[j]) for j in order] == list(range(nb))
    # rank p's range holds exactly Q_p, ascending
    for p in range(G):
        lo, hi = int(offs[p]), int(offs[p + 1])
        inv = np.empty(nb, np.int64)
        inv[pos] = np.arange(nb)
        assert inv[lo:hi].tolist() == O.local_query_blocks(P, p).tolist()
    assert offs[0] == 0 and offs[-1] == nb


@pytest.mark.parametrize("nb,G", [(16, 4), (929, 8), (591, 4), (3072, 8), (7, 3), (1, 1)])
def test_contiguous_placement_is_identity(nb, G):
    pos, offs = O.placement_permutation(placement_contiguous(nb, G), G)
    assert pos.tolist() == list(range(nb))
    counts = np.bincount(placement_contiguous(nb, G), minlength=G)
    assert offs.tolist() == [0] + np.cumsum(counts).tolist()


@pytest.mark.parametrize("T,B,G", [(4, 4, 4), (16, 16, 8), (32, 96, 8), (3, 12, 4), (5, 8, 2)])
def test_periodic_closed_form(T, B, G):
    """Eq. 4 with B blocks per frame and G dividing B: block (t, s) goes to rank floor(G s / B) at offset
    t * (B / G) + (s mod B / G), and rank p starts at p * T * B / G."""
    b = 64
    nb = T * B
    P = placement_periodic(nb, b, B * b, G)
    pos, offs = O.placement_permutation(P, G)
    per = B // G
    for t in range(T):
        for s in range(B):
            j = t * B + s
            assert P[j] == (G * s) // B
            assert pos[j] == (s // per) * (T * per) + t * per + (s % per)
    assert offs.tolist() == [p * T * per for p in range(G + 1)]


@settings(max_examples=40, deadline=None)
@given(outer=st.integers(1, 3), nb=st.integers(1, 40), b=st.sampled_from([1, 2, 64]), C=st.integers(1, 9),
       G=st.integers(1, 6), seed=st.integers(0, 2**31 - 1))
def test_permute_blocks_moves_whole_blocks_and_round_trips(outer, nb, b, C, G, seed):
    rng = np.random.default_rng(seed)
    P = rng.integers(0, G, nb).astype(np.int32)
    pos, offs = O.placement_permutation(P, G)
    x = rng.integers(0, 2**16, (outer, nb * b, C), dtype=np.uint16)
    y = O.permute_blocks(x, pos, b)
    for j in range(nb):
        p = int(pos[j])
        assert np.array_equal(y[:, p * b:(p + 1) * b], x[:, j * b:(j + 1) * b])
    assert np.array_equal(O.permute_blocks(y, pos, b, inverse=True), x)
    assert np.array_equal(O.permute_blocks(O.permute_blocks(x, pos, b, inverse=True), pos, b), x)
    # the sequence-parallel split of the permuted rows gives rank p its own blocks Q_p in order
    for p in range(G):
        shard = y[:, int(offs[p]) * b:int(offs[p + 1]) * b]
        qp = O.local_query_blocks(P, p)
        want = np.concatenate([x[:, j * b:(j + 1) * b] for j in qp], axis=1) if len(qp) else shard
        assert np.array_equal(shard, want)


def test_permutation_preserves_attention():
    """Whole blocks move and their membership is unchanged, so attention of the permuted sequence is the
    permuted attention of the original (softmax attention is equivariant under a common permutation of
    the query and key rows)."""
    rng = np.random.default_rng(5)
    b, nb, d, G = 4, 12, 8, 3
    P = placement_periodic(nb, b, 4 * b, G)
    pos, _ = O.placement_permutation(P, G)
    N = nb * b
    from workloads import bf16_bits_from_f32
    Q, K, V = (bf16_bits_from_f32(rng.standard_normal((1, N, d), dtype=np.float32)) for _ in range(3))
    ones = np.ones((1, nb, 64), np.uint8)
    scale = 1 / math.sqrt(d)
    Oa, la = O.attention(Q, K, V, ones, b, N, scale)
    Qp, Kp, Vp = (O.permute_blocks(t, pos, b) for t in (Q, K, V))
    Ob, lb = O.attention(Qp, Kp, Vp, ones, b, N, scale)
    assert np.allclose(O.permute_blocks(Oa, pos, b), Ob, atol=1e-12, rtol=0)
    assert np.allclose(O.permute_blocks(la[:, :, None], pos, b)[:, :, 0], lb, atol=1e-12, rtol=0)


def test_planted_mistake_descending_inside_rank_is_caught():
    """A permutation that orders a rank's blocks descending fails the split check."""
    P = placement_periodic(32, 64, 64 * 8, 4)
    pos, offs = O.placement_permutation(P, 4)
    bad = pos.copy()
    for p in range(4):
        idx = np.flatnonzero(P == p)
        bad[idx] = pos[idx][::-1]
    inv = np.empty(32, np.int64)
    inv[bad] = np.arange(32)
    assert inv[offs[1]:offs[2]].tolist() != O.local_query_blocks(P, 1).tolist()
