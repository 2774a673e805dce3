"""Pins for the oracle's consumption schedule (CPU only): section 7 of the SparSP text.

The schedule cuts the payload into head chunks: the local segment whole, remote segments into a steady
chunk count, the final remote segment into the drain count (7.1, Figure 11), each segment's chunk with the
highest sparsity last (7.2).  Pinned here: the chunks partition the payload exactly once; their order and
sizes follow the rules, checked on a hand-counted example; their tile counts are brute-force counts of the
mask; and folding the chunks' partial attentions by log-sum-exp, in the plan's order or any other, gives the
attention over the whole row (the online softmax of section 2.3 applied to the pieces).
"""
import itertools
import math

import numpy as np
import pytest

import oracle as O
from workloads import custom, make_inputs


def _plan_inputs(w):
    inp = make_inputs(w)
    U = O.demand_union(inp["mask"], w.nb)
    c = O.compact(U, inp["placement"], w.G)
    tiles = O.segment_tiles(inp["mask"], inp["placement"], w.G, w.nb)
    return inp, c, tiles


CASES = [custom(H=3, d=64, b=64, T=3, HW=320, G=3, r=1, density=0.5),
         custom(H=4, d=128, b=128, T=2, HW=700, G=4, r=2, placement="periodic", density=0.6),
         custom(H=5, d=64, b=64, T=4, HW=256, G=4, r=0, density=0.3, density_range=(0.05, 0.6))]


@pytest.mark.parametrize("w", CASES)
@pytest.mark.parametrize("steady,drain", [(1, 1), (1, 2), (2, 4), (3, 99)])
def test_chunks_partition_the_payload(w, steady, drain):
    inp, c, tiles = _plan_inputs(w)
    plan = O.chunk_plan(c["seg_offsets"], tiles, w.G, w.H, w.r, steady, drain)
    covered = np.zeros(c["S"], dtype=np.int64)
    for ch in plan:
        covered[ch["slot_lo"]:ch["slot_hi"]] += 1
        assert ch["slot_hi"] > ch["slot_lo"]
        # the slots of a chunk are exactly its heads' demanded blocks owned by its source rank
        assert set(c["slot_head"][ch["slot_lo"]:ch["slot_hi"]]) <= set(range(ch["h_lo"], ch["h_hi"]))
        assert np.all(inp["placement"][c["slot_block"][ch["slot_lo"]:ch["slot_hi"]]] == ch["p"])
    assert np.all(covered == 1)                                   # every slot once
    assert sum(ch["tiles"] for ch in plan) == int((inp["mask"][:, :, :w.nb] != 0).sum())
    # segments in ring order, the local one first and whole; tiles non-increasing inside a segment
    ring = [(w.r + k) % w.G for k in range(w.G)]
    seen = [ch["p"] for ch in plan]
    assert seen == sorted(seen, key=ring.index)
    if plan and plan[0]["p"] == w.r:
        assert (plan[0]["h_lo"], plan[0]["h_hi"]) == (0, w.H) and seen.count(w.r) == 1
    for p in set(seen):
        t = [ch["tiles"] for ch in plan if ch["p"] == p]
        assert t == sorted(t, reverse=True)
        n_expect = 1 if p == w.r else min(drain if p == ring[-1] else steady, w.H)
        assert len(t) <= n_expect


def test_hand_counted_plan():
    """4 heads, 3 ranks, rank 0's view.  Tiles per (p, h) and slots per (p, h) are given; with one steady chunk
    and a drain of 4, the plan is: local segment p = 0 whole; p = 1 whole; p = 2 cut into its 4 heads, ordered
    by tiles 7, 5, 5, 1 (ties by head) -- heads 3, 0, 2, 1 -- so head 1 (the sparsest) runs last."""
    H, G = 4, 3
    per_ph = np.array([[2, 1, 1, 3],            # slots of (p, h), p-major
                       [1, 0, 2, 2],
                       [3, 1, 2, 4]])
    seg = np.zeros(G * H + 1, dtype=np.int64)
    seg[1:] = np.cumsum(per_ph.reshape(-1))
    tiles = np.array([[9, 4, 4, 8], [2, 0, 6, 5], [5, 1, 5, 7]])
    plan = O.chunk_plan(seg, tiles, G, H, 0, 1, 4)
    got = [(ch["p"], ch["h_lo"], ch["h_hi"], ch["slot_lo"], ch["slot_hi"], ch["tiles"]) for ch in plan]
    assert got == [(0, 0, 4, 0, 7, 25),
                   (1, 0, 4, 7, 12, 13),
                   (2, 3, 4, 18, 22, 7), (2, 0, 1, 12, 15, 5), (2, 2, 3, 16, 18, 5), (2, 1, 2, 15, 16, 1)]
    # two steady chunks for p = 1 (heads 0-1 hold 1 slot, heads 2-3 four), drain of 2 for p = 2
    plan = O.chunk_plan(seg, tiles, G, H, 0, 2, 2)
    got = [(ch["p"], ch["h_lo"], ch["h_hi"], ch["tiles"]) for ch in plan]
    assert got == [(0, 0, 4, 25), (1, 2, 4, 11), (1, 0, 2, 2), (2, 2, 4, 12), (2, 0, 2, 6)]
    # rank 1's view: ring order 1, 2, 0; the drain segment is p = 0
    plan = O.chunk_plan(seg, tiles, G, H, 1, 1, 2)
    assert [(ch["p"], ch["h_lo"], ch["h_hi"]) for ch in plan] == [(1, 0, 4), (2, 0, 4), (0, 0, 2), (0, 2, 4)]


def test_segment_tiles_brute_force():
    w = custom(H=2, d=64, b=64, T=3, HW=256, G=3, r=2, density=0.4)
    inp = make_inputs(w)
    tiles = O.segment_tiles(inp["mask"], inp["placement"], w.G, w.nb)
    for p in range(w.G):
        for h in range(w.H):
            n = sum(1 for k in range(len(inp["q_blocks"])) for j in range(w.nb)
                    if inp["mask"][h, k, j] and inp["placement"][j] == p)
            assert tiles[p, h] == n


@pytest.mark.parametrize("w", CASES[:2])
def test_chunks_fold_to_full_attention_in_any_order(w):
    inp, c, tiles = _plan_inputs(w)
    plan = O.chunk_plan(c["seg_offsets"], tiles, w.G, w.H, w.r, 2, 3)
    scale = 1.0 / math.sqrt(w.d)
    Lq = len(inp["q_blocks"])
    rng = np.random.default_rng(7)
    orders = [list(range(len(plan))), list(range(len(plan)))[::-1], list(rng.permutation(len(plan)))]
    for h in range(w.H):
        for k in range(Lq):
            full_O, full_lse = O.attention_block(inp["Q"], inp["K"], inp["V"], inp["mask"], h, k, w.b, w.N, scale)
            parts = []
            for ch in plan:
                if ch["h_lo"] <= h < ch["h_hi"]:
                    parts.append(O.attention_block_slots(inp["Q"], inp["K"], inp["V"], inp["mask"], c["slot_of"],
                                                         ch["slot_lo"], ch["slot_hi"], h, k, w.b, w.N, scale))
                else:
                    parts.append(None)                            # the chunk does not touch this head
            for order in orders:
                acc_O = np.zeros_like(full_O)
                acc_lse = np.full(full_lse.shape, -np.inf)
                for i in order:
                    if parts[i] is not None:
                        acc_O, acc_lse = O.lse_merge(acc_O, acc_lse, *parts[i])
                np.testing.assert_allclose(acc_O, full_O, rtol=0, atol=1e-12)
                np.testing.assert_allclose(acc_lse, full_lse, rtol=1e-13, atol=0)


def test_planted_wrong_order_is_caught():
    """A plan that puts the sparsest chunk of the drain segment first fails the ordering rule."""
    H, G = 4, 2
    seg = np.arange(G * H + 1)
    tiles = np.array([[1, 1, 1, 1], [4, 1, 3, 2]])
    plan = O.chunk_plan(seg, tiles, G, H, 0, 1, 4)
    t = [ch["tiles"] for ch in plan if ch["p"] == 1]
    assert t == [4, 3, 2, 1]
    assert t[::-1] != sorted(t, reverse=True)
