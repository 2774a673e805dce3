"""Pins for the oracle's segment-wise attention and log-sum-exp merge (CPU only).

Splitting a row's key set into the per-source-rank segments of the payload and merging the partial
(O, lse) results must reproduce attention over the whole set, in any merge order (the online softmax of
section 2.3 applied to the pieces section 5.1 delivers); the merge is pinned to a direct evaluation over
the union of the two key sets, to the identity on an empty part, and to commutativity.
"""
import itertools
import math

import numpy as np
import pytest

import oracle as O
from oracle import sparsp_oracle as OR
from workloads import custom, make_inputs


@pytest.mark.parametrize("w", [custom(H=2, d=64, b=64, T=3, HW=320, G=3, r=1, density=0.5),
                               custom(H=1, d=128, b=128, T=2, HW=700, G=4, r=2, placement="periodic",
                                      density=0.6)])
def test_segments_merge_to_full_attention_in_any_order(w):
    inp = make_inputs(w)
    scale = 1.0 / math.sqrt(w.d)
    Lq = len(inp["q_blocks"])
    for h in range(w.H):
        for k in range(Lq):
            full_O, full_lse = O.attention_block(inp["Q"], inp["K"], inp["V"], inp["mask"], h, k, w.b, w.N, scale)
            parts = [O.attention_block_segment(inp["Q"], inp["K"], inp["V"], inp["mask"], inp["placement"], p, h, k,
                                               w.b, w.N, scale) for p in range(w.G)]
            for order in itertools.islice(itertools.permutations(range(w.G)), 4):
                acc_O = np.zeros_like(full_O)
                acc_lse = np.full(full_lse.shape, -np.inf)
                for p in order:
                    acc_O, acc_lse = O.lse_merge(acc_O, acc_lse, *parts[p])
                np.testing.assert_allclose(acc_O, full_O, rtol=0, atol=1e-12)
                np.testing.assert_allclose(acc_lse, full_lse, rtol=1e-13, atol=0)


def test_merge_matches_direct_evaluation_over_the_union():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((5, 16))
    k = rng.standard_normal((40, 16)) * 3
    v = rng.standard_normal((40, 16))
    a, b = np.arange(0, 17), np.arange(17, 40)
    Oa, la, _ = OR._attend(q, k[a], v[a], 0.25)
    Ob, lb, _ = OR._attend(q, k[b], v[b], 0.25)
    Om, lm = O.lse_merge(Oa, la, Ob, lb)
    s = q @ k.T * 0.25
    w = np.exp(s - s.max(1, keepdims=True))
    np.testing.assert_allclose(Om, (w / w.sum(1, keepdims=True)) @ v, atol=1e-13)
    np.testing.assert_allclose(lm, np.log(np.exp(s).sum(1)), rtol=1e-14)
    Om2, lm2 = O.lse_merge(Ob, lb, Oa, la)
    np.testing.assert_allclose(Om2, Om, atol=1e-15)
    np.testing.assert_allclose(lm2, lm, rtol=1e-15)


def test_merge_with_empty_part_is_identity_and_empty_stays_empty():
    rng = np.random.default_rng(8)
    Oa, la = rng.standard_normal((4, 8)), rng.standard_normal(4)
    empty_O, empty_l = np.zeros((4, 8)), np.full(4, -np.inf)
    Om, lm = O.lse_merge(Oa, la, empty_O, empty_l)
    np.testing.assert_array_equal(Om, Oa)
    np.testing.assert_array_equal(lm, la)
    Oe, le = O.lse_merge(empty_O, empty_l, empty_O, empty_l)
    assert not Oe.any() and np.all(le == -np.inf)


def test_segment_of_rank_without_selected_blocks_is_empty():
    w = custom(H=1, d=64, b=64, T=4, HW=256, G=4, r=1, mask_kind="identity")
    inp = make_inputs(w)
    # identity mask: rank 1's rows select only its own blocks, so every other segment is empty
    for p in (0, 2, 3):
        Op, lp = O.attention_block_segment(inp["Q"], inp["K"], inp["V"], inp["mask"], inp["placement"], p, 0, 0,
                                           w.b, w.N, 0.125)
        assert not Op.any() and np.all(lp == -np.inf)
