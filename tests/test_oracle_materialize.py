"""Pins for the oracle's mask materialisation from pooled tiles (section 4.2): block-mean pooling,
block scores and the Top-p rule with a Top-k floor.  Checked against plain means, closed forms for
uniform and dominant scores, shift invariance, the pure Top-k special case (tau = 0) and a brute-force
search for the smallest qualifying prefix."""
import itertools
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O
from workloads import bf16_bits_from_f32


def test_pooling_is_the_mean_of_real_rows():
    rng = np.random.default_rng(0)
    b, d, H = 8, 4, 2
    N = 3 * b + 5                                    # last block: 5 real rows, 3 zero rows
    x = rng.standard_normal((H, 4 * b, d)).astype(np.float32)
    x[:, N:] = 0
    X = bf16_bits_from_f32(x)
    xf = O.bf16_to_f64(X)
    p = O.pool_blocks(X, b, N)
    for k in range(4):
        real = min(b, N - k * b)
        assert np.allclose(p[:, k], xf[:, k * b:k * b + real].mean(axis=1), atol=1e-15)
    # identical rows pool to that row
    Y = np.repeat(X[:, :1], 4 * b, axis=1)
    assert np.array_equal(O.pool_blocks(Y, b, 4 * b), np.repeat(O.bf16_to_f64(X[:, :1])[:, None, 0], 4, axis=1))
    # local query blocks: the real-row count follows the logical id
    pq = O.pool_blocks(X[:, 3 * b:4 * b], b, N, block_ids=[3])
    assert np.allclose(pq[:, 0], xf[:, 3 * b:3 * b + 5].mean(axis=1), atol=1e-15)


def test_scores_are_scaled_dot_products():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((2, 3, 5)), rng.standard_normal((2, 7, 5))
    s = O.block_scores(q, k, 0.25)
    for h, i, j in itertools.product(range(2), range(3), range(7)):
        assert math.isclose(s[h, i, j], 0.25 * sum(q[h, i, c] * k[h, j, c] for c in range(5)), abs_tol=1e-13)


def _brute_n(scores, tau, k_min):
    """Smallest prefix (in (-s, j) order) reaching tau of the softmax mass, by trying every length."""
    nb = len(scores)
    order = np.lexsort((np.arange(nb), -np.asarray(scores)))
    p = np.exp(np.asarray(scores) - np.max(scores))
    for n in range(1, nb + 1):
        if p[order[:n]].sum() >= tau * p.sum() * (1 - 1e-15):
            return list(order), min(nb, max(k_min, n))
    return list(order), nb


@settings(max_examples=100, deadline=None)
@given(nb=st.integers(1, 40), tau=st.floats(0, 1), k_min=st.integers(0, 45), seed=st.integers(0, 2**31 - 1),
       spread=st.floats(0.01, 20))
def test_selection_matches_bruteforce(nb, tau, k_min, seed, spread):
    s = np.random.default_rng(seed).standard_normal(nb) * spread
    order, n = O.select_row(s, tau, k_min)
    border, bn = _brute_n(s, tau, k_min)
    assert order == [int(j) for j in border]
    p = np.exp(s - s.max())
    # the two sums round differently: the lengths may differ only where every prefix between them holds tau of
    # the weight up to rounding (e.g. tau = 1 with trailing weights below the total's last digit)
    for m in range(min(n, bn), max(n, bn)):
        assert abs(p[order[:m]].sum() - tau * p.sum()) <= 1e-12 * p.sum(), (m, n, bn)
    assert n >= min(nb, k_min) and n <= nb
    if n > max(1, k_min):
        assert p[order[:n - 1]].sum() < tau * p.sum() * (1 + 1e-12)     # one block fewer is not enough
    assert p[order[:n]].sum() >= tau * p.sum() * (1 - 1e-12) or n == nb


@pytest.mark.parametrize("nb,tau", [(10, 0.35), (929, 0.9 + 1e-4), (64, 0.5 + 1 / 256)])
def test_uniform_scores_closed_form(nb, tau):
    """Equal scores: each block carries 1/nb of the mass and ties go to ascending j, so the first
    ceil(tau * nb) blocks are selected."""
    order, n = O.select_row(np.zeros(nb), tau, 0)
    assert order == list(range(nb)) and n == math.ceil(tau * nb)


def test_dominant_block_and_floor():
    s = np.zeros(50)
    s[17] = 60.0                                     # e^-60 of the mass elsewhere
    order, n = O.select_row(s, 0.999, 0)
    assert order[0] == 17 and n == 1
    assert O.select_row(s, 0.999, 5)[1] == 5         # the Top-k floor
    assert O.select_row(s, 0.0, 0)[1] == 1           # tau = 0: the best block only
    s2 = np.zeros(50)
    s2[17] = 3.0
    assert O.select_row(s2, 1.0, 0)[1] == 50          # tau = 1: every block with nonzero mass


def test_tau_zero_is_top_k_and_shift_invariance():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((2, 6, 8)), rng.standard_normal((2, 30, 8))
    m = O.materialize_mask(q, k, 0.3, 0.0, 7, 64)
    s = O.block_scores(q, k, 0.3)
    for h in range(2):
        for i in range(6):
            top = set(np.argsort(-s[h, i], kind="stable")[:7].tolist())
            assert set(np.flatnonzero(m[h, i]).tolist()) == top
    assert m[:, :, 30:].sum() == 0
    # adding the same vector to every pooled key shifts each row's scores by a constant: same mask
    shift = rng.standard_normal(8)
    for h in range(2):
        for i in range(6):
            c = 0.3 * float(q[h, i] @ shift)
            o1, n1 = O.select_row(s[h, i], 0.8, 3)
            o2, n2 = O.select_row(s[h, i] + c, 0.8, 3)
            assert o1 == o2 and n1 == n2


def test_planted_mistake_ascending_order_is_caught():
    """Selecting the lowest-scoring blocks instead of the highest breaks the tau = 0 Top-k pin."""
    s = np.array([0.1, 3.0, -2.0, 1.0])
    order, n = O.select_row(s, 0.0, 2)
    assert set(order[:n]) == {1, 3}
    assert set(np.argsort(s)[:2].tolist()) != {1, 3}
