"""GPU parity of mask materialisation from pooled tiles (section 4.2) through the C ABI.

Pooling is compared with the fp64 oracle within fp32 summation error.  The mask is a decision taken on
fp32 scores and fp32 prefix sums, so the comparison follows what the arithmetic fixes: a row must equal
the oracle's row unless the oracle's own decision lies within the fp32 error bound of a tie (two scores
at the selection boundary, or the prefix weight at the threshold tau); such a row must still be a valid
selection under that bound (no block left out that certainly outscores one taken in; a length whose
prefix weight reaches tau within the bound, and one block fewer would not).  Rows of the first kind
must make up nearly all rows.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_rank_amd as bsa
import oracle as O
from workloads import CONFIGS, custom, make_inputs

pytestmark = pytest.mark.gpu

U = 2.0 ** -24   # fp32 unit roundoff


def _dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _abs_pool(X, b, N, ids=None):
    """Pooled |x| (fp64): the scale of each pooled value's rounding error."""
    A = O.bf16_to_f64(X)
    H, rows, d = X.shape
    n = rows // b
    ids = np.arange(n) if ids is None else np.asarray(ids)
    out = np.zeros((H, n, d))
    for k in range(n):
        real = min(b, N - int(ids[k]) * b)
        if real > 0:
            out[:, k] = np.abs(A[:, k * b:k * b + real]).sum(axis=1) / real
    return out


def _check_rows(mask_gpu, qp, kp, aq, ak, scale, tau, k_min, b, d, nb):
    """Returns (rows, exact rows); asserts validity of every row."""
    H, Lq = qp.shape[0], qp.shape[1]
    s64 = O.block_scores(qp, kp, scale)
    dq, dk = (b + 4) * U * aq, (b + 4) * U * ak                     # pooled value error bounds
    rows = exact = 0
    for h in range(H):
        E = scale * (np.abs(qp[h]) @ dk[h].T + dq[h] @ np.abs(kp[h]).T + dq[h] @ dk[h].T
                     + (d + 4) * U * (np.abs(qp[h]) @ np.abs(kp[h]).T)) * 2.0 + 1e-30
        for k in range(Lq):
            rows += 1
            s, e = s64[h, k], E[k]
            order, n_o = O.select_row(s, tau, k_min)
            want = np.zeros(nb, bool)
            want[order[:n_o]] = True
            got = mask_gpu[h, k, :nb] != 0
            assert not mask_gpu[h, k, nb:].any()
            if np.array_equal(got, want):
                exact += 1
                continue
            # a different row is allowed only where fp32 rounding can decide it
            ec = 4 * float(e.max()) + (2 * nb + 16) * U
            taken, left = np.flatnonzero(got), np.flatnonzero(~got)
            if len(left):
                assert (s[taken] + e[taken]).min() >= (s[left] - e[left]).max(), (h, k, "order")
            n = len(taken)
            p = np.exp(s - s.max())
            mass = np.sort(p)[::-1].cumsum() / p.sum()
            assert n >= min(nb, k_min) and n <= nb
            if n > max(1, k_min):
                assert mass[n - 2] < tau + ec, (h, k, "too long")
            assert n == nb or mass[n - 1] >= tau - ec, (h, k, "too short")
    return rows, exact


def _run(w, tau, k_min, inp=None):
    inp = inp or make_inputs(w)
    w = inp["workload"]
    Lq = len(inp["q_blocks"])
    g = bsa.geometry(H=w.H, d=w.d, b=w.b, N=w.N, G=w.G, r=w.r, Lq=Lq)
    ids = torch.from_numpy(inp["q_blocks"]).cuda()
    qp = bsa.pool_blocks(g, _dev_bf16(inp["Q"]), block_ids=ids)
    kp = bsa.pool_blocks(g, _dev_bf16(inp["K"]))
    mask = bsa.materialize_mask(g, qp, kp, tau, k_min)
    torch.cuda.synchronize()
    return inp, g, qp.cpu().numpy(), kp.cpu().numpy(), mask.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "small", "ltx_like"])
def test_pooling_matches_oracle(require_gpu, name):
    w = custom(H=3, d=64, T=3, HW=1000, b=64, G=3, k_offset_sigma=3.0) if name == "ltx_like" else CONFIGS[name]
    inp, g, qp, kp, _ = _run(w, 0.5, 1)
    w = inp["workload"]
    for got, X, ids in ((qp, inp["Q"], inp["q_blocks"]), (kp, inp["K"], None)):
        want = O.pool_blocks(X, w.b, w.N, ids)
        bound = (w.b + 4) * U * _abs_pool(X, w.b, w.N, ids) + 1e-30
        assert np.all(np.abs(got - want) <= bound)


CASES = {
    # name: (workload, tau, k_min)
    "tiny_cdf": (CONFIGS["tiny"], 0.9, 2),
    "small_cdf": (CONFIGS["small"], 0.85, 4),
    "small_topk": (CONFIGS["small"], 0.0, 51),
    "column_pattern": (custom(H=4, d=128, T=4, HW=1900, b=128, G=2, k_offset_sigma=3.0), 0.9, 3),
    "d64_b128_ragged": (custom(H=2, d=64, T=3, HW=1000, b=128, G=3), 0.95, 1),
    "floor_everything": (custom(H=2, d=64, T=2, HW=700, b=64, G=2), 0.1, 10_000),
    "tau_one": (custom(H=2, d=128, T=2, HW=700, b=64, G=2), 1.0, 0),
    # rows of more than 1024 blocks take the 512-thread, two-row select
    "wide_d64": (custom(H=2, d=64, T=12, HW=6144, b=64, G=8, k_offset_sigma=3.0), 0.9, 16),
    "wide_d128_ragged": (custom(H=1, d=128, T=37, HW=3600, b=128, G=8), 0.5, 4),
    # rows of more than 4096 blocks take the 1024-thread select (eight, then sixteen blocks per thread)
    "rows_6k_d64": (custom(H=1, d=64, T=2, HW=64 * 3000, b=64, G=64, r=9, k_offset_sigma=3.0), 0.9, 16),
    "rows_12k_d128_ragged": (custom(H=1, d=128, T=1, HW=128 * 12000 - 51, b=128, G=64, r=33), 0.85, 8),
    "rows_16k_d64": (custom(H=1, d=64, T=4, HW=64 * 4096, b=64, G=64, r=60, k_offset_sigma=3.0), 0.5, 32),
}


@pytest.mark.parametrize("case", list(CASES))
def test_mask_matches_oracle(require_gpu, case):
    w, tau, k_min = CASES[case]
    inp, g, qp, kp, mask = _run(w, tau, k_min)
    w = inp["workload"]
    qo = O.pool_blocks(inp["Q"], w.b, w.N, inp["q_blocks"])
    ko = O.pool_blocks(inp["K"], w.b, w.N)
    aq = _abs_pool(inp["Q"], w.b, w.N, inp["q_blocks"])
    ak = _abs_pool(inp["K"], w.b, w.N)
    rows, exact = _check_rows(mask, qo, ko, aq, ak, 1 / math.sqrt(w.d), tau, k_min, w.b, w.d, w.nb)
    assert exact >= 0.98 * rows, (exact, rows)


def _random_case(i: int):
    rng = np.random.default_rng([77, i])
    d, b = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
    if i % 2:  # rows of 1024 to about 4000 blocks: the long-row select
        T, HW, G = int(rng.integers(16, 32)), int(rng.integers(64 * b, 124 * b)), int(rng.choice([4, 8]))
    else:
        T, HW, G = int(rng.integers(1, 6)), int(rng.integers(b, 40 * b)), int(rng.choice([1, 2, 4, 8]))
    w = custom(name=f"mat_random{i}", H=int(rng.integers(1, 3)), d=d, b=b, T=T, HW=HW, G=G, r=int(rng.integers(G)),
               k_offset_sigma=float(rng.choice([0.0, 3.0, 10.0])), seed=500 + i)
    return w, float(rng.choice([0.0, 0.5, 0.85, 0.9, 0.99, 1.0])), int(rng.integers(0, 40))


@pytest.mark.parametrize("i", range(8))
def test_random_geometries(require_gpu, i):
    """Seeded random geometries (both head dims and block sizes, rows on both sides of 1024 blocks, random
    tau and k_min) under the same validity rules."""
    w, tau, k_min = _random_case(i)
    inp, g, qp, kp, mask = _run(w, tau, k_min)
    w = inp["workload"]
    if len(inp["q_blocks"]) == 0:
        return
    print(f"[materialize] random {i}: H={w.H} d={w.d} b={w.b} nb={w.nb} Lq={len(inp['q_blocks'])} tau={tau} "
          f"k_min={k_min}", flush=True)
    qo = O.pool_blocks(inp["Q"], w.b, w.N, inp["q_blocks"])
    ko = O.pool_blocks(inp["K"], w.b, w.N)
    aq = _abs_pool(inp["Q"], w.b, w.N, inp["q_blocks"])
    ak = _abs_pool(inp["K"], w.b, w.N)
    rows, exact = _check_rows(mask, qo, ko, aq, ak, 1 / math.sqrt(w.d), tau, k_min, w.b, w.d, w.nb)
    assert exact >= 0.98 * rows, (exact, rows)


def test_hunyuan_full_size_sampled(require_gpu):
    """The HunyuanVideo-shaped share at full size: pooled keys of all 929 blocks, the mask of every local
    row; rows of the first and last heads checked against the oracle."""
    inp = make_inputs("hunyuan")
    w = inp["workload"]
    inp2, g, qp, kp, mask = _run(w, 0.9, 16, inp=inp)
    heads = [0, w.H - 1]
    sub = lambda a: a[heads]  # noqa: E731
    qo = O.pool_blocks(inp["Q"][heads], w.b, w.N, inp["q_blocks"])
    ko = O.pool_blocks(inp["K"][heads], w.b, w.N)
    aq = _abs_pool(inp["Q"][heads], w.b, w.N, inp["q_blocks"])
    ak = _abs_pool(inp["K"][heads], w.b, w.N)
    rows, exact = _check_rows(sub(mask), qo, ko, aq, ak, 1 / math.sqrt(w.d), 0.9, 16, w.b, w.d, w.nb)
    assert exact >= 0.98 * rows, (exact, rows)


def test_materialized_mask_feeds_the_path(require_gpu):
    """The materialised mask is the input format of the demand union and the attention: run the whole
    path on it and compare with the oracle (union bit-exact, attention within tolerance)."""
    w = CONFIGS["small"]
    inp, g, qp, kp, mask = _run(w, 0.3, 8)
    mask_d = torch.from_numpy(mask).cuda()
    u = bsa.demand_union(g, mask_d, torch.from_numpy(inp["placement"]).cuda())
    packed = bsa.pack_kv(g, _dev_bf16(inp["K"]), _dev_bf16(inp["V"]), u)
    Od, _ = bsa.block_sparse_attn(g, _dev_bf16(inp["Q"]), mask_d, u.slot_of, packed)
    torch.cuda.synchronize()
    U_o = O.demand_union(mask, w.nb)
    assert np.array_equal(u.demand.cpu().numpy().view(np.uint64), O.demand_words(U_o))
    Oo, _ = O.attention(inp["Q"], inp["K"], inp["V"], mask, w.b, w.N, 1 / math.sqrt(w.d),
                        items=[(0, 0), (w.H - 1, g.Lq - 1), (3, 7)])
    for h, k in [(0, 0), (w.H - 1, g.Lq - 1), (3, 7)]:
        err = np.abs(Od.cpu().numpy()[h, k * w.b:(k + 1) * w.b] - Oo[h, k * w.b:(k + 1) * w.b])
        assert err.max() <= 1e-2 and err.mean() <= 1e-3


def test_repeat_runs_are_bit_identical(require_gpu):
    """Pooling sums in a fixed order and the select's threshold search reduces in a fixed order: two runs
    give the same pooled tiles and the same mask, bit for bit (also on rows of more than 1024 blocks)."""
    for w in (CONFIGS["small"], custom(H=2, d=64, T=12, HW=6144, b=64, G=8)):
        a = _run(w, 0.9, 4)
        b = _run(w, 0.9, 4, inp=a[0])
        for x, y in zip(a[2:], b[2:]):
            assert np.array_equal(x, y)
