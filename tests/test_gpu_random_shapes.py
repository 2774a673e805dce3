"""GPU parity over seeded random geometries: head dim and block size in {64, 128} in all four pairings,
1-3 heads, 1-8 ranks with a random local rank, contiguous or periodic placement, token counts with ragged
last blocks, mask densities from a few blocks per row to nearly dense, and K block offsets from none to
large.  For each: union, compaction and pack bit-exact against the oracle; single-pass attention and the
ring-order fold of the segment calls within the attention tolerance on every (head, query block)."""
import math

import numpy as np
import pytest

import oracle as O
from test_gpu_parity import MAX_ABS, _check_attention, _check_union
from workloads import custom, make_inputs

pytestmark = pytest.mark.gpu


def _random_case(i: int):
    rng = np.random.default_rng([2026, i])
    d = int(rng.choice([64, 128]))
    b = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 3, 5, 8]))
    T = int(rng.integers(1, 5))
    HW = int(rng.integers(b // 2, 12 * b))
    return custom(name=f"random{i}", H=int(rng.integers(1, 4)), d=d, b=b, T=T, HW=HW, G=G,
                  r=int(rng.integers(G)), placement=str(rng.choice(["contiguous", "periodic"])),
                  density=float(rng.uniform(0.03, 0.9)), k_offset_sigma=float(rng.choice([0.0, 3.0, 20.0])),
                  seed=1000 + i)


CASES = list(range(16))


@pytest.mark.parametrize("i", CASES)
def test_random_geometry(require_gpu, i):
    import torch
    import block_sparse_attention_rank_amd as bsa
    from _gpu import run_path, to_host_u16, union_host
    w = _random_case(i)
    print(f"[parity] random {i}: H={w.H} d={w.d} b={w.b} N={w.N} nb={w.nb} G={w.G} r={w.r} "
          f"{w.placement} density={w.density:.2f} sigma={w.k_offset_sigma}", flush=True)
    inp = make_inputs(w)
    res = run_path(inp)
    c = _check_union(union_host(res["union"]), inp)
    assert np.array_equal(to_host_u16(res["packed"][:c["S"]]),
                          O.pack(inp["K"], inp["V"], c["slot_block"], c["slot_head"], w.b))
    Lq = len(inp["q_blocks"])
    if Lq == 0:
        return
    items = [(h, k) for h in range(w.H) for k in range(Lq)]
    _check_attention(inp, res["O"].cpu().numpy(), res["lse"].cpu().numpy(), items)

    g, u, dev = res["g"], res["union"], res["dev"]
    ranges = bsa.segment_ranges(u.seg_offsets.cpu().numpy(), w.H, w.G)
    O_run = torch.zeros_like(res["O"])
    lse_run = torch.full_like(res["lse"], float("-inf"))
    for p in [(w.r + k) % w.G for k in range(w.G)]:
        lo, hi = ranges[p]
        bsa.block_sparse_attn_segment_accumulate(g, dev["Q"], dev["mask"], u.slot_of, res["packed"], lo, hi, O_run,
                                                 lse_run, 1.0 / math.sqrt(w.d))
    torch.cuda.synchronize()
    _check_attention(inp, O_run.cpu().numpy(), lse_run.cpu().numpy(), items)
    real = O.real_rows(inp["q_blocks"], w.b, w.N)
    assert np.abs(O_run.cpu().numpy()[:, real] - res["O"].cpu().numpy()[:, real]).max() <= 2 * MAX_ABS
