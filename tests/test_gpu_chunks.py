"""GPU parity of the chunked consumption schedule (section 7 of the SparSP text) through the C ABI.

The schedule comes from sparsp_chunk_plan on the device's own compaction and access counts and must equal
the oracle's plan; folding every chunk with sparsp_block_sparse_attn_chunk_accumulate must match the oracle's
attention on every (head, query block) within the attention bounds; with one chunk per segment it is
bit-identical to the per-segment fold; and a chunk leaves the rows of other heads untouched.
"""
import math

import numpy as np
import pytest

import oracle as O
from workloads import custom, make_inputs

pytestmark = pytest.mark.gpu

MAX_ABS = 1e-2

CASES = {
    "small": None,
    "hetero_heads_d64": custom(H=6, d=64, b=64, T=4, HW=512, G=4, r=1, density_range=(0.03, 0.5)),
    "periodic_d128_pad": custom(H=5, d=128, b=128, T=3, HW=1000, G=4, r=2, placement="periodic", density=0.3),
    "hunyuan": None,
}
PLANS = [(1, 1), (2, 4), (3, 99)]


def _run_plan(res, inp, plan):
    import torch
    import block_sparse_attention_rank_amd as bsa
    g, u, dev = res["g"], res["union"], res["dev"]
    O_run = torch.zeros_like(res["O"])
    lse_run = torch.full_like(res["lse"], float("-inf"))
    for ch in plan:
        bsa.block_sparse_attn_chunk_accumulate(g, dev["Q"], dev["mask"], u.slot_of, res["packed"], ch, O_run, lse_run,
                                               1.0 / math.sqrt(g.d))
    torch.cuda.synchronize()
    return O_run, lse_run


@pytest.mark.parametrize("name", list(CASES))
def test_chunk_schedule_matches_oracle(require_gpu, name):
    import torch
    import block_sparse_attention_rank_amd as bsa
    from _gpu import run_path
    from test_gpu_parity import _check_attention, _inputs
    w = CASES[name]
    inp = _inputs(name) if w is None else make_inputs(w)
    w = inp["workload"]
    print(f"[chunks] {name}", flush=True)
    res = run_path(inp)
    g, u, dev = res["g"], res["union"], res["dev"]
    counts = bsa.demand_counts(g, dev["mask"]).cpu().numpy()
    seg = u.seg_offsets.cpu().numpy()
    c = O.compact(O.demand_union(inp["mask"], w.nb), inp["placement"], w.G)
    tiles = O.segment_tiles(inp["mask"], inp["placement"], w.G, w.nb)
    ranges = bsa.segment_ranges(seg, w.H, w.G)
    ring = [(w.r + k) % w.G for k in range(w.G)]
    seg_O = torch.zeros_like(res["O"])
    seg_lse = torch.full_like(res["lse"], float("-inf"))
    for p in ring:
        bsa.block_sparse_attn_segment_accumulate(g, dev["Q"], dev["mask"], u.slot_of, res["packed"], *ranges[p], seg_O,
                                                 seg_lse)
    torch.cuda.synchronize()
    real = O.real_rows(inp["q_blocks"], w.b, w.N)
    for steady, drain in PLANS:
        plan = bsa.chunk_plan(seg, counts, inp["placement"], w.G, w.r, steady, drain)
        assert plan == O.chunk_plan(c["seg_offsets"], tiles, w.G, w.H, w.r, steady, drain)
        O_run, lse_run = _run_plan(res, inp, plan)
        mx, mean = _check_attention(inp, O_run.cpu().numpy(), lse_run.cpu().numpy())
        if (steady, drain) == (1, 1):
            # one chunk per segment, all heads: the same launches as the per-segment fold
            assert torch.equal(O_run, seg_O) and torch.equal(lse_run, seg_lse)
        d_single = np.abs(O_run.cpu().numpy()[:, real] - res["O"].cpu().numpy()[:, real]).max()
        assert d_single <= 2 * MAX_ABS
        print(f"[chunks] {name} plan ({steady}, {drain}): {len(plan)} chunks, max |dO| {mx:.2e}, mean {mean:.2e}",
              flush=True)


def test_chunk_leaves_other_heads_untouched(require_gpu):
    import torch
    import block_sparse_attention_rank_amd as bsa
    from _gpu import run_path
    inp = make_inputs(custom(H=4, d=64, b=64, T=3, HW=512, G=3, r=1, density=0.4))
    w = inp["workload"]
    res = run_path(inp)
    g, u, dev = res["g"], res["union"], res["dev"]
    seg = u.seg_offsets.cpu().numpy()
    p = (w.r + 1) % w.G
    ch = dict(p=p, h_lo=1, h_hi=3, slot_lo=int(seg[p * w.H + 1]), slot_hi=int(seg[p * w.H + 3]))
    O_run = torch.full_like(res["O"], 7.0)
    lse_run = torch.full_like(res["lse"], 3.0)
    bsa.block_sparse_attn_chunk_accumulate(g, dev["Q"], dev["mask"], u.slot_of, res["packed"], ch, O_run, lse_run)
    torch.cuda.synchronize()
    for h in (0, 3):
        assert torch.all(O_run[h] == 7.0) and torch.all(lse_run[h] == 3.0)
    assert not torch.all(O_run[1:3] == 7.0)
