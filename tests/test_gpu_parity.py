"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle on the same seeded inputs.

Union, compaction indices and packed bytes must be bit-exact.  Attention outputs (bf16 inputs, fp32
accumulation, bf16 probabilities in the P V product) must lie within max |dO| <= 1e-2 and
mean |dO| <= 1e-3 of the oracle over real query rows; lse within 1e-3 * max(1, |lse|).
Every (head, query block) of every workload is compared, the full-size shares included: the oracle runs
item by item on the host's cores (tests/_gpu.py).  The local set Q_r comes from the C ABI
(sparsp_local_query_blocks) and must equal the generator's.
"""
import math
from dataclasses import replace

import numpy as np
import pytest

import oracle as O
from workloads import CONFIGS, custom, make_inputs

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 1e-2, 1e-3
_cache = {}


def _inputs(name):
    if name not in _cache:
        _cache.clear()                     # keep one full-size workload in memory at a time
        _cache[name] = make_inputs(name)
    return _cache[name]


def _oracle_union(inp):
    w = inp["workload"]
    U = O.demand_union(inp["mask"], w.nb)
    return U, O.compact(U, inp["placement"], w.G)


def _check_union(got, inp):
    U, c = _oracle_union(inp)
    assert np.array_equal(got["demand"], O.demand_words(U))
    assert np.array_equal(got["seg_offsets"], c["seg_offsets"])
    assert got["S"] == c["S"]
    assert np.array_equal(got["slot_block"], c["slot_block"])
    assert np.array_equal(got["slot_head"], c["slot_head"])
    assert np.array_equal(got["slot_of"], c["slot_of"])
    return c


def _check_attention(inp, O_dev, lse_dev, items=None, segment=None):
    """Every listed item (all of them by default) against the oracle: max and mean |dO| over real rows, the
    lse bound, and empty rows exactly (0, -inf)."""
    from _gpu import all_items, compare_items
    r = compare_items(inp, O_dev, lse_dev, all_items(inp) if items is None else items, segment=segment)
    assert r["bad_rows"] == 0, f"{r['bad_rows']} rows differ in emptiness"
    assert r["max"] <= MAX_ABS, f"max |dO| = {r['max']:.3e}"
    assert r["mean"] <= MEAN_ABS, f"mean |dO| = {r['mean']:.3e}"
    assert r["lse_rel"] <= 1e-3, f"max rel |dlse| = {r['lse_rel']:.3e}"
    return r["max"], r["mean"]


@pytest.mark.parametrize("name", list(CONFIGS))
def test_union_compaction_pack_bit_exact(require_gpu, name):
    from _gpu import run_path, to_host_u16, union_host
    inp = _inputs(name)
    w = inp["workload"]
    print(f"[parity] union/pack {name}", flush=True)
    res = run_path(inp, attention=False)
    c = _check_union(union_host(res["union"]), inp)
    packed = to_host_u16(res["packed"][:c["S"]])
    expect = O.pack(inp["K"], inp["V"], c["slot_block"], c["slot_head"], w.b)
    assert np.array_equal(packed, expect)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_attention_matches_oracle(require_gpu, name):
    from _gpu import run_path
    inp = _inputs(name)
    w = inp["workload"]
    print(f"[parity] attention {name}", flush=True)
    res = run_path(inp)
    Od, ld = res["O"].cpu().numpy(), res["lse"].cpu().numpy()
    n_items = w.H * len(inp["q_blocks"])
    mx, mean = _check_attention(inp, Od, ld)
    print(f"[parity] {name}: all {n_items} (head, query block) items, max |dO| {mx:.2e}, mean |dO| {mean:.2e}",
          flush=True)


EDGE_CASES = {
    "pad_d128_b128": custom(H=3, d=128, b=128, T=3, HW=300, G=2, r=1, density=0.5),
    "pad_d64_b64": custom(H=2, d=64, b=64, T=5, HW=100, G=3, r=2, density=0.4),
    "d128_b64": custom(H=2, d=128, b=64, T=4, HW=256, G=4, r=3, placement="periodic", density=0.3),
    "d64_b128": custom(H=2, d=64, b=128, T=4, HW=384, G=2, r=0, density=0.5),
    "all_ones": custom(H=2, d=128, b=128, T=2, HW=700, G=2, r=0, mask_kind="ones"),
    "identity": custom(H=2, d=64, b=64, T=3, HW=256, G=3, r=1, mask_kind="identity"),
    "empty_rows": custom(H=2, d=64, b=64, T=2, HW=256, G=2, r=0, mask_kind="zeros"),
    "single_rank": custom(H=1, d=128, b=128, T=2, HW=640, G=1, r=0, density=0.3),
    "k_offsets": custom(H=2, d=64, b=64, T=4, HW=512, G=2, r=1, k_offset_sigma=6.0, density=0.2),
    "many_ranks": custom(H=2, d=64, b=64, T=8, HW=1024, G=64, r=62, placement="periodic", density=0.1),
    "wide_row": custom(H=1, d=128, b=128, T=2, HW=128 * 150, G=2, r=1, density=0.45),
    # per-block K offsets large enough that a row's logits jump by far more than 64 (log2 units) between
    # key blocks, up and down: the running maximum must be raised (and exp2 would overflow) many times
    "logit_jumps_d64": custom(H=2, d=64, b=64, T=4, HW=512, G=2, r=0, k_offset_sigma=40.0, density=0.3),
    "logit_jumps_d128": custom(H=2, d=128, b=128, T=3, HW=640, G=2, r=1, k_offset_sigma=25.0, density=0.5),
    # rows with more selected blocks than one listing pass of the attention kernel holds, so the running
    # softmax state crosses passes: > 1024 selected at d = b = 128, > 512 at b = 64, and selections on
    # both sides of column 1024 at d = 64, b = 128 (one listing step per pass)
    "multipass_d128_b128": custom(H=1, d=128, b=128, T=1, HW=128 * 2200, G=64, r=5, density=0.6),
    "multipass_d64_b64": custom(H=1, d=64, b=64, T=1, HW=64 * 1200, G=32, r=7, density=0.6,
                                k_offset_sigma=4.0),
    "multipass_d64_b128": custom(H=1, d=64, b=128, T=1, HW=128 * 1100 - 37, G=32, r=3, density=0.3),
    "multipass_d128_b64": custom(H=1, d=128, b=64, T=1, HW=64 * 1200, G=32, r=20, density=0.6),
    # full-size shares in the two mixed (d, b) shapes: the HunyuanVideo-shaped share with 64-token blocks
    # (d = 128, b = 64: the 32-key stage pipeline) and the LTX-Video-shaped share with 128-token blocks
    "hunyuan_b64": replace(CONFIGS["hunyuan"], name="hunyuan_b64", b=64),
    "ltx_b128": replace(CONFIGS["ltx"], name="ltx_b128", b=128),
}


@pytest.mark.parametrize("case", list(EDGE_CASES))
def test_edge_cases(require_gpu, case):
    from _gpu import run_path, to_host_u16, union_host
    w = EDGE_CASES[case]
    inp = make_inputs(w)
    print(f"[parity] edge {case}: H={w.H} d={w.d} b={w.b} N={w.N} G={w.G} r={w.r}", flush=True)
    res = run_path(inp)
    c = _check_union(union_host(res["union"]), inp)
    assert np.array_equal(to_host_u16(res["packed"][:c["S"]]),
                          O.pack(inp["K"], inp["V"], c["slot_block"], c["slot_head"], w.b))
    _check_attention(inp, res["O"].cpu().numpy(), res["lse"].cpu().numpy())


def test_no_local_blocks(require_gpu):
    """A rank that owns no block (Lq = 0): the demand is empty and attention launches nothing."""
    from _gpu import run_path, union_host
    w = custom(H=2, d=64, b=64, T=1, HW=128, G=4, r=3)          # nb = 2 < G: rank 3 owns nothing
    inp = make_inputs(w)
    assert len(inp["q_blocks"]) == 0
    res = run_path(inp)
    got = union_host(res["union"])
    assert got["S"] == 0 and np.all(got["slot_of"] == -1) and not got["demand"].any()
    assert res["O"].numel() == 0


def test_pack_respects_capacity(require_gpu):
    """slot_capacity below S truncates the pack; nothing past the capacity is written."""
    import torch
    import block_sparse_attention_rank_amd as bsa
    from _gpu import run_path, to_host_u16, union_host
    w = custom(H=2, d=64, b=64, T=2, HW=512, G=2, r=0, density=0.6)
    inp = make_inputs(w)
    res = run_path(inp, attention=False)
    got = union_host(res["union"])
    cap = got["S"] // 2
    buf = torch.full((got["S"], 2, w.b * w.d), 7.0, dtype=torch.bfloat16, device="cuda")
    bsa.pack_kv(res["g"], res["dev"]["K"], res["dev"]["V"], res["union"], out=buf[:cap])
    torch.cuda.synchronize()
    expect = O.pack(inp["K"], inp["V"], got["slot_block"], got["slot_head"], w.b)
    host = to_host_u16(buf)
    assert np.array_equal(host[:cap], expect[:cap])
    assert np.all(host[cap:] == 0x40E0)                          # bf16 7.0 untouched


def test_repeat_runs_are_bit_identical(require_gpu):
    from _gpu import run_path, to_host_u16
    inp = make_inputs(custom(H=3, d=128, b=128, T=3, HW=1000, G=4, r=1, density=0.4))
    a = run_path(inp)
    b = run_path(inp, dev=a["dev"])
    for key in ("seg_offsets", "slot_of", "demand"):
        assert np.array_equal(getattr(a["union"], key).cpu().numpy(), getattr(b["union"], key).cpu().numpy())
    S = int(a["union"].seg_offsets[-1].item())
    assert np.array_equal(to_host_u16(a["packed"][:S]), to_host_u16(b["packed"][:S]))
    assert np.array_equal(a["O"].cpu().numpy(), b["O"].cpu().numpy())
    assert np.array_equal(a["lse"].cpu().numpy(), b["lse"].cpu().numpy())


SEGMENT_CASES = {
    "small": None,
    "seg_d128_periodic": custom(H=2, d=128, b=128, T=3, HW=1280, G=4, r=1, placement="periodic", density=0.4),
    "seg_d64_ragged": custom(H=2, d=64, b=64, T=5, HW=200, G=3, r=2, density=0.5, k_offset_sigma=6.0),
    "hunyuan": None,
}


@pytest.mark.parametrize("name", list(SEGMENT_CASES))
def test_segments_and_merge(require_gpu, name):
    """Attention over each source rank's segment of the payload, then the log-sum-exp merge in ring order
    (the local segment first, then ring distance 1, 2, ...): every segment and the merged result match the
    oracle, and the merged result matches the single pass."""
    import torch
    import block_sparse_attention_rank_amd as bsa
    from _gpu import run_path
    w = SEGMENT_CASES[name]
    inp = _inputs(name) if w is None else make_inputs(w)
    w = inp["workload"]
    print(f"[parity] segments {name}", flush=True)
    res = run_path(inp)
    g, u = res["g"], res["union"]
    dev = res["dev"]
    ranges = bsa.segment_ranges(u.seg_offsets.cpu().numpy(), w.H, w.G)
    scale = 1.0 / math.sqrt(w.d)
    acc_O = torch.zeros_like(res["O"])
    acc_lse = torch.full_like(res["lse"], float("-inf"))
    order = [(w.r + k) % w.G for k in range(w.G)]
    for p in order:
        lo, hi = ranges[p]
        O_p, lse_p = bsa.block_sparse_attn_segment(g, dev["Q"], dev["mask"], u.slot_of, res["packed"], lo, hi, scale)
        bsa.merge_partial(g, acc_O, acc_lse, O_p, lse_p)
        torch.cuda.synchronize()
        _check_attention(inp, O_p.cpu().numpy(), lse_p.cpu().numpy(), segment=p)
    mx, mean = _check_attention(inp, acc_O.cpu().numpy(), acc_lse.cpu().numpy())
    real = O.real_rows(inp["q_blocks"], w.b, w.N)
    d_single = np.abs(acc_O.cpu().numpy()[:, real] - res["O"].cpu().numpy()[:, real])
    # both are within MAX_ABS of the exact result; they differ in where the probabilities were rounded to
    # bf16 (relative to each piece's running maximum), so they agree to the sum of the two distances
    assert d_single.max() <= 2 * MAX_ABS, d_single.max()
    print(f"[parity] segments {name}: merged max {mx:.2e}, vs single pass {d_single.max():.2e}", flush=True)


@pytest.mark.parametrize("name", list(SEGMENT_CASES))
def test_segment_accumulate(require_gpu, name):
    """The fused segment call folds each segment into the running (O, lse) in place, in ring order and in
    reverse order: the result matches the oracle's full attention and the two-call path (segment + merge)."""
    import torch
    import block_sparse_attention_rank_amd as bsa
    from _gpu import run_path
    w = SEGMENT_CASES[name]
    inp = _inputs(name) if w is None else make_inputs(w)
    w = inp["workload"]
    print(f"[parity] segment accumulate {name}", flush=True)
    res = run_path(inp)
    g, u, dev = res["g"], res["union"], res["dev"]
    ranges = bsa.segment_ranges(u.seg_offsets.cpu().numpy(), w.H, w.G)
    scale = 1.0 / math.sqrt(w.d)
    ring = [(w.r + k) % w.G for k in range(w.G)]
    results = []
    for order in (ring, ring[::-1]):
        O_run = torch.zeros_like(res["O"])
        lse_run = torch.full_like(res["lse"], float("-inf"))
        two_O = torch.zeros_like(res["O"])
        two_lse = torch.full_like(res["lse"], float("-inf"))
        for p in order:
            lo, hi = ranges[p]
            bsa.block_sparse_attn_segment_accumulate(g, dev["Q"], dev["mask"], u.slot_of, res["packed"], lo, hi,
                                                     O_run, lse_run, scale)
            O_p, lse_p = bsa.block_sparse_attn_segment(g, dev["Q"], dev["mask"], u.slot_of, res["packed"], lo, hi,
                                                       scale)
            bsa.merge_partial(g, two_O, two_lse, O_p, lse_p)
        torch.cuda.synchronize()
        _check_attention(inp, O_run.cpu().numpy(), lse_run.cpu().numpy())
        real = O.real_rows(inp["q_blocks"], w.b, w.N)
        # the fused and two-call paths round the same partial results; only the merge arithmetic differs
        d_two = np.abs(O_run.cpu().numpy()[:, real] - two_O.cpu().numpy()[:, real])
        assert d_two.max() <= 1e-5, d_two.max()
        l_run, l_two = lse_run.cpu().numpy()[:, real], two_lse.cpu().numpy()[:, real]
        assert np.array_equal(np.isfinite(l_run), np.isfinite(l_two))
        fin = np.isfinite(l_two)
        assert np.abs(l_run[fin] - l_two[fin]).max() <= 1e-5 * max(1.0, float(np.abs(l_two[fin]).max()))
        results.append(O_run.cpu().numpy()[:, real])
    assert np.abs(results[0] - results[1]).max() <= 2 * MAX_ABS


def test_segment_accumulate_leaves_untouched_rows(require_gpu):
    """A segment with no selected block for some query blocks leaves their running rows bit-for-bit as they
    were (here: a sentinel), and an empty slot range touches nothing."""
    import torch
    import block_sparse_attention_rank_amd as bsa
    from _gpu import run_path
    inp = make_inputs(custom(H=2, d=64, b=64, T=4, HW=640, G=4, r=0, mask_kind="identity"))
    w = inp["workload"]
    res = run_path(inp)
    g, u, dev = res["g"], res["union"], res["dev"]
    ranges = bsa.segment_ranges(u.seg_offsets.cpu().numpy(), w.H, w.G)
    O_run = torch.full_like(res["O"], 7.0)
    lse_run = torch.full_like(res["lse"], 3.0)
    for p in range(1, w.G):                      # identity mask: rank 0's rows select only rank 0's blocks
        lo, hi = ranges[p]
        assert lo == hi
        bsa.block_sparse_attn_segment_accumulate(g, dev["Q"], dev["mask"], u.slot_of, res["packed"], lo, hi,
                                                 O_run, lse_run)
    bsa.block_sparse_attn_segment_accumulate(g, dev["Q"], dev["mask"], u.slot_of, res["packed"], 0, 0, O_run, lse_run)
    torch.cuda.synchronize()
    assert torch.all(O_run == 7.0) and torch.all(lse_run == 3.0)


def test_maximum_blocks(require_gpu):
    """nb = 16384 (the library's limit) with 16 ranks under periodic placement: union, compaction and the
    pack bit-exact; attention on every query block."""
    from _gpu import run_path, to_host_u16, union_host
    w = custom(H=1, d=64, b=64, T=16, HW=65536, G=16, r=5, placement="periodic", density=0.002)
    assert w.nb == 16384
    inp = make_inputs(w)
    print(f"[parity] maximum blocks: nb={w.nb} Lq={len(inp['q_blocks'])}", flush=True)
    res = run_path(inp)
    c = _check_union(union_host(res["union"]), inp)
    assert np.array_equal(to_host_u16(res["packed"][:c["S"]]),
                          O.pack(inp["K"], inp["V"], c["slot_block"], c["slot_head"], w.b))
    _check_attention(inp, res["O"].cpu().numpy(), res["lse"].cpu().numpy())


def test_segment_accumulate_is_deterministic(require_gpu):
    """Folding the same segments in the same order twice gives bit-identical (O, lse)."""
    import torch
    import block_sparse_attention_rank_amd as bsa
    from _gpu import run_path
    inp = make_inputs(custom(H=3, d=128, b=128, T=3, HW=1000, G=4, r=1, density=0.4))
    w = inp["workload"]
    res = run_path(inp)
    g, u, dev = res["g"], res["union"], res["dev"]
    ranges = bsa.segment_ranges(u.seg_offsets.cpu().numpy(), w.H, w.G)
    outs = []
    for _ in range(2):
        O_run = torch.zeros_like(res["O"])
        lse_run = torch.full_like(res["lse"], float("-inf"))
        for p in [(w.r + k) % w.G for k in range(w.G)]:
            bsa.block_sparse_attn_segment_accumulate(g, dev["Q"], dev["mask"], u.slot_of, res["packed"], *ranges[p],
                                                     O_run, lse_run)
        torch.cuda.synchronize()
        outs.append((O_run.cpu().numpy(), lse_run.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
