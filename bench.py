#!/usr/bin/env python3
"""Benchmark one sequence-parallel rank's share of block-sparse attention on one MI355X.

A step is one pass of the whole hot path over one synthetic workload already resident in HBM:
demand union + compaction (sparsp_demand_union), the K/V pack (sparsp_pack_kv) and block-sparse
attention (sparsp_block_sparse_attn), all enqueued on torch's current stream.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config hunyuan] [--no-cpu]

Prints one JSON line.  ``value`` is the effective attention throughput of the whole step: the
algorithmic FLOPs of the selected tiles (4*b*b*d per selected (head, query block, key block)) divided by
the step time.  Per-kernel durations come from HIP events recorded on the launch stream around every
call in the timed steps.  After them, a few cold-cache repetitions time the pack and the attention with
the L2s and the Infinity Cache flushed before each.  ``cpu_baseline`` times the fp64 CPU oracle on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_DENSE_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "block-sparse attn effective TFLOP/s + KV pack GB/s, one rank's share"
COLD_REPS = 5                  # cold-cache repetitions after the timed steps
FLUSH_BYTES = 512 << 20        # read before a cold launch: twice the 256 MB Infinity Cache


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="hunyuan")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-comm", action="store_true", help="skip the communication-volume accounting")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle attention sample")
    ap.add_argument("--cold-reps", type=int, default=COLD_REPS,
                    help="repetitions with the caches flushed before the pack and before the attention")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the warmup, run one plain float32 device copy of this many MiB (read + write of "
                         "known size) so profiler byte counters can be scaled against it")
    return ap.parse_args()


# The source file of each profiled kernel; its digest (with the shared internal header) tells whether a
# stored counter measurement still describes the kernel being run.
KERNEL_SOURCES = {"bsa_fwd": "attention.hip", "pack": "pack.hip", "permute": "permute.hip", "pool": "materialize.hip",
                  "select": "materialize.hip", "union": "union_compact.hip", "counts": "accounting.hip",
                  "merge": "merge.hip"}


def kernel_sources_digest(kernel: str | None = None) -> str:
    """Digest of one kernel's source file and the shared internal header (all sources when kernel is None)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_attention_rank_amd", "csrc")
    names = sorted(os.listdir(csrc)) if kernel is None else ["sparsp_internal.h", KERNEL_SOURCES[kernel]]
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches these sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("sources_digest") != kernel_sources_digest(kernel):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(inp, budget_s: float, pairs: int, attn_flops: float):
    """Time the CPU oracle: union + compaction + pack on the whole workload, attention on as many
    (head, query block) items as fit in the budget; extrapolate the attention to all items."""
    import numpy as np
    import oracle as O

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    w = inp["workload"]
    t0 = time.perf_counter()
    U = O.demand_union(inp["mask"], w.nb)
    c = O.compact(U, inp["placement"], w.G)
    t_union = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.pack(inp["K"], inp["V"], c["slot_block"], c["slot_head"], w.b)
    t_pack = time.perf_counter() - t0
    H, Lq = w.H, len(inp["q_blocks"])
    rng = np.random.default_rng(0)
    order = rng.permutation(H * Lq)
    scale = 1.0 / math.sqrt(w.d)
    done_pairs, n_items, t_attn = 0, 0, 0.0
    for idx in order:
        h, k = divmod(int(idx), Lq)
        t0 = time.perf_counter()
        O.attention_block(inp["Q"], inp["K"], inp["V"], inp["mask"], h, k, w.b, w.N, scale)
        t_attn += time.perf_counter() - t0
        done_pairs += int(inp["mask"][h, k, :w.nb].sum())
        n_items += 1
        if t_attn >= budget_s:
            break
    t_attn_full = t_attn * pairs / max(done_pairs, 1)
    t_step = t_union + t_pack + t_attn_full
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:  # pragma: no cover
        pass
    slot_bytes = 2 * w.b * w.d * 2
    return {
        "value": attn_flops / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": (f"fp64 NumPy oracle on {w.name}: union+compaction and pack on the whole workload "
                   f"({t_union:.2f} s, {t_pack:.2f} s); attention on {n_items} of {H * Lq} (head, query block) "
                   f"items ({done_pairs} of {pairs} tiles, {t_attn:.1f} s), extrapolated by tile count to "
                   f"{t_attn_full:.0f} s; value = all tiles' FLOPs / ({t_union:.2f} + {t_pack:.2f} + "
                   f"{t_attn_full:.0f}) s"),
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model,
        "union_compact_s": round(t_union, 4),
        "union_mask_GBps": round(inp["mask"].size / t_union / 1e9, 3),
        "pack_s": round(t_pack, 4),
        "pack_GBps": round(2 * len(c["slot_block"]) * slot_bytes / t_pack / 1e9, 3),
        "attn_sample_s": round(t_attn, 2),
        "attn_GFLOPs": round(4.0 * w.b * w.b * w.d * done_pairs / t_attn / 1e9, 2),
    }


def comm_accounting(w, inp, g, torch, bsa):
    """Communication volume of the workload's masks, every logical row drawn, for G = 2, 4, 8 under the
    contiguous and the periodic placement: blocks moved by demand-directed delivery, by a relaying ring
    and by a dense ring (sections 3.1, 3.3 and 5.1), from the GPU's demand unions of every rank's rows.
    Also the Figure 4 sharing metric of this rank's received remote blocks."""
    import dataclasses

    import numpy as np
    from workloads.configs import make_mask, placement_for

    mask_all = make_mask(w, np.arange(w.nb, dtype=np.int32))
    dev_all = torch.from_numpy(mask_all).cuda()
    slot_bytes = 2 * w.b * w.d * 2
    table = []
    for placement in ("contiguous", "periodic"):
        for G in (2, 4, 8):
            wg = dataclasses.replace(w, G=G, placement=placement, r=0)
            P = placement_for(wg)
            Pd = torch.from_numpy(P).cuda()
            words = []
            for c in range(G):
                q = np.flatnonzero(P == c)
                gc = bsa.geometry(H=w.H, d=w.d, b=w.b, N=w.N, G=G, r=c, Lq=len(q))
                rows = dev_all[:, torch.from_numpy(q).cuda(), :].contiguous()
                words.append(bsa.demand_union(gc, rows, Pd).demand.cpu().numpy().view(np.uint64))
            v = bsa.comm_volume(np.stack(words), P, G)
            n = np.bincount(P, minlength=G)
            remote_dense = int(sum(w.H * (w.nb - n[c]) for c in range(G)))
            direct, relay, dense = int(v["direct"].sum()), int(v["relay"].sum()), int(v["dense"].sum())
            table.append({
                "placement": placement, "G": G,
                "direct_blocks": direct, "relay_block_hops": relay, "dense_ring_block_hops": dense,
                "direct_GB": round(direct * slot_bytes / 1e9, 3), "relay_GB": round(relay * slot_bytes / 1e9, 3),
                "dense_ring_GB": round(dense * slot_bytes / 1e9, 3),
                "reduction_vs_all_remote": round(1 - direct / remote_dense, 4) if remote_dense else None,
                "relay_over_direct": round(relay / direct, 3) if direct else None,
            })
    # Figure 4: how many of this rank's local query blocks use each remote block it receives
    Lq = len(inp["q_blocks"])
    mask_d = torch.from_numpy(inp["mask"]).cuda()
    cnt = bsa.demand_counts(g, mask_d)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    evs[0].record()
    for _ in range(10):
        bsa.demand_counts(g, mask_d, out=cnt)
    evs[1].record()
    torch.cuda.synchronize()
    c = cnt.cpu().numpy()
    remote = (inp["placement"][None, :] != w.r) & (c > 0)
    frac = c[remote] / max(1, Lq)
    return {
        "placements": table,
        "sharing_rank_r": {"remote_blocks": int(remote.sum()),
                           "used_by_ge_10pct": round(float((frac >= 0.10).mean()), 4) if frac.size else None,
                           "used_by_ge_30pct": round(float((frac >= 0.30).mean()), 4) if frac.size else None},
        "counts_kernel_us": round(evs[0].elapsed_time(evs[1]) * 100, 2),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share only; --gpus {args.gpus} is not supported (use --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_attention_rank_amd as bsa
    from workloads import CONFIGS, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    w = CONFIGS[args.config]
    t0 = time.perf_counter()
    inp = make_inputs(w)
    print(f"[bench] inputs for {w.name} drawn in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    Lq = len(inp["q_blocks"])
    g = bsa.geometry(H=w.H, d=w.d, b=w.b, N=w.N, G=w.G, r=w.r, Lq=Lq)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    mask = torch.from_numpy(inp["mask"]).cuda()
    placement = torch.from_numpy(inp["placement"]).cuda()
    Q, K, V = bf16(inp["Q"]), bf16(inp["K"]), bf16(inp["V"])
    u = bsa.empty_union(g)
    packed = torch.empty((g.H * g.nb, 2, g.b * g.d), dtype=torch.bfloat16, device="cuda")
    O = torch.empty((g.H, Lq * g.b, g.d), dtype=torch.float32, device="cuda")
    lse = torch.empty((g.H, Lq * g.b), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(g.d)
    stream = torch.cuda.current_stream()

    pairs = int(inp["mask"][:, :, :w.nb].astype(np.int64).sum())
    attn_flops = 4.0 * g.b * g.b * g.d * pairs
    mask_bytes = int(inp["mask"].size)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        bsa.demand_union(g, mask, placement, out=u)
        if ev is not None:
            ev[1].record(stream)
        bsa.pack_kv(g, K, V, u, out=packed)
        if ev is not None:
            ev[2].record(stream)
        bsa.block_sparse_attn(g, Q, mask, u.slot_of, packed, scale, out=(O, lse))
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    S = int(u.seg_offsets[-1].item())
    seg = u.seg_offsets.cpu().numpy()
    own_lo, own_hi = int(seg[w.r * g.H]), int(seg[(w.r + 1) * g.H])
    slot_bytes = 2 * g.b * g.d * 2
    pack_bytes = 2 * S * slot_bytes            # read + write

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = lambda a, b: float(np.mean([e[a].elapsed_time(e[b]) for e in events]))  # noqa: E731
    t_union, t_pack, t_attn = ms(0, 1), ms(1, 2), ms(2, 3)
    warm_pack = [e[1].elapsed_time(e[2]) for e in events]
    warm_attn = [e[2].elapsed_time(e[3]) for e in events]
    ms_per_step = wall * 1e3 / args.steps
    print(f"[bench] {w.name}: union {t_union * 1e3:.1f} us, pack {t_pack * 1e3:.1f} us, "
          f"attention {t_attn:.3f} ms, step {ms_per_step:.3f} ms", file=sys.stderr, flush=True)

    # Cold caches: before the union + pack and again before the attention, a read of twice the Infinity
    # Cache's size evicts the L2s and the Infinity Cache, so each timed kernel starts with its inputs in HBM.
    # A read, not a write: a written flush buffer would leave dirty lines whose write-back the next kernel
    # pays for (measured: 40 us, 8 %, on the hunyuan pack).
    cold = None
    if args.cold_reps > 0:
        flush = torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device="cuda")
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.cold_reps)]
        for e in cev:
            flush.sum()
            e[0].record(stream)
            bsa.demand_union(g, mask, placement, out=u)
            e[1].record(stream)
            bsa.pack_kv(g, K, V, u, out=packed)
            e[2].record(stream)
            flush.sum()
            e[3].record(stream)
            bsa.block_sparse_attn(g, Q, mask, u.slot_of, packed, scale, out=(O, lse))
            e[4].record(stream)
        torch.cuda.synchronize()
        del flush
        c_union = [e[0].elapsed_time(e[1]) for e in cev]
        c_pack = [e[1].elapsed_time(e[2]) for e in cev]
        c_attn = [e[3].elapsed_time(e[4]) for e in cev]
        cold = {
            "reps": args.cold_reps,
            "union_compact_us_median": round(float(np.median(c_union)) * 1e3, 2),
            "pack_us_median": round(float(np.median(c_pack)) * 1e3, 2),
            "pack_us_min": round(min(c_pack) * 1e3, 2),
            "pack_GBps_median": round(pack_bytes / (float(np.median(c_pack)) * 1e-3) / 1e9, 1),
            "attn_ms_median": round(float(np.median(c_attn)), 4),
            "attn_ms_min": round(min(c_attn), 4),
            "attn_TFLOPs_median": round(attn_flops / (float(np.median(c_attn)) * 1e-3) / 1e12, 2),
        }
        print(f"[bench] {w.name}: cold caches: pack {cold['pack_us_median']:.1f} us, attention "
              f"{cold['attn_ms_median']:.3f} ms (medians of {args.cold_reps})", file=sys.stderr, flush=True)

    # Segment-wise consumption: attention over each source rank's segment (local first, then ring
    # distance 1, 2, ...) and the log-sum-exp merge of the partial results, as the payload would arrive.
    ranges = bsa.segment_ranges(seg, g.H, g.G)
    order = [(w.r + k) % w.G for k in range(w.G)]
    parts = [(torch.empty_like(O), torch.empty_like(lse)) for _ in order]
    accO, accL = torch.empty_like(O), torch.empty_like(lse)
    seg_steps = max(3, args.steps // 4)

    def seg_step(ev=None):
        accO.zero_()
        accL.fill_(float("-inf"))
        for i, p in enumerate(order):
            if ev is not None:
                ev[2 * i].record(stream)
            bsa.block_sparse_attn_segment(g, Q, mask, u.slot_of, packed, ranges[p][0], ranges[p][1], scale,
                                          out=parts[i])
            if ev is not None:
                ev[2 * i + 1].record(stream)
            bsa.merge_partial(g, accO, accL, *parts[i])
        if ev is not None:
            ev[2 * len(order)].record(stream)

    seg_step()
    torch.cuda.synchronize()
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(order) + 1)] for _ in range(seg_steps)]
    for i in range(seg_steps):
        seg_step(sev[i])
    torch.cuda.synchronize()
    seg_total = float(np.mean([e[0].elapsed_time(e[-1]) for e in sev]))
    seg_attn = float(np.mean([sum(e[2 * i].elapsed_time(e[2 * i + 1]) for i in range(len(order))) for e in sev]))
    merge_ms = (seg_total - seg_attn) / max(1, len(order))
    merge_bytes = (3 * O.numel() + 3 * lse.numel()) * 4  # read O, O_part, lse x2; write O, lse
    print(f"[bench] {w.name}: segmented attention {seg_total:.3f} ms ({len(order)} segments), merge "
          f"{merge_ms * 1e3:.1f} us each", file=sys.stderr, flush=True)

    # The same consumption with the fused call: each segment folded straight into the running result.
    def fused_step():
        accO.zero_()
        accL.fill_(float("-inf"))
        for p in order:
            bsa.block_sparse_attn_segment_accumulate(g, Q, mask, u.slot_of, packed, ranges[p][0], ranges[p][1], accO,
                                                     accL, scale)

    fused_step()
    torch.cuda.synchronize()
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(seg_steps)]
    for e in fev:
        accO.zero_()
        accL.fill_(float("-inf"))
        e[0].record(stream)
        for p in order:
            bsa.block_sparse_attn_segment_accumulate(g, Q, mask, u.slot_of, packed, ranges[p][0], ranges[p][1], accO,
                                                     accL, scale)
        e[1].record(stream)
    torch.cuda.synchronize()
    fused_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in fev]))
    print(f"[bench] {w.name}: segmented attention, fused fold {fused_ms:.3f} ms", file=sys.stderr, flush=True)

    # Placement permutation (section 4.3) of the layer's hidden states [nb*b][H*d] bf16 into rank-major
    # block order and back: each call reads and writes every byte once.
    pos, _ = bsa.placement_permutation(inp["placement"], g.G)
    pos_d = torch.from_numpy(pos).cuda()
    hidden = torch.randn((g.nb * g.b, g.H * g.d), device="cuda").to(torch.bfloat16)
    hidden_p = torch.empty_like(hidden)
    hidden_r = torch.empty_like(hidden)
    for _ in range(2):
        bsa.permute_blocks(hidden, pos_d, g.b, out=hidden_p)
        bsa.permute_blocks(hidden_p, pos_d, g.b, inverse=True, out=hidden_r)
    perm_steps = max(3, args.steps // 2)
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(perm_steps)]
    for e in pev:
        e[0].record(stream)
        bsa.permute_blocks(hidden, pos_d, g.b, out=hidden_p)
        e[1].record(stream)
        bsa.permute_blocks(hidden_p, pos_d, g.b, inverse=True, out=hidden_r)
        e[2].record(stream)
    torch.cuda.synchronize()
    assert torch.equal(hidden_r, hidden), "permutation round trip changed the hidden states"
    t_perm = float(np.mean([e[0].elapsed_time(e[1]) for e in pev]))
    t_iperm = float(np.mean([e[1].elapsed_time(e[2]) for e in pev]))
    perm_bytes = 2 * hidden.numel() * hidden.element_size()
    del hidden, hidden_p, hidden_r
    print(f"[bench] {w.name}: permutation of hidden states {t_perm * 1e3:.1f} us, inverse {t_iperm * 1e3:.1f} us",
          file=sys.stderr, flush=True)

    # Mask materialisation from pooled tiles (section 4.2): pool K (every block) and the local Q blocks,
    # then score and select every local row (Top-p 0.9 with a Top-k floor of 16 blocks).
    mat = None
    if g.nb <= 4096:
        ids_d = torch.from_numpy(inp["q_blocks"]).cuda()
        kp = bsa.pool_blocks(g, K)
        qp = bsa.pool_blocks(g, Q, block_ids=ids_d)
        mat_mask = bsa.materialize_mask(g, qp, kp, 0.9, 16)
        mev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(max(3, args.steps // 2))]
        for e in mev:
            e[0].record(stream)
            bsa.pool_blocks(g, K, out=kp)
            e[1].record(stream)
            bsa.pool_blocks(g, Q, block_ids=ids_d, out=qp)
            e[2].record(stream)
            bsa.materialize_mask(g, qp, kp, 0.9, 16, out=mat_mask)
            e[3].record(stream)
        torch.cuda.synchronize()
        t_pk, t_pq, t_sel = (float(np.mean([e[i].elapsed_time(e[i + 1]) for e in mev])) for i in range(3))
        k_bytes = K.numel() * 2 * w.N // (g.nb * g.b)          # real rows of K are read
        mat = {"pool_k_us": round(t_pk * 1e3, 2), "pool_k_GBps": round(k_bytes / (t_pk * 1e-3) / 1e9, 1),
               "pool_q_us": round(t_pq * 1e3, 2), "select_us": round(t_sel * 1e3, 2),
               "tau": 0.9, "k_min": 16,
               "density": round(float(mat_mask[:, :, :g.nb].float().mean().item()), 4)}
        del kp, qp, mat_mask
        print(f"[bench] {w.name}: mask materialisation: pool K {t_pk * 1e3:.1f} us, pool Q {t_pq * 1e3:.1f} us, "
              f"select {t_sel * 1e3:.1f} us", file=sys.stderr, flush=True)

    comm = None
    if not args.no_comm and g.nb <= 1024:
        t0 = time.perf_counter()
        comm = comm_accounting(w, inp, g, torch, bsa)
        print(f"[bench] {w.name}: communication accounting took {time.perf_counter() - t0:.1f} s", file=sys.stderr,
              flush=True)

    attn_tflops = attn_flops / (t_attn * 1e-3) / 1e12
    pack_gbs = pack_bytes / (t_pack * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(attn_flops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.note}",
            "H": g.H, "d": g.d, "b": g.b, "N": g.N, "nb": g.nb, "G": g.G, "r": g.r, "Lq": Lq,
            "placement": w.placement, "selected_tiles": pairs,
            "density": round(pairs / (g.H * Lq * g.nb), 4),
            "slots_S": S, "union_fraction": round(S / (g.H * g.nb), 4),
            "wire_slots": S - (own_hi - own_lo), "wire_bytes": (S - (own_hi - own_lo)) * slot_bytes,
        },
        "components": {
            "union_compact_us": round(t_union * 1e3, 2),
            "union_mask_GBps": round(mask_bytes / (t_union * 1e-3) / 1e9, 1),
            "pack_us": round(t_pack * 1e3, 2),
            "pack_GBps": round(pack_gbs, 1),
            "pack_frac_hbm": round(pack_gbs / HBM_PEAK_GBS, 4),
            "attn_ms": round(t_attn, 4),
            "attn_TFLOPs": round(attn_tflops, 2),
            "attn_frac_bf16": round(attn_tflops / BF16_DENSE_TFLOPS, 4),
            "warm": {"pack_us_median": round(float(np.median(warm_pack)) * 1e3, 2),
                     "pack_us_min": round(min(warm_pack) * 1e3, 2),
                     "attn_ms_median": round(float(np.median(warm_attn)), 4),
                     "attn_ms_min": round(min(warm_attn), 4)},
            "cold": cold,
            "segmented_attn_ms": round(seg_total, 4),
            "segmented_attn_TFLOPs": round(attn_flops / (seg_total * 1e-3) / 1e12, 2),
            "merge_us": round(merge_ms * 1e3, 2),
            "segmented_fused_attn_ms": round(fused_ms, 4),
            "segmented_fused_attn_TFLOPs": round(attn_flops / (fused_ms * 1e-3) / 1e12, 2),
            "merge_GBps": round(merge_bytes / (merge_ms * 1e-3) / 1e9, 1) if merge_ms > 0 else None,
            "permute_hidden_bytes": perm_bytes,
            "permute_us": round(t_perm * 1e3, 2),
            "permute_GBps": round(perm_bytes / (t_perm * 1e-3) / 1e9, 1),
            "permute_inverse_us": round(t_iperm * 1e3, 2),
            "permute_inverse_GBps": round(perm_bytes / (t_iperm * 1e-3) / 1e9, 1),
        },
        "roofline": {
            "kernel": "bsa_fwd_kernel",
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / BF16_DENSE_TFLOPS, 4),
            "traffic": measured_traffic("bsa_fwd", w.name),
        },
        "roofline_pack": {
            "kernel": "pack_kernel",
            "bound": "hbm",
            "achieved": round(pack_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(pack_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("pack", w.name),
        },
        "comm_volume": comm,
        "mask_materialisation": mat,
        "sources_digest": {k: kernel_sources_digest(k) for k in ("bsa_fwd", "pack")},
    }
    if not args.no_cpu:
        t0 = time.perf_counter()
        rec["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds, pairs, attn_flops)
        print(f"[bench] cpu baseline took {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
