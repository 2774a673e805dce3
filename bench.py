#!/usr/bin/env python3
"""Benchmark one sequence-parallel rank's share of block-sparse attention on one MI355X.

A step is one pass of the whole hot path over one synthetic workload already resident in HBM:
demand union + compaction (sparsp_demand_union), the K/V pack (sparsp_pack_kv) and block-sparse
attention (sparsp_block_sparse_attn), all enqueued on torch's current stream.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config hunyuan] [--extra tiny,small,wan,ltx] [--no-cpu]

Prints one JSON line.  ``value`` is the effective attention throughput of the whole step on the headline
workload: the algorithmic FLOPs of the selected tiles (4*b*b*d per selected (head, query block, key block))
divided by the step time.  Per-kernel durations come from HIP events recorded on the launch stream around
every call in the timed steps; the shader clock over the timed steps, and over a run of attention launches
alone, comes from a clock sampler on a side stream.  The same run measures a dense bf16 GEMM and a device
copy as ceilings, times cold-cache repetitions, the segment and chunk folds of the payload, the placement
permutation, the mask materialisation and the communication-volume accounting, repeats the core
measurements on the other workloads (``extra_configs``), and times the fp64 CPU oracle on the headline
workload (``cpu_baseline``).
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
PEAK_CLOCK_GHZ = 2.4           # the clock the published peaks are stated at
METRIC = "block-sparse attn effective TFLOP/s + KV pack GB/s, one rank's share"
COLD_REPS = 5                  # cold-cache repetitions after the timed steps
FLUSH_BYTES = 512 << 20        # read before a cold launch: twice the 256 MB Infinity Cache
CHUNK_PLANS = ((1, 1), (1, 2), (1, 4), (2, 4), (1, 8), (4, 24))


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="hunyuan", help="headline workload")
    ap.add_argument("--extra", default="tiny,small,wan,ltx",
                    help="other workloads measured after the headline (comma-separated; empty for none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-comm", action="store_true", help="skip the communication-volume accounting")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the dense GEMM and device copy ceilings")
    ap.add_argument("--cpu-seconds", type=float, default=90.0,
                    help="time limit of the oracle attention; items past it are extrapolated by tile count")
    ap.add_argument("--cold-reps", type=int, default=COLD_REPS,
                    help="repetitions with the caches flushed before the pack and before the attention")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the warmup, run one plain float32 device copy of this many MiB (read + write of "
                         "known size) so profiler byte counters can be scaled against it")
    return ap.parse_args(argv)


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


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(inp, budget_s: float, pairs: int, attn_flops: float):
    """Time the CPU oracle on the whole workload: union + compaction and pack, then the attention of every
    (head, query block) item, the items spread over the host's cores (at most 16 threads, BLAS one thread
    per call).  Items left when ``budget_s`` runs out are extrapolated by tile count (none at the default
    budget on the shares measured here)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle as O
    from threadpoolctl import threadpool_limits

    w = inp["workload"]
    t0 = time.perf_counter()
    U = O.demand_union(inp["mask"], w.nb)
    c = O.compact(U, inp["placement"], w.G)
    t_union = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.pack(inp["K"], inp["V"], c["slot_block"], c["slot_head"], w.b)
    t_pack = time.perf_counter() - t0
    H, Lq = w.H, len(inp["q_blocks"])
    items = [(h, k) for h in range(H) for k in range(Lq)]
    scale = 1.0 / math.sqrt(w.d)
    workers = _workers()
    deadline = time.perf_counter() + budget_s

    def one(item):
        if time.perf_counter() > deadline:
            return 0
        h, k = item
        O.attention_block(inp["Q"], inp["K"], inp["V"], inp["mask"], h, k, w.b, w.N, scale)
        return int(np.count_nonzero(inp["mask"][h, k, :w.nb]))

    t0 = time.perf_counter()
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        done = list(ex.map(one, items))
    t_attn = time.perf_counter() - t0
    done_pairs = int(sum(done))
    n_items = int(sum(1 for x in done if x > 0))
    t_attn_full = t_attn * pairs / max(done_pairs, 1)
    t_step = t_union + t_pack + t_attn_full
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:  # pragma: no cover
        pass
    slot_bytes = 2 * w.b * w.d * 2
    whole = done_pairs == pairs
    return {
        "value": attn_flops / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": int(workers),
        "kind": "oracle",
        "sample": (f"fp64 NumPy oracle on {w.name}, whole workload: union+compaction ({t_union:.2f} s), pack "
                   f"({t_pack:.2f} s) and attention of "
                   + (f"all {H * Lq} (head, query block) items ({pairs} tiles) in {t_attn:.1f} s"
                      if whole else
                      f"{n_items} of {H * Lq} items ({done_pairs} of {pairs} tiles, {t_attn:.1f} s), "
                      f"extrapolated by tile count to {t_attn_full:.0f} s")
                   + f" on {workers} threads; value = all tiles' FLOPs / total time"),
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model,
        "union_compact_s": round(t_union, 4),
        "union_mask_GBps": round(inp["mask"].size / max(t_union, 1e-9) / 1e9, 3),
        "pack_s": round(t_pack, 4),
        "pack_GBps": round(2 * len(c["slot_block"]) * slot_bytes / max(t_pack, 1e-9) / 1e9, 3),
        "attn_s": round(t_attn, 2),
        "attn_items": n_items,
        "attn_GFLOPs": round(4.0 * w.b * w.b * w.d * done_pairs / max(t_attn, 1e-9) / 1e9, 2),
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
    del mask_all
    slot_bytes = 2 * w.b * w.d * 2
    table = []
    for placement in ("contiguous", "periodic"):
        for G in (2, 4, 8):
            wg = dataclasses.replace(w, G=G, placement=placement, r=0)
            P = placement_for(wg)
            Pd = torch.from_numpy(P).cuda()
            words = []
            for c in range(G):
                q = bsa.local_query_blocks(P, G, c)
                gc = bsa.geometry(H=w.H, d=w.d, b=w.b, N=w.N, G=G, r=c, Lq=len(q))
                rows = dev_all[:, torch.from_numpy(q.astype(np.int64)).cuda(), :].contiguous()
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
    del dev_all
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


def _ms(evs, a, b):
    return [e[a].elapsed_time(e[b]) for e in evs]


def ceilings(torch, bsa, copy_bytes: int):
    """Same-run ceilings: a dense bf16 GEMM (torch.matmul, 8192^3) with the shader clock it ran at, and a
    device-to-device copy of ``copy_bytes`` (read + write counted)."""
    import numpy as np
    from block_sparse_attention_rank_amd.measure import ClockWindow

    n = 8192
    a = torch.randn((n, n), device="cuda").to(torch.bfloat16)
    b = torch.randn((n, n), device="cuda").to(torch.bfloat16)
    c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    reps = 20
    stream = torch.cuda.current_stream()
    bt = b.t().contiguous().t()                    # the column-major form of b (same values)
    forms = {"nn": lambda: torch.matmul(a, b, out=c), "nt": lambda: torch.matmul(a, bt, out=c)}
    best = None
    for name, f in forms.items():
        for _ in range(3):
            f()
        cw = ClockWindow(max_seconds=0.2)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        cw.start(stream)
        for e in ev:
            e[0].record(stream)
            f()
            e[1].record(stream)
        cw.stop(stream)
        clk_form = cw.result()["ghz"]               # synchronises
        r = (float(np.median(_ms(ev, 0, 1))), clk_form, name)
        if best is None or r[0] < best[0]:
            best = r
    t, clk_ghz, form = best
    clk = {"ghz": clk_ghz}
    gemm_tflops = 2.0 * n ** 3 / (t * 1e-3) / 1e12
    del a, b, bt, c
    src = torch.empty(copy_bytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(10)]
    for e in ev:
        e[0].record(stream)
        dst.copy_(src)
        e[1].record(stream)
    torch.cuda.synchronize()
    tc = float(np.median(_ms(ev, 0, 1)))
    del src, dst
    return {
        "gemm_bf16_8192_ms": round(t, 4),
        "gemm_bf16_TFLOPs": round(gemm_tflops, 1),
        "gemm_bf16_frac": round(gemm_tflops / BF16_DENSE_TFLOPS, 4),
        "gemm_clock_ghz": clk["ghz"],
        "gemm_form": form,
        "copy_bytes": 2 * copy_bytes,
        "copy_us": round(tc * 1e3, 2),
        "copy_GBps": round(2 * copy_bytes / (tc * 1e-3) / 1e9, 1),
        "copy_frac_hbm": round(2 * copy_bytes / (tc * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
    }


class Share:
    """One workload resident on the device, with its union, pack and attention buffers."""

    def __init__(self, name, torch, bsa):
        import numpy as np
        from workloads import CONFIGS, make_inputs

        self.torch, self.bsa = torch, bsa
        self.w = w = CONFIGS[name]
        t0 = time.perf_counter()
        self.inp = inp = make_inputs(w)
        q_blocks = bsa.local_query_blocks(inp["placement"], w.G, w.r)     # the local set, once per geometry
        assert np.array_equal(q_blocks, inp["q_blocks"])
        self.Lq = Lq = len(q_blocks)
        self.g = g = bsa.geometry(H=w.H, d=w.d, b=w.b, N=w.N, G=w.G, r=w.r, Lq=Lq)

        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

        self.mask = torch.from_numpy(inp["mask"]).cuda()
        self.placement = torch.from_numpy(inp["placement"]).cuda()
        self.Q, self.K, self.V = bf16(inp["Q"]), bf16(inp["K"]), bf16(inp["V"])
        self.u = bsa.empty_union(g)
        self.packed = torch.empty((g.H * g.nb, 2, g.b * g.d), dtype=torch.bfloat16, device="cuda")
        self.O = torch.empty((g.H, Lq * g.b, g.d), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((g.H, Lq * g.b), dtype=torch.float32, device="cuda")
        self.scale = 1.0 / math.sqrt(g.d)
        self.stream = torch.cuda.current_stream()
        self.pairs = int(inp["mask"][:, :, :w.nb].astype(np.int64).sum())
        self.attn_flops = 4.0 * g.b * g.b * g.d * self.pairs
        self.mask_bytes = int(inp["mask"].size)
        print(f"[bench] inputs for {w.name} drawn in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    def union(self):
        self.bsa.demand_union(self.g, self.mask, self.placement, out=self.u)

    def pack(self):
        self.bsa.pack_kv(self.g, self.K, self.V, self.u, out=self.packed)

    def attention(self):
        self.bsa.block_sparse_attn(self.g, self.Q, self.mask, self.u.slot_of, self.packed, self.scale,
                                   out=(self.O, self.lse))

    def step(self, ev=None):
        s = self.stream
        if ev is not None:
            ev[0].record(s)
        self.union()
        if ev is not None:
            ev[1].record(s)
        self.pack()
        if ev is not None:
            ev[2].record(s)
        self.attention()
        if ev is not None:
            ev[3].record(s)

    def fold(self, chunks):
        """The running (O, lse) from (0, -inf), every chunk folded in order (chunk_accumulate)."""
        self.O.zero_()
        self.lse.fill_(float("-inf"))
        for ch in chunks:
            self.bsa.block_sparse_attn_chunk_accumulate(self.g, self.Q, self.mask, self.u.slot_of, self.packed, ch,
                                                        self.O, self.lse, self.scale)

    def release(self):
        for k in ("mask", "placement", "Q", "K", "V", "u", "packed", "O", "lse"):
            setattr(self, k, None)
        self.torch.cuda.empty_cache()


def measure(sh: Share, steps: int, warmup: int, full: bool, args):
    """Timed steps and the components of one share.  ``full`` adds cold caches, the two-call segment path,
    the chunk sweep, the permutation and the mask materialisation."""
    import numpy as np
    from block_sparse_attention_rank_amd.measure import ClockWindow

    torch, bsa, g, w = sh.torch, sh.bsa, sh.g, sh.w
    stream = sh.stream
    for _ in range(warmup):
        sh.step()
    torch.cuda.synchronize()
    if full and args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    S = int(sh.u.seg_offsets[-1].item())
    seg = sh.u.seg_offsets.cpu().numpy()
    own_lo, own_hi = int(seg[w.r * g.H]), int(seg[(w.r + 1) * g.H])
    slot_bytes = 2 * g.b * g.d * 2
    pack_bytes = 2 * S * slot_bytes            # read + write

    # the timed steps: K steps between two synchronisations, events around every call
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        sh.step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_union, t_pack, t_attn = (float(np.mean(_ms(events, a, a + 1))) for a in range(3))
    warm_pack, warm_attn = _ms(events, 1, 2), _ms(events, 2, 3)
    ms_per_step = wall * 1e3 / steps

    # The same steps again with the shader clock sampled beside them, then attention launches alone with
    # their clock.  The sampler runs a little past each window and is waited for before the next one.
    cw = ClockWindow(max_seconds=1.5 * steps * ms_per_step * 1e-3 + 0.01)
    cw.start(stream)
    for i in range(steps):
        sh.step()
    cw.stop(stream)
    clk_steps = cw.result()
    reps = max(10, steps)
    aev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    cw = ClockWindow(max_seconds=1.5 * reps * t_attn * 1e-3 + 0.01)
    cw.start(stream)
    for e in aev:
        e[0].record(stream)
        sh.attention()
        e[1].record(stream)
    cw.stop(stream)
    clk_attn = cw.result()
    t_attn_alone = float(np.mean(_ms(aev, 0, 1)))
    print(f"[bench] {w.name}: union {t_union * 1e3:.1f} us, pack {t_pack * 1e3:.1f} us, attention {t_attn:.3f} ms "
          f"(alone {t_attn_alone:.3f} ms at {clk_attn['ghz']} GHz), step {ms_per_step:.3f} ms", file=sys.stderr,
          flush=True)

    attn_tflops = sh.attn_flops / (t_attn * 1e-3) / 1e12
    pack_gbs = pack_bytes / (t_pack * 1e-3) / 1e9
    out = {
        "config": {
            "workload": f"{w.name}: {w.note}",
            "H": g.H, "d": g.d, "b": g.b, "N": g.N, "nb": g.nb, "G": g.G, "r": g.r, "Lq": sh.Lq,
            "placement": w.placement, "selected_tiles": sh.pairs,
            "density": round(sh.pairs / max(1, g.H * sh.Lq * g.nb), 4),
            "slots_S": S, "union_fraction": round(S / (g.H * g.nb), 4),
            "wire_slots": S - (own_hi - own_lo), "wire_bytes": (S - (own_hi - own_lo)) * slot_bytes,
        },
        "ms_per_step": round(ms_per_step, 4),
        "value": round(sh.attn_flops / (ms_per_step * 1e-3) / 1e12, 3),
        "components": {
            "union_compact_us": round(t_union * 1e3, 2),
            "union_mask_GBps": round(sh.mask_bytes / (t_union * 1e-3) / 1e9, 1),
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
            "clock_ghz_steps": clk_steps["ghz"],
            "clock_samples_steps": clk_steps["samples_in_window"],
            "attn_alone_ms": round(t_attn_alone, 4),
            "attn_alone_clock_ghz": clk_attn["ghz"],
            "clock_samples_attn": clk_attn["samples_in_window"],
        },
        "roofline": {
            "kernel": "bsa_fwd_kernel",
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / BF16_DENSE_TFLOPS, 4),
            "traffic": measured_traffic("bsa_fwd", w.name),
            "clock_ghz": clk_attn["ghz"],
            "frac_of_peak_at_measured_clock": (round(sh.attn_flops / (t_attn_alone * 1e-3) / 1e12 /
                                                     (BF16_DENSE_TFLOPS * clk_attn["ghz"] / PEAK_CLOCK_GHZ), 4)
                                               if clk_attn["ghz"] else None),
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
    }
    comp = out["components"]

    # The payload consumed segment by segment (the local one first, then ring distance 1, 2, ...), each
    # folded into the running result in one launch per segment.
    ranges = bsa.segment_ranges(seg, g.H, g.G)
    order = [(w.r + k) % w.G for k in range(w.G)]
    seg_chunks = [dict(p=p, h_lo=0, h_hi=g.H, slot_lo=ranges[p][0], slot_hi=ranges[p][1]) for p in order]
    fold_reps = max(3, steps // 4)

    def time_fold(chunks):
        sh.fold(chunks)
        torch.cuda.synchronize()
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(fold_reps)]
        for e in fev:
            sh.O.zero_()
            sh.lse.fill_(float("-inf"))
            e[0].record(stream)
            for ch in chunks:
                bsa.block_sparse_attn_chunk_accumulate(g, sh.Q, sh.mask, sh.u.slot_of, sh.packed, ch, sh.O, sh.lse,
                                                       sh.scale)
            e[1].record(stream)
        torch.cuda.synchronize()
        return float(np.median(_ms(fev, 0, 1)))

    fused_ms = time_fold(seg_chunks)
    comp["segmented_fused_attn_ms"] = round(fused_ms, 4)
    comp["segmented_fused_attn_TFLOPs"] = round(sh.attn_flops / (fused_ms * 1e-3) / 1e12, 2)
    print(f"[bench] {w.name}: segmented attention, fused fold {fused_ms:.3f} ms", file=sys.stderr, flush=True)

    if full:
        # Cold caches: before the union + pack and again before the attention, a read of twice the Infinity
        # Cache's size evicts the L2s and the Infinity Cache, so each timed kernel starts with its inputs in
        # HBM.  A read, not a write: a written flush buffer would leave dirty lines whose write-back the next
        # kernel pays for.
        if args.cold_reps > 0:
            flush = torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device="cuda")
            cev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.cold_reps)]
            for e in cev:
                flush.sum()
                e[0].record(stream)
                sh.union()
                e[1].record(stream)
                sh.pack()
                e[2].record(stream)
                flush.sum()
                e[3].record(stream)
                sh.attention()
                e[4].record(stream)
            torch.cuda.synchronize()
            del flush
            c_union, c_pack, c_attn = _ms(cev, 0, 1), _ms(cev, 1, 2), _ms(cev, 3, 4)
            comp["cold"] = {
                "reps": args.cold_reps,
                "union_compact_us_median": round(float(np.median(c_union)) * 1e3, 2),
                "pack_us_median": round(float(np.median(c_pack)) * 1e3, 2),
                "pack_us_min": round(min(c_pack) * 1e3, 2),
                "pack_GBps_median": round(pack_bytes / (float(np.median(c_pack)) * 1e-3) / 1e9, 1),
                "attn_ms_median": round(float(np.median(c_attn)), 4),
                "attn_ms_min": round(min(c_attn), 4),
                "attn_TFLOPs_median": round(sh.attn_flops / (float(np.median(c_attn)) * 1e-3) / 1e12, 2),
            }

        # The two-call form: each segment's partial result written out, then merged by log-sum-exp.
        parts = [(torch.empty_like(sh.O), torch.empty_like(sh.lse)) for _ in order]
        accO, accL = torch.empty_like(sh.O), torch.empty_like(sh.lse)

        def seg_step(ev=None):
            accO.zero_()
            accL.fill_(float("-inf"))
            for i, p in enumerate(order):
                if ev is not None:
                    ev[2 * i].record(stream)
                bsa.block_sparse_attn_segment(g, sh.Q, sh.mask, sh.u.slot_of, sh.packed, ranges[p][0], ranges[p][1],
                                              sh.scale, out=parts[i])
                if ev is not None:
                    ev[2 * i + 1].record(stream)
                bsa.merge_partial(g, accO, accL, *parts[i])
            if ev is not None:
                ev[2 * len(order)].record(stream)

        seg_step()
        torch.cuda.synchronize()
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(order) + 1)] for _ in range(fold_reps)]
        for e in sev:
            seg_step(e)
        torch.cuda.synchronize()
        seg_total = float(np.mean([e[0].elapsed_time(e[-1]) for e in sev]))
        seg_attn = float(np.mean([sum(e[2 * i].elapsed_time(e[2 * i + 1]) for i in range(len(order))) for e in sev]))
        merge_ms = (seg_total - seg_attn) / max(1, len(order))
        merge_bytes = (3 * sh.O.numel() + 3 * sh.lse.numel()) * 4   # read O, O_part, lse x2; write O, lse
        del parts, accO, accL
        comp["segmented_attn_ms"] = round(seg_total, 4)
        comp["segmented_attn_TFLOPs"] = round(sh.attn_flops / (seg_total * 1e-3) / 1e12, 2)
        comp["merge_us"] = round(merge_ms * 1e3, 2)
        comp["merge_GBps"] = round(merge_bytes / (merge_ms * 1e-3) / 1e9, 1) if merge_ms > 0 else None

        # Chunked consumption (section 7): (steady, drain) head-chunk counts, fold time against chunk count.
        counts = bsa.demand_counts(g, sh.mask).cpu().numpy()
        sweep = []
        for steady, drain in CHUNK_PLANS:
            plan = bsa.chunk_plan(seg, counts, sh.inp["placement"], g.G, g.r, steady, drain)
            t = time_fold(plan)
            sweep.append({"chunks_steady": steady, "chunks_drain": drain, "chunks": len(plan), "fold_ms": round(t, 4),
                          "over_single_pass": round(t / t_attn, 3),
                          "last_chunk_tiles": plan[-1]["tiles"] if plan else 0})
        comp["chunk_sweep"] = sweep
        print(f"[bench] {w.name}: chunk sweep " + ", ".join(f"{s['chunks']} chunks {s['fold_ms']:.3f} ms"
                                                              for s in sweep), file=sys.stderr, flush=True)

    # Placement permutation (section 4.3), on every workload: the layer's hidden states [nb*b][H*d] bf16 into
    # rank-major block order and back; each call reads and writes every byte once.
    pos, _ = bsa.placement_permutation(sh.inp["placement"], g.G)
    pos_d = torch.from_numpy(pos).cuda()
    hidden = torch.randn((g.nb * g.b, g.H * g.d), device="cuda").to(torch.bfloat16)
    hidden_p = torch.empty_like(hidden)
    hidden_r = torch.empty_like(hidden)
    for _ in range(2):
        bsa.permute_blocks(hidden, pos_d, g.b, out=hidden_p)
        bsa.permute_blocks(hidden_p, pos_d, g.b, inverse=True, out=hidden_r)
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(max(3, steps // 2))]
    for e in pev:
        e[0].record(stream)
        bsa.permute_blocks(hidden, pos_d, g.b, out=hidden_p)
        e[1].record(stream)
        bsa.permute_blocks(hidden_p, pos_d, g.b, inverse=True, out=hidden_r)
        e[2].record(stream)
    torch.cuda.synchronize()
    assert torch.equal(hidden_r, hidden), "permutation round trip changed the hidden states"
    t_perm, t_iperm = float(np.mean(_ms(pev, 0, 1))), float(np.mean(_ms(pev, 1, 2)))
    perm_bytes = 2 * hidden.numel() * hidden.element_size()
    del hidden, hidden_p, hidden_r
    comp.update({"permute_hidden_bytes": perm_bytes, "permute_us": round(t_perm * 1e3, 2),
                 "permute_GBps": round(perm_bytes / (t_perm * 1e-3) / 1e9, 1),
                 "permute_inverse_us": round(t_iperm * 1e3, 2),
                 "permute_inverse_GBps": round(perm_bytes / (t_iperm * 1e-3) / 1e9, 1)})

    # Mask materialisation from pooled tiles (section 4.2): pool K (every block) and the local Q blocks,
    # then score and select every local row (Top-p 0.9 with a Top-k floor of 16 blocks).
    if g.nb <= 16384:
        ids_d = torch.from_numpy(sh.inp["q_blocks"]).cuda()
        kp = bsa.pool_blocks(g, sh.K)
        qp = bsa.pool_blocks(g, sh.Q, block_ids=ids_d)
        mat_mask = bsa.materialize_mask(g, qp, kp, 0.9, 16)
        mev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(max(3, steps // 2))]
        for e in mev:
            e[0].record(stream)
            bsa.pool_blocks(g, sh.K, out=kp)
            e[1].record(stream)
            bsa.pool_blocks(g, sh.Q, block_ids=ids_d, out=qp)
            e[2].record(stream)
            bsa.materialize_mask(g, qp, kp, 0.9, 16, out=mat_mask)
            e[3].record(stream)
        torch.cuda.synchronize()
        t_pk, t_pq, t_sel = (float(np.mean(_ms(mev, i, i + 1))) for i in range(3))
        k_bytes = sh.K.numel() * 2 * w.N // (g.nb * g.b)          # real rows of K are read
        out["mask_materialisation"] = {
            "pool_k_us": round(t_pk * 1e3, 2), "pool_k_GBps": round(k_bytes / (t_pk * 1e-3) / 1e9, 1),
            "pool_q_us": round(t_pq * 1e3, 2), "select_us": round(t_sel * 1e3, 2), "tau": 0.9, "k_min": 16,
            "density": round(float(mat_mask[:, :, :g.nb].float().mean().item()), 4)}
        del kp, qp, mat_mask

    if not args.no_comm:
        t0 = time.perf_counter()
        out["comm_volume"] = comm_accounting(w, sh.inp, g, torch, bsa)
        print(f"[bench] {w.name}: communication accounting took {time.perf_counter() - t0:.1f} s", file=sys.stderr,
              flush=True)
    return out


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share only; --gpus {args.gpus} is not supported (use --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_attention_rank_amd as bsa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    sh = Share(args.config, torch, bsa)
    head = measure(sh, args.steps, args.warmup, True, args)
    S = head["config"]["slots_S"]
    inp, pairs, flops = sh.inp, sh.pairs, sh.attn_flops
    sh.release()
    ceil = None
    if not args.no_ceilings:
        ceil = ceilings(torch, bsa, S * 2 * sh.g.b * sh.g.d * 2)
        print(f"[bench] ceilings: bf16 GEMM {ceil['gemm_bf16_TFLOPs']} TFLOP/s at {ceil['gemm_clock_ghz']} GHz, "
              f"copy {ceil['copy_GBps']} GB/s", file=sys.stderr, flush=True)

    extra = {}
    for name in [n for n in args.extra.split(",") if n and n != args.config]:
        xs = Share(name, torch, bsa)
        r = measure(xs, args.steps, args.warmup, False, args)
        xs.release()
        extra[name] = r
        del xs

    rec = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
        "components": head["components"],
        "roofline": head["roofline"],
        "roofline_pack": head["roofline_pack"],
        "ceilings": ceil,
        "comm_volume": head.get("comm_volume"),
        "mask_materialisation": head.get("mask_materialisation"),
        "extra_configs": extra,
        "sources_digest": {k: kernel_sources_digest(k) for k in ("bsa_fwd", "pack")},
    }
    if not args.no_cpu:
        t0 = time.perf_counter()
        rec["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds, pairs, flops)
        print(f"[bench] cpu baseline took {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
