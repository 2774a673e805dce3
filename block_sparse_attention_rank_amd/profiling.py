"""Summaries of rocprofv3 CSV output for the library's kernels (measurement tooling; no GPU needed).

    python -m block_sparse_attention_rank_amd.profiling trace  KT_DIR  --warmup W --steps K
    python -m block_sparse_attention_rank_amd.profiling stats  KT_DIR  --warmup W --steps K
    python -m block_sparse_attention_rank_amd.profiling traffic FETCH_DIR WRITE_DIR --warmup W --steps K \
        --workload NAME --calibration-mib MIB [--cold-reps C] [--json-dir profiles]
    python -m block_sparse_attention_rank_amd.profiling attn-counters PMC_DIR --warmup W --steps K

The inputs are the directories written by ``rocprofv3 --kernel-trace --stats --output-format csv -o run``
and ``rocprofv3 --pmc <counter> --output-format csv -o run`` around ``bench.py``.  bench.py launches, in
order: W + K single-pass steps (union, compaction, pack, attention), C cold-cache repetitions of the same
launches (each after a fill that flushes the caches), then the segment-wise attention and its merges, the
permutation legs and the mask materialisation legs; the first W + K launches of bsa_fwd_kernel and
pack_kernel are the single-pass ones and the last K of them are timed.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import re
from collections import defaultdict



def short_name(name: str) -> str:
    """A kernel's short name: torch's elementwise kernels and the runtime's copy/fill kernels by their
    family, this library's kernels by their name, anything else by its first name token."""
    m = re.search(r"(\w*elementwise\w*|__amd_rocclr_\w+)", name)
    if m:
        return m.group(1)
    m = re.search(r"(\w+_kernel)\b", name)
    if m:
        return m.group(1)
    return re.sub(r"^void\s+", "", name).split("(")[0].split("<")[0][:40]


def _rows(path: str) -> list[dict]:
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(d: str, suffix: str) -> str:
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def trace(kt_dir: str, warmup: int, steps: int) -> str:
    rows = _rows(_find(kt_dir, "kernel_trace.csv"))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    by = defaultdict(list)
    for r in rows:
        by[short_name(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in by.values())
    out = ["| kernel | calls | average us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| {k} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} | "
                   f"{100 * sum(v) / total:.1f} % |")
    out += ["", "Launches of the timed single-pass steps (warmup excluded):", "",
            "| kernel | launches | average us | median us |", "|---|---|---|---|"]
    for k in ("bsa_fwd_kernel", "pack_kernel", "compact_kernel", "union_kernel"):
        v = by.get(k, [])[warmup:warmup + steps]
        if v:
            med = sorted(v)[len(v) // 2]
            out.append(f"| {k} | {len(v)} | {sum(v) / len(v):.1f} | {med:.1f} |")
    return "\n".join(out)


def stats(kt_dir: str) -> str:
    """rocprofv3's own --stats table (every launch of each kernel), with short kernel names."""
    rows = _rows(_find(kt_dir, "kernel_stats.csv"))
    out = ["| kernel | calls | total ms | average us | min us | max us | share |", "|---|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        out.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
                   f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                   f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} % |")
    return "\n".join(out)


def _counter_by_dispatch(pmc_dir: str, counter: str):
    vals = defaultdict(float)
    meta = {}
    for r in _rows(_find(pmc_dir, "counter_collection.csv")):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        vals[d] += float(r["Counter_Value"])
        meta[d] = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]),
                   (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return [(d, meta[d][0], meta[d][1], vals[d], meta[d][2]) for d in sorted(vals)]


def _calibration(disp, warmup: int):
    """Counter value of the calibration multiply: bench.py runs it between the warmup steps and the first
    timed step, after a fill of its source, so it is the last elementwise dispatch before the first timed
    union_kernel."""
    unions = [i for i, (_, k, _, _, _) in enumerate(disp) if k == "union_kernel"]
    stop = unions[warmup] if len(unions) > warmup else len(disp)
    cands = [v for _, k, _, v, _ in disp[:stop] if "elementwise" in k]
    return cands[-1] if cands else None


def _single_pass(disp, warmup: int, steps: int, cold_reps: int = 0):
    """Per kernel, the dispatches that one step of the path makes (warmup and timed steps), those of the
    cold-cache repetitions, plus all dispatches of the other kernels grouped by grid size."""
    groups = defaultdict(list)
    seen = defaultdict(int)
    for d, k, grid, v, dur in disp:
        if k in ("bsa_fwd_kernel", "pack_kernel", "union_kernel", "compact_kernel"):
            seen[k] += 1
            if warmup + steps < seen[k] <= warmup + steps + cold_reps:
                groups[(k + " (cold caches)", None)].append(v)
                continue
            if seen[k] > warmup + steps + cold_reps:
                if k != "bsa_fwd_kernel":
                    continue
                groups[(k + " (segments)", None)].append(v)
                continue
            groups[(k, None)].append(v)
        else:
            groups[(k, grid)].append(v)
    return groups


def traffic(fetch_dir: str, write_dir: str, warmup: int, steps: int, workload: str, calib_mib: int,
            json_dir: str | None, digests: dict | None, cold_reps: int = 0) -> str:
    f = _counter_by_dispatch(fetch_dir, "FETCH_SIZE")
    w = _counter_by_dispatch(write_dir, "WRITE_SIZE")
    calib_kib = calib_mib * 1024
    f_cal, w_cal = _calibration(f, warmup), _calibration(w, warmup)
    rs = calib_kib / f_cal if f_cal else 1.0
    ws = calib_kib / w_cal if w_cal else 1.0
    gf, gw = _single_pass(f, warmup, steps, cold_reps), _single_pass(w, warmup, steps, cold_reps)
    out = [f"Calibration: a float32 multiply of {calib_mib} MiB reads and writes exactly {calib_mib} MiB; FETCH_SIZE "
           f"reports {f_cal:.0f} KiB and WRITE_SIZE {w_cal:.0f} KiB for it, so the read scale is {rs:.4f} and the "
           f"write scale {ws:.4f}.", "",
           "| kernel | grid | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read bytes | scaled write bytes | "
           "total bytes |", "|---|---|---|---|---|---|---|---|"]
    recs = {}
    for key in sorted(gf, key=lambda x: (x[0], x[1] or 0)):
        if key not in gw or "elementwise" in key[0] or "copyBuffer" in key[0] or "Fill" in key[0]:
            continue
        fk = sum(gf[key]) / len(gf[key])
        wk = sum(gw[key]) / len(gw[key])
        rb, wb = fk * 1024 * rs, wk * 1024 * ws
        out.append(f"| {key[0]} | {key[1] if key[1] is not None else '-'} | {len(gf[key])} | {fk:.1f} | {wk:.1f} | "
                   f"{rb:.4g} | {wb:.4g} | {rb + wb:.4g} |")
        if key[1] is None and key[0] in ("bsa_fwd_kernel", "pack_kernel"):
            recs[key[0]] = (rb, wb)
    if json_dir:
        for kname, (rb, wb) in recs.items():
            base = kname.replace("_kernel", "")
            rec = {"kernel": kname, "workload": workload, "sources_digest": (digests or {}).get(base),
                   "read_bytes": int(rb), "write_bytes": int(wb), "bytes_per_launch": int(rb + wb),
                   "read_scale": rs, "write_scale": ws, "summary": f"profiles/hbm_traffic_{workload}.md"}
            with open(os.path.join(json_dir, f"{base}_{workload}_traffic.json"), "w") as fh:
                json.dump(rec, fh, indent=1)
    return "\n".join(out)


def attn_counters(pmc_dir: str, warmup: int, steps: int) -> str:
    """Utilisation of the single-pass bsa_fwd_kernel launches from whichever of these counters the pass
    collected: MFMA busy and LDS busy / conflicts (SQ_VALU_MFMA_BUSY_CYCLES, SQ_LDS_IDX_ACTIVE,
    SQ_LDS_BANK_CONFLICT), or the VALU mix (SQ_INSTS_VALU, SQ_INSTS_MFMA, SQ_ACTIVE_INST_VALU); all with
    GRBM_GUI_ACTIVE for the clock."""
    rows = _rows(_find(pmc_dir, "counter_collection.csv"))
    per = defaultdict(lambda: defaultdict(float))
    dur = {}
    for r in rows:
        if short_name(r["Kernel_Name"]) != "bsa_fwd_kernel":
            continue
        d = int(r["Dispatch_Id"])
        per[d][r["Counter_Name"]] += float(r["Counter_Value"])
        dur[d] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    valu_mix = any("SQ_INSTS_VALU" in per[d] for d in per)
    if valu_mix:
        out = ["| dispatch | duration us | clock GHz | VALU instructions per MFMA | VALU busy | MFMA busy |",
               "|---|---|---|---|---|---|"]
    else:
        out = ["| dispatch | duration us | clock GHz | MFMA busy | LDS busy | LDS conflicts / access |",
               "|---|---|---|---|---|---|"]
    for d in sorted(per)[:warmup + steps]:
        c = per[d]
        active = c["GRBM_GUI_ACTIVE"] / 8.0
        clock = active / (dur[d] * 1e3)
        mfma = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * 1024)
        if valu_mix:
            # SQ_INSTS_VALU counts MFMAs among the VALU instructions; SQ_ACTIVE_INST_VALU is per wave, in
            # quad-cycles, summed over all waves: divided by active cycles x 1024 SIMDs it is the busy share
            # of a SIMD's VALU issue summed over its waves
            ratio = (c["SQ_INSTS_VALU"] - c["SQ_INSTS_MFMA"]) / max(1.0, c["SQ_INSTS_MFMA"])
            vbusy = 4 * c["SQ_ACTIVE_INST_VALU"] / (active * 1024)
            out.append(f"| {d} | {dur[d]:.1f} | {clock:.3f} | {ratio:.2f} | {vbusy:.3f} | {mfma:.3f} |")
        else:
            lds = c["SQ_LDS_IDX_ACTIVE"] / (active * 256)
            conf = c["SQ_LDS_BANK_CONFLICT"] / max(1.0, c["SQ_LDS_IDX_ACTIVE"] - c["SQ_LDS_BANK_CONFLICT"])
            out.append(f"| {d} | {dur[d]:.1f} | {clock:.3f} | {mfma:.3f} | {lds:.3f} | {conf:.3f} |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["trace", "stats", "traffic", "attn-counters"])
    ap.add_argument("dirs", nargs="+")
    ap.add_argument("--warmup", type=int, required=True)
    ap.add_argument("--steps", type=int, required=True)
    ap.add_argument("--workload", default="hunyuan")
    ap.add_argument("--calibration-mib", type=int, default=1024)
    ap.add_argument("--cold-reps", type=int, default=0, help="bench.py's --cold-reps of the profiled run")
    ap.add_argument("--json-dir", default=None)
    a = ap.parse_args()
    if a.mode == "trace":
        print(trace(a.dirs[0], a.warmup, a.steps))
    elif a.mode == "stats":
        print(stats(a.dirs[0]))
    elif a.mode == "traffic":
        import importlib.util
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        spec = importlib.util.spec_from_file_location("bench", os.path.join(root, "bench.py"))
        bench = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(bench)
        digests = {k: bench.kernel_sources_digest(k) for k in ("bsa_fwd", "pack")}
        print(traffic(a.dirs[0], a.dirs[1], a.warmup, a.steps, a.workload, a.calibration_mib, a.json_dir, digests,
                      a.cold_reps))
    else:
        print(attn_counters(a.dirs[0], a.warmup, a.steps))


if __name__ == "__main__":
    main()
