"""The rocprofv3 summariser on small synthetic CSV files (no GPU): kernel names are shortened, timed
launches exclude the warmup, the calibration multiply is found between the warmup and the first timed
step, and per-launch traffic is scaled by it."""
import csv
import json
import os

from block_sparse_attention_rank_amd import profiling as P

KT_FIELDS = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
PMC_FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value", "Start_Timestamp",
              "End_Timestamp"]


def _write(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def _name(k):
    return f"void sparsp::(anonymous namespace)::{k}<128, 128>(unsigned short const*, int)"


def test_short_names():
    assert P.short_name(_name("bsa_fwd_kernel")) == "bsa_fwd_kernel"
    assert P.short_name("void at::native::vectorized_elementwise_kernel<4, X>(int)") == "vectorized_elementwise_kernel"


def test_trace_excludes_warmup(tmp_path):
    rows, t = [], 0
    for step, dur in enumerate([50, 40, 10, 12]):          # 2 warmup launches, then 2 timed
        rows.append({"Kernel_Name": _name("bsa_fwd_kernel"), "Start_Timestamp": t, "End_Timestamp": t + dur * 1000})
        t += 10 ** 6
    _write(str(tmp_path / "kt" / "run_kernel_trace.csv"), KT_FIELDS, rows)
    out = P.trace(str(tmp_path / "kt"), warmup=2, steps=2)
    assert "| bsa_fwd_kernel | 2 | 11.0 |" in out


def test_traffic_calibration_and_scaling(tmp_path):
    def dispatches(counter, calib_value, pack_value):
        seq = [("union_kernel", 0), ("pack_kernel", pack_value),                      # warmup step
               ("vectorized_elementwise_kernel", 0),                                    # fill of the source
               ("vectorized_elementwise_kernel", calib_value),                          # calibration multiply
               ("union_kernel", 0), ("pack_kernel", pack_value)]                        # timed step
        return [{"Dispatch_Id": i + 1, "Kernel_Name": _name(k) if "elementwise" not in k else f"void {k}<4>(int)",
                 "Grid_Size": 256, "Counter_Name": counter, "Counter_Value": v, "Start_Timestamp": 0,
                 "End_Timestamp": 1000} for i, (k, v) in enumerate(seq)]
    _write(str(tmp_path / "f" / "run_counter_collection.csv"), PMC_FIELDS, dispatches("FETCH_SIZE", 512.0, 100.0))
    _write(str(tmp_path / "w" / "run_counter_collection.csv"), PMC_FIELDS, dispatches("WRITE_SIZE", 1024.0, 300.0))
    out = P.traffic(str(tmp_path / "f"), str(tmp_path / "w"), warmup=1, steps=1, workload="unit", calib_mib=1,
                    json_dir=str(tmp_path), digests={"pack": "abc"})
    assert "read scale is 2.0000 and the write scale 1.0000" in out
    rec = json.load(open(tmp_path / "pack_unit_traffic.json"))
    assert rec["read_bytes"] == 100 * 1024 * 2 and rec["write_bytes"] == 300 * 1024
    assert rec["sources_digest"] == "abc"


def test_traffic_cold_repetitions_kept_apart(tmp_path):
    # warmup 1 + timed 1 single-pass packs, then 2 cold-cache packs with more HBM traffic: the single-pass
    # record averages only the first two, the cold ones get their own row
    seq = [("pack_kernel", 100.0), ("vectorized_elementwise_kernel", 512.0), ("union_kernel", 0),
           ("pack_kernel", 100.0), ("pack_kernel", 400.0), ("pack_kernel", 600.0)]

    def rows(counter):
        return [{"Dispatch_Id": i + 1, "Kernel_Name": _name(k) if "elementwise" not in k else f"void {k}<4>(int)",
                 "Grid_Size": 256, "Counter_Name": counter, "Counter_Value": v, "Start_Timestamp": 0,
                 "End_Timestamp": 1000} for i, (k, v) in enumerate(seq)]
    _write(str(tmp_path / "f" / "run_counter_collection.csv"), PMC_FIELDS, rows("FETCH_SIZE"))
    _write(str(tmp_path / "w" / "run_counter_collection.csv"), PMC_FIELDS, rows("WRITE_SIZE"))
    out = P.traffic(str(tmp_path / "f"), str(tmp_path / "w"), warmup=1, steps=1, workload="unit", calib_mib=1,
                    json_dir=str(tmp_path), digests={}, cold_reps=2)
    rec = json.load(open(tmp_path / "pack_unit_traffic.json"))
    assert rec["read_bytes"] == 100 * 1024 * 2
    assert "| pack_kernel (cold caches) | - | 2 | 500.0 |" in out


def test_stats_table(tmp_path):
    fields = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"]
    _write(str(tmp_path / "kt" / "run_kernel_stats.csv"), fields, [
        {"Name": _name("pack_kernel"), "Calls": 2, "TotalDurationNs": 1000000, "AverageNs": 500000, "Percentage": 20.0,
         "MinNs": 400000, "MaxNs": 600000, "StdDev": 1},
        {"Name": _name("bsa_fwd_kernel"), "Calls": 2, "TotalDurationNs": 4000000, "AverageNs": 2000000,
         "Percentage": 80.0, "MinNs": 1900000, "MaxNs": 2100000, "StdDev": 1}])
    out = P.stats(str(tmp_path / "kt")).splitlines()
    assert out[2] == "| bsa_fwd_kernel | 2 | 4.00 | 2000.0 | 1900.0 | 2100.0 | 80.0 % |"
    assert out[3].startswith("| pack_kernel | 2 | 1.00 | 500.0 |")
