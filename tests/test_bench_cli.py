"""bench.py's contract on the host (no GPU): more than one GPU is refused with a message, the CPU-oracle
baseline reports the documented fields, and a stored traffic record is used only while its digest matches
the kernel sources."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_fields_on_tiny():
    from workloads import CONFIGS, make_inputs
    b = _bench()
    w = CONFIGS["tiny"]
    inp = make_inputs(w)
    pairs = int(inp["mask"][:, :, :w.nb].sum())
    flops = 4.0 * w.b * w.b * w.d * pairs
    rec = b.cpu_baseline(inp, 0.5, pairs, flops)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1 and rec["host_cpus"] >= 1
    assert rec["pack_GBps"] > 0 and rec["attn_GFLOPs"] > 0
    assert "tiny" in rec["sample"]
    json.dumps(rec)  # one JSON line


def test_stored_traffic_needs_matching_digest(tmp_path, monkeypatch):
    b = _bench()
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = {"sources_digest": b.kernel_sources_digest("pack"), "bytes_per_launch": 123}
    (prof / "pack_unit_traffic.json").write_text(json.dumps(good))
    (prof / "bsa_fwd_unit_traffic.json").write_text(json.dumps({"sources_digest": "stale", "bytes_per_launch": 9}))
    digests = {k: b.kernel_sources_digest(k) for k in ("pack", "bsa_fwd")}
    monkeypatch.setattr(b, "kernel_sources_digest", lambda k=None: digests[k])
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.measured_traffic("pack", "unit") == 123
    assert b.measured_traffic("bsa_fwd", "unit") is None
    assert b.measured_traffic("pack", "absent") is None
