"""Shader-clock windows (include/sparsp_measure.h, block_sparse_attention_rank_amd/measure.py) on the GPU.

The runtime maps streams onto a few hardware queues, so a sampler on a side stream that shares the measured
stream's queue would run before the window and leave no sample inside it.  Every window below brackets a
fixed spin on the measured stream and must hold samples and a plausible clock, for several windows in a row
and for several measured streams.
"""
import pytest

pytestmark = pytest.mark.gpu


def _window(stream, spin_cycles=20_000_000):
    import torch
    from block_sparse_attention_rank_amd.measure import ClockWindow
    cw = ClockWindow(max_seconds=0.06)
    cw.start(stream)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(spin_cycles)
    cw.stop(stream)
    return cw.result()


def test_clock_windows_in_a_row(require_gpu):
    import torch
    s = torch.cuda.current_stream()
    for i in range(9):
        r = _window(s)
        print(f"[measure] window {i}: {r}", flush=True)
        assert r["samples_in_window"] >= 10, r
        assert 0.3 < r["ghz"] < 3.5, r


def test_clock_windows_on_several_streams(require_gpu):
    import torch
    streams = [torch.cuda.Stream() for _ in range(6)]
    for i, s in enumerate(streams):
        r = _window(s)
        print(f"[measure] stream {i}: {r}", flush=True)
        assert r["samples_in_window"] >= 10, r
        assert 0.3 < r["ghz"] < 3.5, r


def test_clock_window_without_a_concurrent_stream(require_gpu, monkeypatch):
    """Where no stream runs beside the measured one (a profiler serialising kernels), a window samples
    nothing and reports no clock instead of failing."""
    import torch
    from block_sparse_attention_rank_amd import measure
    monkeypatch.setattr(measure, "_runs_beside", lambda *args: False)
    monkeypatch.setattr(measure, "_SIDE", {})
    s = torch.cuda.Stream()
    r = _window(s)
    print(f"[measure] serialised: {r}", flush=True)
    assert r == {"samples_in_window": 0, "window_us": None, "ghz": None}
