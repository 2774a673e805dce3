"""Shader-clock measurement around device work (include/sparsp_measure.h): a sampler kernel on a side stream
records (shader clock, wall clock) pairs while the measured kernels run on the main stream, and two wall-clock
timestamps in the main stream's order mark the window whose average shader clock is reported."""
from __future__ import annotations

import ctypes

from ._lib import check, load

# Side stream per measured stream, checked to run beside it.  The HIP runtime maps streams onto a few
# hardware queues (GPU_MAX_HW_QUEUES, 4 by default); a side stream that shares the measured stream's queue
# runs the sampler before the window instead of during it.
_SIDE: dict = {}


def _runs_beside(lib, khz: int, main, side) -> bool:
    """True when a sampler launched on ``side`` takes samples while ``main`` is busy."""
    import torch
    interval = max(1, int(round(20e-6 * khz * 1e3)))              # 20 us
    n = 256                                                       # about 5 ms of sampling
    samples = torch.zeros(2 * n, dtype=torch.int64, device="cuda")
    ts = torch.zeros(2, dtype=torch.int64, device="cuda")
    side.wait_stream(main)
    check(lib.sparsp_clock_sampler(ctypes.c_void_p(samples.data_ptr()), n, interval,
                                   ctypes.c_void_p(side.cuda_stream)))
    with torch.cuda.stream(main):
        torch.cuda._sleep(1_000_000)
    check(lib.sparsp_wall_timestamp(ctypes.c_void_p(ts.data_ptr()), ctypes.c_void_p(main.cuda_stream)))
    with torch.cuda.stream(main):
        torch.cuda._sleep(1_000_000)
    check(lib.sparsp_wall_timestamp(ctypes.c_void_p(ts.data_ptr() + 8), ctypes.c_void_p(main.cuda_stream)))
    torch.cuda.synchronize()
    smp = samples.cpu().numpy().reshape(-1, 2)
    t0, t1 = (int(x) for x in ts.cpu().numpy())
    w = smp[:, 1]
    return int(((w >= t0) & (w <= t1)).sum()) >= 2


def side_stream(main=None):
    """A stream whose work runs concurrently with ``main`` (the current stream by default), or None when no
    stream does (a profiler that serialises kernels, for one)."""
    import torch
    main = main if main is not None else torch.cuda.current_stream()
    key = main.cuda_stream
    if key not in _SIDE:
        lib = load()
        khz = ctypes.c_int32(0)
        check(lib.sparsp_wall_clock_khz(ctypes.byref(khz)))
        _SIDE[key] = None
        for _ in range(16):
            cand = torch.cuda.Stream()             # default priority
            if _runs_beside(lib, khz.value, main, cand):
                _SIDE[key] = cand
                break
    return _SIDE[key]


class ClockWindow:
    """Average shader clock over a window of one stream's work.

        cw = ClockWindow(max_seconds=0.5)
        cw.start(stream); ...launches on stream...; cw.stop(stream)
        ghz = cw.result()["ghz"]

    The sampler takes a sample every ``interval_us`` microseconds for at most ``max_seconds`` and then exits by
    itself; the window must end before it does (result() reports how many samples fell inside).  Where no
    stream runs beside the measured one, nothing is sampled and the clock is reported as None."""

    def __init__(self, max_seconds: float = 0.5, interval_us: float = 20.0):
        import torch
        lib = load()
        khz = ctypes.c_int32(0)
        check(lib.sparsp_wall_clock_khz(ctypes.byref(khz)))
        self.khz = khz.value
        self.interval = max(1, int(round(interval_us * 1e-6 * self.khz * 1e3)))
        self.n = max(2, int(max_seconds * self.khz * 1e3 / self.interval) + 1)
        self.samples = torch.zeros(2 * self.n, dtype=torch.int64, device="cuda")
        self.ts = torch.zeros(2, dtype=torch.int64, device="cuda")
        self._lib = lib

    def start(self, stream=None, lead_cycles: int = 2_000_000) -> None:
        """Start the sampler beside ``stream``.  The stream first idles ``lead_cycles`` shader cycles (about a
        millisecond) so that the sampler is running before the window opens."""
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        side = side_stream(s)
        if side is None:
            return
        side.wait_stream(s)                        # the sampler starts after the work queued so far
        check(self._lib.sparsp_clock_sampler(ctypes.c_void_p(self.samples.data_ptr()), self.n, self.interval,
                                             ctypes.c_void_p(side.cuda_stream)))
        with torch.cuda.stream(s):
            torch.cuda._sleep(int(lead_cycles))
        check(self._lib.sparsp_wall_timestamp(ctypes.c_void_p(self.ts.data_ptr()), ctypes.c_void_p(s.cuda_stream)))

    def stop(self, stream=None) -> None:
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        check(self._lib.sparsp_wall_timestamp(ctypes.c_void_p(self.ts.data_ptr() + 8), ctypes.c_void_p(s.cuda_stream)))

    def result(self) -> dict:
        import torch
        torch.cuda.synchronize()
        smp = self.samples.cpu().numpy().reshape(-1, 2)
        t0, t1 = (int(x) for x in self.ts.cpu().numpy())
        if t0 == 0:                                # not started: no stream ran beside the measured one
            return dict(samples_in_window=0, window_us=None, ghz=None)
        smp = smp[smp[:, 1] > 0]
        inside = smp[(smp[:, 1] >= t0) & (smp[:, 1] <= t1)]
        out = dict(samples_in_window=int(len(inside)), window_us=round((t1 - t0) / self.khz * 1e3, 1), ghz=None)
        if len(inside) >= 2:
            dc = float(inside[-1, 0] - inside[0, 0])
            dw = float(inside[-1, 1] - inside[0, 1])
            out["ghz"] = round(dc / dw * self.khz * 1e3 / 1e9, 4)
        return out
