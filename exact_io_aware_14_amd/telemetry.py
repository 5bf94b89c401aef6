"""Shader clock and board power while kernels run (AMD SMI's GPU metrics).

Used by bench.py to report the clock and power the timed kernels ran at: the
published peaks are quoted at 2.4 GHz, and under a sustained matrix-heavy load an
MI355X board reaches its power limit (1400 W) and lowers the clock, so a % of peak
figure needs the clock beside it.  The metrics refresh about once a second, so the
sampler is meant for a load held for a second or more; samples taken while the
GPU reports under half its cycles busy (idle gaps, stale readings) are dropped.
Sampling is best effort: without the AMD SMI library every reading is None.
"""
from __future__ import annotations

import threading
import time


class ClockSampler:
    """Context manager: samples the per-XCD shader clocks (MHz, mean over XCDs), the
    socket power (W) and the busy share every ``period`` seconds on a thread."""

    def __init__(self, period: float = 0.05, device_index: int = 0):
        self.period = period
        self.device_index = device_index
        self.clocks: list[float] = []
        self.powers: list[float] = []
        self.power_limit_w = None
        self._stop = threading.Event()
        self._thread = None
        self._smi = None
        self._handle = None

    def _open(self):
        try:
            import amdsmi

            amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
            handles = amdsmi.amdsmi_get_processor_handles()
            if self.device_index < len(handles):
                self._smi, self._handle = amdsmi, handles[self.device_index]
                try:
                    lim = self._smi.amdsmi_get_power_info(self._handle).get("power_limit")
                    if isinstance(lim, (int, float)) and lim > 0:
                        self.power_limit_w = lim / 1e6 if lim > 1e5 else float(lim)  # reported in µW
                except Exception:
                    pass
        except Exception:  # no SMI library or no access: readings stay None
            self._smi = None

    def _sample(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._handle)
        act = m.get("average_gfx_activity")
        if not isinstance(act, (int, float)) or act < 50:
            return
        clks = m.get("current_gfxclks")
        clks = [c for c in clks if isinstance(c, (int, float)) and 0 < c < 10000] if isinstance(clks, (list, tuple)) else []
        clk = sum(clks) / len(clks) if clks else m.get("current_gfxclk")
        pw = m.get("current_socket_power")
        if isinstance(clk, (int, float)) and 0 < clk < 10000:
            self.clocks.append(float(clk))
        if isinstance(pw, (int, float)) and 0 < pw < 10000:
            self.powers.append(float(pw))

    def _run(self):
        while not self._stop.is_set():
            try:
                self._sample()
            except Exception:
                return
            time.sleep(self.period)

    def __enter__(self):
        self._open()
        if self._smi is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join(timeout=2.0)
        if self._smi is not None:
            try:
                self._smi.amdsmi_shut_down()
            except Exception:
                pass
        return False

    def summary(self) -> dict:
        def mean(v):
            return round(sum(v) / len(v), 1) if v else None

        return {"gfxclk_mhz_mean": mean(self.clocks), "gfxclk_mhz_min": min(self.clocks) if self.clocks else None,
                "socket_power_w_mean": mean(self.powers), "socket_power_w_max": max(self.powers) if self.powers else None,
                "power_limit_w": self.power_limit_w, "busy_samples": len(self.clocks)}


def soak(fn, seconds: float = 1.5, sync=None) -> dict:
    """Run ``fn`` back to back for about ``seconds`` (synchronising with ``sync``
    between rounds) while sampling; returns the sampler's summary."""
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            fn()
            if sync is not None:
                sync()
    return clk.summary()
