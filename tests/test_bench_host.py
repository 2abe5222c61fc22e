"""Host logic of bench.py that runs without a GPU: the GFX clock parser and its
sample threshold, and the argument checks that refuse a run before any device
work."""
import subprocess
import sys
from pathlib import Path

import bench

ROOT = Path(__file__).resolve().parents[1]

# The layout `amd-smi metric -g 0 -c` prints: one block per GFX engine, then the
# memory and video clocks, whose CLK lines must not count.
SMI_TEXT = "GPU: 0\n    CLOCK:\n" + "".join(
    f"        GFX_{i}:\n            CLK: {2000 + 10 * i} MHz\n            MIN_CLK: 500 MHz\n"
    f"            MAX_CLK: 2400 MHz\n            CLK_LOCKED: DISABLED\n            DEEP_SLEEP: ENABLED\n"
    for i in range(8)) + (
    "        MEM_0:\n            CLK: 1900 MHz\n            MIN_CLK: 900 MHz\n"
    "        VCLK_0:\n            CLK: 29 MHz\n")


class _Out:
    def __init__(self, text):
        self.stdout = text


def test_clock_parser_averages_the_gfx_engines_only(monkeypatch):
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: _Out(SMI_TEXT))
    assert bench.ClockSampler._sample() == sum(2000 + 10 * i for i in range(8)) / 8


def test_clock_parser_without_tool_or_clock_lines(monkeypatch):
    def missing(*a, **k):
        raise FileNotFoundError("amd-smi")
    monkeypatch.setattr(subprocess, "run", missing)
    assert bench.ClockSampler._sample() is None
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: _Out("GPU: 0\n    CLOCK:\n"))
    assert bench.ClockSampler._sample() is None


def test_clock_report_needs_enough_samples():
    c = bench.ClockSampler()
    c.means = [2400.0] + [2200.0] * 7
    assert c.report() is None  # under nine samples: no figure
    c.means = [2400.0] + [2200.0] * 4 + [2300.0] * 4
    r = c.report()
    assert r["samples"] == 8 and r["mean"] == 2250.0  # the first sample is dropped
    assert r["min_sample"] == 2200.0 and r["max_sample"] == 2300.0


def _bench(*args):
    return subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    p = _bench("--gpus", "2")
    assert p.returncode == 2 and "--gpus 2 is not supported" in p.stderr


def test_sustained_mode_rejects_bad_sizes():
    for n in ("12", "4", "32768"):  # not a multiple of 8; below 8; a dW of 4 GiB
        p = _bench("--mode", "sustained", "--size", n)
        assert p.returncode == 2 and "--size" in p.stderr, (n, p.stderr)
