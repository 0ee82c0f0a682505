"""Host logic of bench.py that needs no GPU: the one-GPU guard, the HBM
traffic read from the committed counter summaries (and its refusal once the
kernel sources differ from those the summary was taken on), and the clock
reading's report."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


@pytest.mark.parametrize("key", sorted(bench.COUNTER_SUMMARY))
def test_traffic_from_summaries(key, monkeypatch):
    """Each summary parses; its traffic, when the sources match, is above the
    algorithmic bytes of one call (Q, K, V, O once: 0.65 GB at seg1); with a
    different source hash the bench reports none."""
    got = bench.measured_traffic(*key)
    if got is not None:
        assert isinstance(got, int) and got > 0.6e9
    monkeypatch.setattr(bench, "source_hash", lambda files: "0" * 16)
    assert bench.measured_traffic(*key) is None


def test_unknown_workload_has_no_traffic():
    assert bench.measured_traffic("bf16", "no-such-workload") is None


def _sampler(samples, info=None):
    s = bench.ClockSampler(enabled=False)
    s.info = info if info is not None else {"max_clk_mhz": 2400, "power_limit_w": 1_400_000_000}
    s.samples = samples
    return s


def test_clock_report_skips_the_settling_readings():
    # 0.0 .. 2.0 s every 0.1 s: the first half second reads a stale idle clock
    samples = [(0.1 * i, 100.0 if i < 5 else 1800.0 + i, 1300.0) for i in range(21)]
    r = _sampler(samples).report()
    assert r["gfxclk_mhz_min"] >= 1805
    assert r["samples"] == 16
    assert r["power_limit_w"] == 1400            # microwatts read as watts
    assert r["socket_power_w_mean"] == 1300
    assert r["max_clk_mhz"] == 2400


def test_clock_report_needs_a_second_of_readings():
    samples = [(0.1 * i, 1800.0, 1300.0) for i in range(14)]     # 1.3 s in all
    assert _sampler(samples).report() is None
    assert _sampler([]).report() is None
    s = _sampler([(0.1 * i, 1800.0, 1300.0) for i in range(30)])
    s.info = None                                                # no amdsmi
    assert s.report() is None
