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


@pytest.mark.parametrize("key", sorted(bench.PROFILED))
def test_traffic_from_summaries(key, monkeypatch):
    """Each summary parses; its traffic, when the sources match, is above the
    algorithmic bytes of one call (Q, K, V, O once: 0.65 GB at seg1); with a
    different source hash the bench reports none."""
    got = bench.measured_traffic(key)
    if got is not None:
        assert isinstance(got, int) and got > 0.6e9
    ms = bench.profiled_call_ms(key)
    if ms is not None:
        assert 1.0 < ms < 200.0
    monkeypatch.setattr(bench, "source_hash", lambda files: "0" * 16)
    assert bench.measured_traffic(key) is None
    assert bench.profiled_call_ms(key) is None


def test_unknown_workload_has_no_traffic():
    assert bench.measured_traffic("no-such-workload") is None
    assert bench.profiled_call_ms("no-such-workload") is None


def test_short_kernel_names():
    s = bench.short_kernel_name
    assert s("segattn::(anonymous namespace)::attn_bf16_kernel<false, false>(segattn::AttnArgs)") \
        == "attn_bf16_kernel<false, false>"
    assert s("segattn::(anonymous namespace)::combine_kernel(segattn::AttnArgs, int)") == "combine_kernel"
    assert s("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, "
             "std::array<char*, 1ul> >(int, at::native::FillFunctor<float>, std::array<char*, 1ul>)"
             ).startswith("vectorized_elementwise_kernel<4, at::native::FillFunctor<float>")


def _trace_csv(path, rows):
    with open(path, "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for name, start, end in rows:
            f.write(f'"{name}",{start},{end}\n')


def test_trace_summary_round_trip(tmp_path, monkeypatch, capsys):
    """A synthetic kernel trace: the summary's steady mean skips each kernel's
    first two calls, and the call time the roofline reads adds the merge
    kernel per attention launch."""
    name = "segattn::(anonymous namespace)::attn_bf16_kernel<false, false>(segattn::AttnArgs)"
    comb = "segattn::(anonymous namespace)::combine_kernel(segattn::AttnArgs, int)"
    rows, t0 = [], 0
    for i, us in enumerate([20000, 15000, 10000, 10000, 10000, 10000]):   # two warm-up calls
        rows.append((name, t0, t0 + us * 1000))
        rows.append((comb, t0 + us * 1000, t0 + us * 1000 + 30_000))
        t0 += us * 1000 + 100_000
    os.makedirs(tmp_path / "run" / "host")
    _trace_csv(tmp_path / "run" / "host" / "1_kernel_trace.csv", rows)
    bench.summarize_trace([str(tmp_path / "run")], "bf16", "synthetic", "none")
    text = capsys.readouterr().out
    assert "attn_bf16_kernel<false, false>" in text and "combine_kernel" in text
    prof = tmp_path / "profiles"
    os.makedirs(prof)
    (prof / "attn_bf16_seg1_kernel_trace.txt").write_text(text)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda files: text.split("}: ")[1].split()[0])
    assert abs(bench.profiled_call_ms("seg1") - (10.0 + 0.03)) < 1e-6


def test_pmc_summary_round_trip(tmp_path, monkeypatch, capsys):
    """Two counter passes merge per kernel; values are summed over a
    dispatch's rows and averaged over dispatches; the traffic is
    2 FETCH_SIZE + WRITE_SIZE KiB per call."""
    name = "segattn::(anonymous namespace)::attn_fp8_kernel<false>(segattn::AttnArgs)"
    for pas, counter, vals in (("p1", "FETCH_SIZE", [100.0, 300.0]), ("p2", "WRITE_SIZE", [50.0, 50.0])):
        os.makedirs(tmp_path / pas)
        with open(tmp_path / pas / "run_counter_collection.csv", "w") as f:
            f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
            for d, v in enumerate(vals):
                f.write(f'{d},"{name}",{counter},{v / 2}\n{d},"{name}",{counter},{v / 2}\n')
    bench.summarize_pmc([str(tmp_path / "p1"), str(tmp_path / "p2")], "fp8", "synthetic", "none")
    text = capsys.readouterr().out
    prof = tmp_path / "profiles"
    os.makedirs(prof)
    (prof / "attn_fp8_fp8seg8_counters.txt").write_text(text)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda files: text.split("}: ")[1].split()[0])
    assert bench.measured_traffic("fp8seg8") == int(1024 * (2 * 200.0 + 50.0))


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
