"""Host-side parts of bench.py: the FLOP counts it reports, the clock
summary, and the one-GPU guard. No GPU, no library calls."""
import subprocess
import sys

import pytest

import bench


def test_small_executed_flops_by_hand():
    # tiny fp32 matrix 64 x 32: m = 32 (rows of X = columns of G), n = 64, one
    # 512-column slice; 5 steps -> 17 products of 32 x 32
    fl = bench.small_executed_flops([(64, 32)])
    assert fl == 2 * (32 * 64 + 2 * 32 * 32 * 64 + 1 * 17 * 32 ** 3)
    # attention gate 24 x 2304: m = 24, five slices each running the steps
    fl = bench.small_executed_flops([(24, 2304)])
    assert fl == 2 * (24 * 2304 + 2 * 24 * 24 * 2304 + 5 * 17 * 32 ** 3)
    # m rounded up to 8 rows; empty matrices cost nothing; one step = one product
    assert bench.small_executed_flops([(18, 2304)]) == bench.small_executed_flops([(24, 2304)])
    assert bench.small_executed_flops([(0, 100), (100, 0)]) == 0
    assert bench.small_executed_flops([(8, 512)], steps=1) == 2 * (8 * 512 + 2 * 64 * 512 + 32 ** 3)


def test_metric_and_algorithmic_flops():
    f, a = bench.metric_flops_per_kind([(8192, 6144), (20, 300)])
    m, n = 6144, 8192
    assert f == {"syrk": 2 * m * m * n, "poly": 2 * m ** 3, "update": 2 * m * m * n}
    assert a == {"syrk": m * m * n, "poly": m ** 3, "update": 2 * m * m * n}
    # 5 steps of the per-kind metric FLOPs are the metric's 5 (4 m^2 n + 2 m^3)
    from newton_schulz_04_amd import workloads as wl
    assert 5 * sum(f.values()) == wl.flops_per_matrix(8192, 6144)


def test_pass_bytes():
    b = bench.pass_bytes([(8192, 6144), (16, 4096)], 2)
    # the small matrix has no norm or normalize pass of its own
    assert b["norm_partial"] == 8192 * 6144 * 2
    assert b["prep"] == 8192 * 6144 * 2 + 6144 * 8192 * 2 * 2


def _sampler_with(samples, t_mark, cap=1400.0, error=None):
    s = bench.GpuClockSampler.__new__(bench.GpuClockSampler)
    s.samples, s.t_mark, s.error, s.power_cap_w = samples, t_mark, error, cap
    s._thread = None

    class _NoSmi:
        @staticmethod
        def amdsmi_shut_down():
            pass

    s._smi = _NoSmi()
    return s


def test_clock_summary_covers_the_timed_window_only():
    idle = [(0.0, [100] * 8, 250.0), (0.5, [104] * 8, 260.0)]
    busy = [(1.0 + 0.1 * i, [1700, 1660, 1740, 1680, 1750, 1640, 1790, 1660], 1392.0) for i in range(5)]
    late = [(9.0, [2400] * 8, 300.0)]
    out = _sampler_with(idle + busy + late, t_mark=1.0).stop(t_end=2.0)
    assert out["samples"] == 5
    assert out["gfxclk_mhz"] == pytest.approx(sum(busy[0][1]) / 8, abs=0.1)
    assert out["gfxclk_mhz_per_xcd"] == busy[0][1]
    assert out["socket_power_w"] == 1392.0 and out["power_cap_w"] == 1400.0


def test_clock_summary_of_a_short_pass_takes_the_last_earlier_sample():
    # no sample inside [t_mark, t_end]: the snapshot in effect when it began
    samples = [(0.1, [900] * 8, 500.0), (0.3, [1200] * 8, 800.0), (5.0, [2400] * 8, 300.0)]
    out = _sampler_with(samples, t_mark=0.35).stop(t_end=0.36)
    assert out["samples"] == 1 and out["gfxclk_mhz"] == 1200 and "note" in out


def test_clock_summary_reports_why_it_is_missing():
    assert "error" in _sampler_with([], t_mark=0.0).stop(t_end=1.0)
    out = _sampler_with([(0.5, [1700] * 8, 1000.0)], t_mark=0.0, error="ImportError: no amdsmi").stop(1.0)
    assert out == {"error": "ImportError: no amdsmi"}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout and "--gpus" in r.stderr


def test_traffic_record_is_keyed_to_the_code_not_its_comments():
    from newton_schulz_04_amd.profiling import code_only
    a = "int f(int x) { // doubles x\n    return 2 * x; /* the\n result */ }\n"
    b = "int f(int x) {   // twice x, reworded\n  return 2 * x;  }"
    c = "int f(int x) { return 3 * x; }"
    assert code_only(a) == code_only(b) == "int f(int x) { return 2 * x; }"
    assert code_only(c) != code_only(a)
    # the committed dense-batch record matches the current sources, so the
    # bench reports its traffic
    assert bench.measured_traffic("dense_lowrank", "update") is not None
    assert bench.measured_traffic("no_such_workload", "update") is None
