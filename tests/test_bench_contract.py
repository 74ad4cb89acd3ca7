"""The measurement harness on the CPU: the one-GPU rule, the FLOP convention, the main
kernel each workload runs, the amd-smi parser and the traffic lookup."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_flop_convention():
    # 2.5 x the forward's 4 N^2 d per (batch, query head); causal halves it.
    assert bench.flops_bwd(8, 16, 2048, 128, False) == pytest.approx(687.194767360e9)
    assert bench.flops_bwd(1, 16, 16384, 128, True) == pytest.approx(0.5 * 2.5 * 4 * 16384 ** 2 * 128 * 16)
    assert bench.flops_bwd(4, 32, 4096, 64, True) * 2 == bench.flops_bwd(4, 32, 4096, 64, False)


def test_main_kernel_names():
    # 128-row tiles: the two-waves kernel; its full-mask instance writes dQ itself.
    assert bench.main_kernel_name(2048, 128, "auto", False) == "bwd_pair_kernel<128, true, false, true>"
    assert bench.main_kernel_name(4096, 64, "auto", True) == "bwd_pair_kernel<64, true, false, false>"
    # 64-row tiles (N < 512) or the one-wave kernel chosen explicitly.
    assert bench.main_kernel_name(256, 64, "auto", False) == "bwd_main_kernel<64, 2, true, false, false, false>"
    assert bench.main_kernel_name(2048, 128, "one_wave", False) == \
        "bwd_main_kernel<128, 4, true, false, false, false>"


def test_workloads_use_a_schedule_valid_for_their_mask():
    for name, (B, H, Hkv, N, d, causal, best, others, ci) in bench.WORKLOADS.items():
        assert H % Hkv == 0 and d in (64, 128), name
        assert best == ("sym_shift" if causal else "shift"), name
        assert ("causal" in name) == causal, name


def test_amd_smi_parser():
    doc = [{"gpu": 0,
            "clock": {"gfx_0": {"clk": {"value": 1846, "unit": "MHz"}}, "gfx_1": {"clk": {"value": 1797, "unit": "MHz"}},
                      "mem_0": {"clk": {"value": 1900, "unit": "MHz"}}},
            "power": {"socket_power": {"value": 1383, "unit": "W"}, "gfx_voltage": {"value": 700, "unit": "mV"}}}]
    got = bench.parse_smi(doc)
    assert got == {"gfx_clk_mhz": [1846.0, 1797.0], "power_w": [1383.0]}
    assert bench.parse_smi({}) == {"gfx_clk_mhz": [], "power_w": []}


def test_traffic_lookup_refuses_another_kernel():
    # The committed counters are reported only for the kernel (name and source hash) they
    # were taken from.
    assert bench.traffic_bytes("full-d128-N2048", "bwd_main_kernel<128, 4, true, false, false, false>") is None
    assert bench.traffic_bytes("no-such-workload", "bwd_pair_kernel<128, true, false, true>") is None


def test_clock_summary_leaves_idle_readings_out():
    # An idle snapshot (300 W at the full 2.4 GHz) among loaded readings does not raise
    # the mean clock; the fraction is taken at the mean of the loaded readings.
    loaded = {"gfx_clk_mhz": [1800.0, 1700.0], "power_w": [1390.0]}
    idle = {"gfx_clk_mhz": [2400.0, 2400.0], "power_w": [300.0]}
    got = bench.clock_summary([idle, loaded, loaded], 850.0)
    assert got["readings_in_mean"] == 2
    assert got["mean_gfx_mhz"] == 1750.0
    peak = bench.PEAK_BF16_TFLOPS * 1750.0 / bench.PEAK_CLOCK_MHZ
    assert abs(got["main_kernel_frac_at_mean_clock"] - round(850.0 / peak, 4)) < 1e-12
    # No power readings: every reading counts; no clocks: no mean.
    assert bench.clock_summary([{"gfx_clk_mhz": [1800.0], "power_w": []}], 850.0)["readings_in_mean"] == 1
    assert bench.clock_summary([], 850.0) == {"readings_in_mean": 0}
