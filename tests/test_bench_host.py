"""CPU checks of the benchmark's host logic: the one-GPU contract and the
algorithmic FLOP and byte counts its roofline uses."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_flop_and_byte_counts_at_d20():
    B, T, H, D = 32, 2048, 10, 128
    fl = bench.train_flops(B, T, H, D)
    unit = B * H * T * T * D
    assert unit == 171798691840                      # causal: half of 2 T^2 D per head
    assert fl["fwd"] == 2 * unit and fl["dkdv"] == 4 * unit and fl["dq"] == unit
    assert fl["fwd+bwd"] == 7 * unit
    by = bench.design_bytes(B, T, H, D)
    t = B * T * H * D * 2
    r = B * H * T * 4
    assert by["fwd"] == 4 * t + r                   # q, k, v read, o written, lse written
    assert by["delta"] == 2 * t + r
    nblk = T // 32
    assert by["dq"] == 2 * t + B * H * nblk * (nblk + 1) // 2 * 2048
    mb = bench.method_bytes(B, T, H, D)
    assert mb["dkdv"] == 6 * t + 2 * r              # q, k, v, dO, lse, delta in; dk, dv out
    assert mb["dq"] == 5 * t + 2 * r                # q, k, v, dO, lse, delta in; dq out
    # the step minimum quoted for d20: 674 MB forward, 1345 MB backward
    assert mb["fwd_min"] == 673710080 and mb["bwd_min"] == 1344798720


@pytest.mark.parametrize("T,W,expect", [(4, None, 10), (4, 0, 4), (4, 1, 7), (4, 10, 10),
                                        (2048, 1024, 1574400)])
def test_visible_pairs(T, W, expect):
    """Pairs (i, j) with j <= i (and i - j <= W): brute force for small T, and
    the figure the sliding-window line reports at T = 2048, W = 1024."""
    assert bench.visible_pairs(T, W) == expect
    if T <= 16:
        brute = sum(1 for i in range(T) for j in range(i + 1) if W is None or i - j <= W)
        assert brute == expect


def test_sclk_sampler_reads_the_starred_level(tmp_path, monkeypatch):
    """The clock sampler takes the starred line of pp_dpm_sclk (the driver's
    current level) and reports the busiest card's distribution."""
    import glob
    busy = tmp_path / "busy"
    idle = tmp_path / "idle"
    busy.write_text("0: 500Mhz\n1: 2024Mhz *\n2: 2400Mhz\n")
    idle.write_text("S: 113Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    monkeypatch.setattr(glob, "glob", lambda pattern: [str(idle), str(busy)])
    calls = []
    res = bench.sample_sclk(lambda: calls.append(1) or __import__("time").sleep(0.005), 0.05)
    assert calls and res["source"] == str(busy)
    assert res["median_MHz"] == 2024.0 and res["min_MHz"] == res["max_MHz"] == 2024.0
    monkeypatch.setattr(glob, "glob", lambda pattern: [])
    assert bench.sample_sclk(lambda: None, 0.01)["source"] is None


def test_sclk_sampler_reports_board_power_and_cap(tmp_path, monkeypatch):
    """Beside the clock, the sampler reads the card's hwmon power1_input
    (microwatts) and reports it in watts with the power1_cap limit."""
    import glob
    real_glob = glob.glob
    dev = tmp_path / "card0" / "device"
    hw = dev / "hwmon" / "hwmon3"
    hw.mkdir(parents=True)
    (dev / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 2100Mhz *\n")
    (hw / "power1_input").write_text("1350000000\n")
    (hw / "power1_cap").write_text("1400000000\n")
    monkeypatch.setattr(glob, "glob", lambda pattern: [str(dev / "pp_dpm_sclk")]
                        if pattern.startswith("/sys/class/drm") else real_glob(pattern))
    res = bench.sample_sclk(lambda: __import__("time").sleep(0.005), 0.05)
    assert res["median_MHz"] == 2100.0
    pw = res["power"]
    assert pw["source"] == str(hw / "power1_input") and pw["samples"] >= 1
    assert pw["median_W"] == pw["max_W"] == 1350.0 and pw["cap_W"] == 1400.0
