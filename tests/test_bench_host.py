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
    by = bench.train_bytes(B, T, H, D)
    t = B * T * H * D * 2
    assert by["fwd"] == 4 * t + B * H * T * 4       # q, k, v read, o written, lse written
    assert by["delta"] == 2 * t + B * H * T * 4
    nblk = T // 32
    assert by["dq"] == 2 * t + B * H * nblk * (nblk + 1) // 2 * 2048


@pytest.mark.parametrize("T,W,expect", [(4, None, 10), (4, 0, 4), (4, 1, 7), (4, 10, 10),
                                        (2048, 1024, 1574400)])
def test_visible_pairs(T, W, expect):
    """Pairs (i, j) with j <= i (and i - j <= W): brute force for small T, and
    the figure the sliding-window line reports at T = 2048, W = 1024."""
    assert bench.visible_pairs(T, W) == expect
    if T <= 16:
        brute = sum(1 for i in range(T) for j in range(i + 1) if W is None or i - j <= W)
        assert brute == expect
