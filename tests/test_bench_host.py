"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the roofline arithmetic, the bracket
split of the timed steps, the algorithmic byte counts of the decode workloads and the plausibility
check of clock readings."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from scaled_dot_product_fa2_amd import inputs as I  # noqa: E402


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == int(n) and "one GPU" in line["error"]


def test_roofline_fractions():
    m = bench.roofline_mfma(flops=2.5e12, ms=2.0, traffic=None)  # 1.25 PFLOP/s
    assert m["bound"] == "mfma" and m["achieved"] == pytest.approx(1250.0)
    assert m["frac"] == pytest.approx(0.5) and m["peak"] == 2500.0
    h = bench.roofline_hbm(nbytes=4e9, ms=1.0, traffic=123)  # 4 TB/s
    assert h["bound"] == "hbm" and h["achieved"] == pytest.approx(4000.0)
    assert h["frac"] == pytest.approx(0.5) and h["traffic"] == 123


@pytest.mark.parametrize("steps,brackets", [(20, 4), (21, 4), (3, 4), (1, 1), (50, 4), (7, 3)])
def test_brackets_cover_the_steps_exactly(steps, brackets):
    sizes = bench._bracket_sizes(steps, brackets)
    assert sum(sizes) == steps and len(sizes) == min(brackets, steps)
    assert max(sizes) - min(sizes) <= 1 and min(sizes) >= 1


def test_decode_algorithmic_bytes():
    # K and V rows once (4 d bytes per key and KV head), Q and O in bf16, LSE in fp32
    assert bench.algorithmic_bytes(I.WORKLOADS["decode_gqa_nq1"]) == 268_567_552
    assert bench.algorithmic_bytes(I.WORKLOADS["decode_gqa_nq4"]) == 268_963_840


def test_clock_readings_that_imply_an_overbusy_matrix_core_are_withdrawn():
    # 1175 TFLOP/s needs at least 1175 / (2500 * 0.9) * 2400 = 1253 MHz
    kept = bench.checked_clock({"mhz": 1600.0, "spin_ms": 1.0}, 1175.0)
    assert kept["mhz"] == 1600.0 and "note" not in kept
    gone = bench.checked_clock({"mhz": 1146.0, "spin_ms": 1.0}, 1175.0)
    assert gone["mhz"] is None and gone["mhz_read"] == 1146.0 and "starved" in gone["note"]
    assert bench.checked_clock({"mhz": None}, 1175.0) == {"mhz": None}
    assert bench.checked_clock({"mhz": 900.0}, None)["mhz"] == 900.0
