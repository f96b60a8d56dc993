"""bench.py's host logic on the CPU: the refusal of more than one GPU, the
algorithmic work it divides by, the parity metrics it reports and the
clock-file parsing (no GPU, no timing)."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from linear_attention_recurrence_04_amd import inputs as gi  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_work_of_the_workloads():
    """Bytes and flops per call as the workload definitions give them: the
    27B prefill reads q, k (bf16, 16 key heads), v, log g, beta, h0 and
    writes o and hT; decode reads and writes the fp32 state once per step."""
    p = gi.QWEN27B_PREFILL
    assert bench.prefill_bytes(p) == 549_453_824
    per_token_head = 6 * 128 * 128 + 64 * (128 + 2 * 128) + 2 * 64 * 128 / 3
    assert bench.prefill_useful_flops(p) == pytest.approx(per_token_head * 16384 * 48)
    assert bench.prefill_useful_flops(p) == pytest.approx(100.93e9, rel=1e-3)
    d = gi.QWEN27B_DECODE
    state = 64 * 48 * 128 * 128 * 4
    assert bench.decode_bytes(d) == 2 * state + 64 * (2 * 16 * 128 * 2 + 2 * 48 * 128 * 2 + 8 * 48)
    assert bench.decode_bytes(d) == pytest.approx(404.77e6, rel=1e-4)


def test_parity_metrics():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((1, 50, 3, 8))
    m = bench.parity_metrics(ref.copy(), ref)
    assert m["cos"] == pytest.approx(1.0) and m["max_abs"] == 0.0 and m["rel_fro"] == 0.0
    assert m["norm_ratio"] == pytest.approx(1.0)
    g = ref.copy()
    g[:, :, 1] *= 1.01                      # one head off by 1 %
    assert bench.worst_head_rel(g, ref, (0, 2)) == pytest.approx(0.01)
    m = bench.parity_metrics(g, ref)
    assert 0 < m["rel_fro"] < 0.01 and m["norm_ratio"] > 1.0
    assert bench.parity_metrics(-ref, ref)["cos"] == pytest.approx(-1.0)


def test_clock_level_parsing(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 2103Mhz *\n2: 2400Mhz\n")
    assert bench._current_level_mhz(str(f)) == 2103
    f.write_text("0: 500Mhz\n1: 157Mhz\n2: 2400Mhz *\n")
    assert bench._current_level_mhz(str(f)) == 2400
    f.write_text("garbage\n")
    assert bench._current_level_mhz(str(f)) is None
    assert bench._current_level_mhz(str(tmp_path / "missing")) is None


def test_timing_summary_units():
    t = {"median_ms": 0.3886, "burst_mean_ms": 0.3951, "min_ms": 0.381, "p10_ms": 0.382,
         "p90_ms": 0.392, "max_ms": 0.43, "calls": 20}
    s = bench.timing_summary(t)
    assert s["median_us"] == pytest.approx(388.6) and s["calls"] == 20
