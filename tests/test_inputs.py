"""Seeded input generator: determinism, dtype rounding, recipe ranges (CPU)."""
import numpy as np
import torch

from linear_attention_recurrence_04_amd import inputs as gi


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0,
                        np.array([0.0, -0.0, 1e-40, 3.0e38, -7.5, 1.00390625, 1.01171875],
                                 np.float32)])
    ours = gi.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(gi.bf16_bits_to_f32(ours),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_prefill_deterministic_and_ranges():
    p = gi.TINY_F32
    a = gi.make_prefill(p, 3)
    b = gi.make_prefill(p, 3)
    c = gi.make_prefill(p, 4)
    for n in ("q", "k", "v", "log_g", "beta"):
        assert np.array_equal(a[n], b[n])
        assert not np.array_equal(a[n], c[n])
    assert a["h0"] is None
    assert a["q"].shape == (1, 128, 2, 64) and a["v"].shape == (1, 128, 2, 64)
    assert np.all(a["log_g"] <= -0.01) and np.all(a["log_g"] >= -0.5)
    assert np.all((a["beta"] > 0) & (a["beta"] < 1))


def test_qwen_gate_law_nonpositive_and_bf16_storage():
    p = gi.Problem("t", 1, 64, 2, 6, 16, 16, 16, "bf16", "qwen", "normal")
    a = gi.make_prefill(p, 0)
    assert np.all(a["log_g"] <= 0.0)
    for n in ("q", "k", "v"):
        assert np.array_equal(gi.round_to_bf16(a[n]), a[n])
    assert a["h0"].shape == (1, 6, 16, 16)
    assert abs(np.std(a["h0"]) - 0.02) < 0.003


def test_decode_steps_windows_reproducible():
    p = gi.DecodeProblem("t", 2, 1, 3, 8, 8, 10)
    full = gi.make_decode_steps(p, 7)
    win = gi.make_decode_steps(p, 7, steps=3, first_step=4)
    for n in full:
        assert np.array_equal(full[n][4:7], win[n])
    assert full["q"].shape == (10, 2, 1, 8) and full["log_g"].shape == (10, 2, 3)
    assert np.all(full["log_g"] <= 0)
