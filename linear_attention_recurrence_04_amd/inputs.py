"""Seeded synthetic inputs for the gated delta rule (numpy only).

This module is shared by the tests, the benchmark, the smoke check and the
oracle driver.  It draws random numbers and rounds them to the storage dtype;
it holds none of the recurrence's arithmetic (no normalisation, no decay
cumsum, no state update).

Workload shapes mirror the pages:
  * 0.8B head shape: 16 key heads / 16 value heads, head dim 128
    ("Qwen3.5 Gated Delta Net NKI Kernel for AWS Neuron", table
    "Supported Models");
  * 27B head shape: 16 key heads shared 1:3 by 48 value heads, head dim 128
    ("Add Qwen3.6-27B contrib model with vLLM APC baseline", table
    "Architecture");
  * long prompts processed as consecutive 512-token context-encoding calls
    carrying the recurrent state (same table, "CTE bucket 512").

Gate law for the Qwen-shaped workloads: log g = -exp(A_log) * softplus(dt),
which is never positive ("Qwen3.5 Gated Delta Net NKI Kernel for AWS Neuron",
section "Correctness Contract"); the bias of softplus is folded into dt.

Draw order (PCG64 via numpy.random.default_rng(seed)):
  q, k, v, beta-logits, then the log-decay draws (uniforms, or A_log then dt),
  then the initial state.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# --------------------------------------------------------------------------
# bf16 storage helpers (round-to-nearest-even, like every IEEE conversion)
# --------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE) and return the 16-bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array holding exactly the bf16-representable neighbour of x."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


# --------------------------------------------------------------------------
# problem description
# --------------------------------------------------------------------------


@dataclass
class Problem:
    """Shapes and input recipe of one prefill workload."""
    name: str
    B: int
    T: int
    Hk: int
    Hv: int
    dk: int
    dv: int
    chunk: int
    dtype: str            # "f32" or "bf16": storage dtype of q, k, v and o
    gate: str             # "uniform": log g ~ U(lo, hi); "qwen": -exp(A_log) softplus(dt)
    h0: str               # "zero" or "normal" (N(0, 0.02))
    gate_lo: float = -0.5
    gate_hi: float = -0.01
    extra: dict = field(default_factory=dict)

    @property
    def tokens(self) -> int:
        return self.B * self.T


# The five workloads (shape + recipe).  Names describe what they are.
TINY_F32 = Problem("tiny_fp32_B1_T128_H2_d64", 1, 128, 2, 2, 64, 64, 32, "f32", "uniform", "zero")
QWEN08B_PREFILL = Problem("qwen0.8b_prefill_B1_T2048_Hk16_Hv16_d128", 1, 2048, 16, 16, 128, 128, 64,
                          "bf16", "uniform", "normal")
QWEN27B_PREFILL = Problem("qwen27b_prefill_B1_T16384_Hk16_Hv48_d128", 1, 16384, 16, 48, 128, 128, 64,
                          "bf16", "qwen", "normal")
QWEN27B_LONG = Problem("qwen27b_long_B1_T131072_Hk16_Hv48_d128_512x256", 1, 131072, 16, 48, 128, 128,
                       64, "bf16", "qwen", "zero", extra={"call_tokens": 512})


@dataclass
class DecodeProblem:
    name: str
    B: int
    Hk: int
    Hv: int
    dk: int
    dv: int
    steps: int
    dtype: str = "bf16"


QWEN27B_DECODE = DecodeProblem("qwen27b_decode_B64_Hk16_Hv48_d128", 64, 16, 48, 128, 128, 1000)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the storage dtype; returned as float32 holding exact values."""
    x = x.astype(np.float32)
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def _gates(rng: np.random.Generator, shape_bt: tuple, Hv: int, gate: str,
           lo: float, hi: float, a_log: Optional[np.ndarray] = None) -> np.ndarray:
    """Log-decay draws of shape shape_bt + (Hv,), float32."""
    if gate == "uniform":
        return rng.uniform(lo, hi, size=shape_bt + (Hv,)).astype(np.float32)
    if gate == "qwen":
        if a_log is None:
            a_log = rng.uniform(-2.0, 1.0, size=(Hv,))
        dt = rng.standard_normal(size=shape_bt + (Hv,))
        return (-np.exp(a_log) * softplus(dt)).astype(np.float32)
    raise ValueError(gate)


def make_prefill(p: Problem, seed: int, T: Optional[int] = None) -> dict:
    """Seeded inputs of one prefill call.

    Returns float32 arrays (values exactly representable in the storage
    dtype): q, k [B,T,Hk,dk]; v [B,T,Hv,dv]; log_g, beta [B,T,Hv]; h0
    [B,Hv,dk,dv] or None.  ``T`` overrides the problem's length (same recipe).
    """
    T = p.T if T is None else T
    rng = np.random.default_rng(seed)
    B, Hk, Hv, dk, dv = p.B, p.Hk, p.Hv, p.dk, p.dv
    q = _store(rng.standard_normal((B, T, Hk, dk)), p.dtype)
    k = _store(rng.standard_normal((B, T, Hk, dk)), p.dtype)
    v = _store(rng.standard_normal((B, T, Hv, dv)), p.dtype)
    beta = sigmoid(rng.standard_normal((B, T, Hv))).astype(np.float32)
    log_g = _gates(rng, (B, T), Hv, p.gate, p.gate_lo, p.gate_hi)
    h0 = None
    if p.h0 == "normal":
        h0 = (0.02 * rng.standard_normal((B, Hv, dk, dv))).astype(np.float32)
    return {"q": q, "k": k, "v": v, "log_g": log_g, "beta": beta, "h0": h0}


def make_long_segment(p: Problem, seed: int, call: int) -> dict:
    """Inputs of one call of a long prompt processed in fixed-size calls.

    Call ``call`` covers tokens [call*Tc, (call+1)*Tc), Tc = p.extra["call_tokens"],
    drawn from its own stream so any call is reproducible alone; A_log (a
    per-value-head model parameter) is shared by every call.  Same recipe and
    draw order as make_prefill; the initial state of the prompt is zero.
    """
    Tc = p.extra["call_tokens"]
    B, Hk, Hv, dk, dv = p.B, p.Hk, p.Hv, p.dk, p.dv
    a_log = np.random.default_rng([seed, 7]).uniform(-2.0, 1.0, size=(Hv,))
    rng = np.random.default_rng([seed, 1000 + call])
    q = _store(rng.standard_normal((B, Tc, Hk, dk)), p.dtype)
    k = _store(rng.standard_normal((B, Tc, Hk, dk)), p.dtype)
    v = _store(rng.standard_normal((B, Tc, Hv, dv)), p.dtype)
    beta = sigmoid(rng.standard_normal((B, Tc, Hv))).astype(np.float32)
    log_g = _gates(rng, (B, Tc), Hv, p.gate, p.gate_lo, p.gate_hi, a_log=a_log)
    return {"q": q, "k": k, "v": v, "log_g": log_g, "beta": beta, "h0": None}


def make_decode_state(p: DecodeProblem, seed: int) -> np.ndarray:
    """Initial decode state [B,Hv,dk,dv] ~ N(0, 0.02), float32."""
    rng = np.random.default_rng([seed, 1])
    return (0.02 * rng.standard_normal((p.B, p.Hv, p.dk, p.dv))).astype(np.float32)


def decode_a_log(p: DecodeProblem, seed: int) -> np.ndarray:
    """A_log ~ U(-2, 1), fixed per (sequence, value head) for the whole decode run."""
    rng = np.random.default_rng([seed, 2])
    return rng.uniform(-2.0, 1.0, size=(p.B, p.Hv))


def make_decode_steps(p: DecodeProblem, seed: int, steps: Optional[int] = None,
                      first_step: int = 0) -> dict:
    """Seeded per-step decode inputs for steps [first_step, first_step+steps).

    Each step's draws come from its own stream, so any window of steps is
    reproducible on its own.  Returns float32 arrays with a leading step axis:
    q, k [S,B,Hk,dk]; v [S,B,Hv,dv]; log_g, beta [S,B,Hv].
    """
    steps = p.steps if steps is None else steps
    a_log = decode_a_log(p, seed)
    out = {n: [] for n in ("q", "k", "v", "log_g", "beta")}
    for s in range(first_step, first_step + steps):
        rng = np.random.default_rng([seed, 100 + s])
        out["q"].append(_store(rng.standard_normal((p.B, p.Hk, p.dk)), p.dtype))
        out["k"].append(_store(rng.standard_normal((p.B, p.Hk, p.dk)), p.dtype))
        out["v"].append(_store(rng.standard_normal((p.B, p.Hv, p.dv)), p.dtype))
        out["beta"].append(sigmoid(rng.standard_normal((p.B, p.Hv))).astype(np.float32))
        dt = rng.standard_normal((p.B, p.Hv))
        out["log_g"].append((-np.exp(a_log) * softplus(dt)).astype(np.float32))
    return {n: np.stack(v_) if v_ else np.zeros((0,), np.float32) for n, v_ in out.items()}


def custom_prefill(B: int, T: int, Hk: int, Hv: int, dk: int, dv: int, *, seed: int,
                   dtype: str = "f32", gate: str = "uniform", h0: str = "zero",
                   gate_lo: float = -0.5, gate_hi: float = -0.01, chunk: int = 64) -> dict:
    """Same recipe at an arbitrary shape (edge cases and sweeps)."""
    p = Problem("custom", B, T, Hk, Hv, dk, dv, chunk, dtype, gate, h0, gate_lo, gate_hi)
    return make_prefill(p, seed)


def make_raw_gates(shape_rows: tuple, Hv: int, seed: int) -> dict:
    """Raw gate inputs of the fused gate prologue, fp32: projections a, b
    [*shape_rows, Hv] ~ N(0, 1); per-value-head A_log ~ U(-2, 1) and
    dt_bias ~ N(0, 0.5^2).  (The gate law itself is applied by the kernels
    and by the oracle, not here.)"""
    rng = np.random.default_rng(10_000 + seed)
    a = rng.standard_normal(tuple(shape_rows) + (Hv,)).astype(np.float32)
    b = rng.standard_normal(tuple(shape_rows) + (Hv,)).astype(np.float32)
    A_log = rng.uniform(-2.0, 1.0, Hv).astype(np.float32)
    dt_bias = (0.5 * rng.standard_normal(Hv)).astype(np.float32)
    return {"a": a, "b": b, "A_log": A_log, "dt_bias": dt_bias}
