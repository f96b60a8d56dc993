"""GPU parity of the operations around the recurrence against the fp64
oracle: the causal conv1d with its carried state (gdn_causal_conv1d) and the
gated RMS norm (gdn_gated_rmsnorm).  Outputs are rounded to the storage
dtype, so the bar per element is half a unit in the last place of that dtype
on top of fp32 arithmetic (bf16: 2^-8 relative); the carried state holds
inputs, so it is compared bitwise."""
import numpy as np
import pytest

import oracle
from gpu_common import BF16_REL, dev, dev32, host, metrics, say, torch_mod
from linear_attention_recurrence_04_amd import binding as gdn

pytestmark = pytest.mark.gpu

ULP_REL = {"bf16": 2.0 ** -8, "f32": 2.0 ** -20}


def close(gpu, ref, dtype, label, scale=None):
    d = np.abs(gpu - ref)
    scale = np.abs(ref) if scale is None else scale
    worst = float(np.max(d - ULP_REL[dtype] * scale)) if d.size else 0.0
    m = metrics(gpu, ref)
    say(f"  {label}: max|d| {m['max_abs']:.3e}, rel_fro {m['rel_fro']:.3e}")
    assert worst <= 1e-6, (label, worst)
    if dtype == "bf16":
        assert m["rel_fro"] <= BF16_REL


def bf16_round(x):
    """Round fp32 values to bf16 (RNE), returned as fp32 (the stored inputs)."""
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def conv_case(B, T, C, K, dtype, seed, state=True, bias=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, T, C)).astype(np.float32)
    st = rng.standard_normal((B, K - 1, C)).astype(np.float32) if state else None
    if dtype == "bf16":
        x = bf16_round(x)
        st = bf16_round(st) if st is not None else None
    w = (rng.standard_normal((C, K)) / np.sqrt(K)).astype(np.float32)
    b = (0.1 * rng.standard_normal(C)).astype(np.float32) if bias else None
    return x, st, w, b


def run_conv(x, st, w, b, dtype, silu=True, in_place=False):
    torch = torch_mod()
    xd = dev(x, dtype)
    sd = dev(st, dtype) if st is not None else None
    wd = dev32(w)
    bd = dev32(b) if b is not None else None
    if in_place and sd is not None:
        y, so = gdn.gdn_causal_conv1d(xd, wd, bd, sd, silu=silu, state_out=sd)
    else:
        y, so = gdn.gdn_causal_conv1d(xd, wd, bd, sd, silu=silu)
    torch.cuda.synchronize()
    return y, so


@pytest.mark.parametrize("B,T,C,K,dtype,state,bias,silu", [
    (1, 1, 64, 4, "bf16", True, True, True),
    (2, 37, 128, 4, "bf16", True, True, True),
    (1, 2, 64, 4, "bf16", True, False, True),      # fewer tokens than the carried state
    (2, 16, 64, 2, "bf16", False, True, False),
    (3, 100, 96, 3, "f32", True, True, True),
    (1, 33, 32, 1, "f32", False, False, True),     # K = 1: no state
    (2, 129, 2048, 4, "bf16", True, True, True),   # several token tiles and channel blocks
])
def test_conv1d_matches_oracle(B, T, C, K, dtype, state, bias, silu):
    say(f"conv1d B={B} T={T} C={C} K={K} {dtype} state={state} bias={bias} silu={silu}")
    x, st, w, b = conv_case(B, T, C, K, dtype, seed=T + C, state=state, bias=bias)
    y, so = run_conv(x, st, w, b, dtype, silu=silu)
    y_ref, s_ref = oracle.causal_conv1d(x, w, b, st, silu=silu)
    close(host(y), y_ref, dtype, "y")
    if K > 1:
        assert np.array_equal(host(so), s_ref)


def test_conv1d_state_only_and_empty():
    """T = 0 copies the state; no state in and K = 4 with T = 2 pads with zeros."""
    torch = torch_mod()
    x, st, w, b = conv_case(2, 0, 64, 4, "bf16", seed=1)
    y, so = run_conv(x, st, w, b, "bf16")
    assert y.numel() == 0 and np.array_equal(host(so), st)
    x, _, w, b = conv_case(2, 2, 64, 4, "bf16", seed=2, state=False)
    y, so = run_conv(x, None, w, b, "bf16")
    y_ref, s_ref = oracle.causal_conv1d(x, w, b, None)
    close(host(y), y_ref, "bf16", "no state")
    assert np.array_equal(host(so), s_ref)
    torch.cuda.synchronize()


def test_conv1d_split_invariance_and_in_place_state():
    """One call over 64 tokens and calls of 5, 1, 26, 1 and 31 tokens carrying
    the state in place: bitwise the same outputs and final state."""
    torch = torch_mod()
    x, st, w, b = conv_case(2, 64, 256, 4, "bf16", seed=3)
    y1, s1 = run_conv(x, st, w, b, "bf16")
    state = dev(st, "bf16")
    xd, wd, bd = dev(x, "bf16"), dev32(w), dev32(b)
    outs, t0 = [], 0
    for n in (5, 1, 26, 1, 31):
        y, _ = gdn.gdn_causal_conv1d(xd[:, t0:t0 + n].contiguous(), wd, bd, state, state_out=state)
        outs.append(y)
        t0 += n
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=1), y1) and torch.equal(state, s1)


def test_conv1d_one_tile_and_multi_tile_calls_agree():
    """A call of 200 tokens (four tiles: the state written by the separate
    state kernel) against calls of 64, 1, 70 and 65 tokens (one tile: the conv
    kernel writes the state itself; more: the state kernel), the state carried
    in place: bitwise the same outputs and final state."""
    torch = torch_mod()
    x, st, w, b = conv_case(3, 200, 512, 4, "bf16", seed=6)
    y1, s1 = run_conv(x, st, w, b, "bf16")
    state = dev(st, "bf16")
    xd, wd, bd = dev(x, "bf16"), dev32(w), dev32(b)
    outs, t0 = [], 0
    for n in (64, 1, 70, 65):
        y, _ = gdn.gdn_causal_conv1d(xd[:, t0:t0 + n].contiguous(), wd, bd, state, state_out=state)
        outs.append(y)
        t0 += n
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=1), y1) and torch.equal(state, s1)


def test_conv1d_decode_steps_in_place():
    """27B decode shape: 64 sequences, C = 10240 channels (q, k: 2 x 16 x 128;
    v: 48 x 128), 20 single-token calls updating the state in place, bitwise
    one 20-token call, and within the bar of the oracle."""
    torch = torch_mod()
    x, st, w, b = conv_case(64, 20, 10240, 4, "bf16", seed=4)
    y1, s1 = run_conv(x, st, w, b, "bf16")
    state = dev(st, "bf16")
    xd, wd, bd = dev(x, "bf16"), dev32(w), dev32(b)
    outs = []
    for t in range(20):
        y, _ = gdn.gdn_causal_conv1d(xd[:, t:t + 1].contiguous(), wd, bd, state, state_out=state)
        outs.append(y)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=1), y1) and torch.equal(state, s1)
    y_ref, s_ref = oracle.causal_conv1d(x, w, b, st)
    close(host(y1), y_ref, "bf16", "decode steps")
    assert np.array_equal(host(s1), s_ref)


def test_conv1d_full_27b_prefill():
    """B=1, T=16384, C=10240, K=4, bf16 (the 27B projections of one layer):
    every element against the oracle."""
    say("conv1d 27B prefill shape")
    x, st, w, b = conv_case(1, 16384, 10240, 4, "bf16", seed=5)
    y, so = run_conv(x, st, w, b, "bf16")
    y_ref, s_ref = oracle.causal_conv1d(x, w, b, st)
    close(host(y), y_ref, "bf16", "27B conv1d")
    assert np.array_equal(host(so), s_ref)


def norm_case(rows, D, dtype, seed, gate=True):
    rng = np.random.default_rng(seed)
    x = (3.0 * rng.standard_normal((rows, D))).astype(np.float32)
    z = rng.standard_normal((rows, D)).astype(np.float32) if gate else None
    if dtype == "bf16":
        x = bf16_round(x)
        z = bf16_round(z) if z is not None else None
    w = rng.uniform(0.5, 1.5, D).astype(np.float32)
    return x, z, w


@pytest.mark.parametrize("rows,D,dtype,gate", [
    (1, 128, "bf16", True), (1000, 128, "bf16", True), (7, 64, "bf16", False),
    (33, 256, "bf16", True), (5, 512, "bf16", True), (10, 128, "f32", True), (3, 16, "bf16", True),
    (513, 32, "f32", False),
])
def test_gated_rmsnorm_matches_oracle(rows, D, dtype, gate):
    torch = torch_mod()
    x, z, w = norm_case(rows, D, dtype, seed=rows + D, gate=gate)
    xd = dev(x, dtype)
    y = gdn.gdn_gated_rmsnorm(xd, dev(z, dtype) if z is not None else None, dev32(w), 1e-6)
    torch.cuda.synchronize()
    y_ref = oracle.gated_rmsnorm(x, z, w, eps=1e-6)
    close(host(y), y_ref, dtype, f"rmsnorm {rows}x{D} {dtype}")
    # in place gives bitwise the same result
    gdn.gdn_gated_rmsnorm(xd, dev(z, dtype) if z is not None else None, dev32(w), 1e-6, out=xd)
    torch.cuda.synchronize()
    assert torch.equal(xd, y)


@pytest.mark.parametrize("rows,D,dtype", [(77, 128, "bf16"), (5, 512, "bf16"), (10, 128, "f32")])
def test_gated_rmsnorm_writes_nothing_past_the_rows(rows, D, dtype):
    """The lanes past the last row of a ragged block (their stores dropped by
    the buffer bound, not by a branch) leave the memory after y untouched."""
    torch = torch_mod()
    x, z, w = norm_case(rows, D, dtype, seed=3 * rows + D)
    big = dev(np.full((rows + 64, D), 7.0, dtype=np.float32), dtype)
    y = big[:rows]
    gdn.gdn_gated_rmsnorm(dev(x, dtype), dev(z, dtype), dev32(w), 1e-6, out=y)
    torch.cuda.synchronize()
    assert torch.all(big[rows:] == 7.0)
    close(host(y), oracle.gated_rmsnorm(x, z, w, eps=1e-6), dtype, f"rmsnorm {rows}x{D} into a larger buffer")


def test_gated_rmsnorm_zero_rows_and_nan_isolation():
    torch = torch_mod()
    x, z, w = norm_case(16, 128, "bf16", seed=9)
    x[3] = 0.0
    x[7, 5] = np.nan
    y = host(gdn.gdn_gated_rmsnorm(dev(x, "bf16"), dev(z, "bf16"), dev32(w), 1e-6))
    torch.cuda.synchronize()
    assert np.array_equal(y[3], np.zeros(128))
    assert np.all(np.isnan(y[7]))
    keep = [r for r in range(16) if r != 7]
    y_ref = oracle.gated_rmsnorm(x[keep], z[keep], w, eps=1e-6)
    close(y[keep], y_ref, "bf16", "rows beside a NaN row")


def test_gated_rmsnorm_full_27b_output():
    """The 27B prefill output: 16384 tokens x 48 value heads rows of 128."""
    torch = torch_mod()
    say("gated rmsnorm 27B output shape")
    x, z, w = norm_case(16384 * 48, 128, "bf16", seed=10)
    y = gdn.gdn_gated_rmsnorm(dev(x, "bf16"), dev(z, "bf16"), dev32(w), 1e-6)
    torch.cuda.synchronize()
    y_ref = oracle.gated_rmsnorm(x, z, w, eps=1e-6)
    close(host(y), y_ref, "bf16", "27B rmsnorm")
