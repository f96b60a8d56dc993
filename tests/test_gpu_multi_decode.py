"""GPU parity of gdn_decode_multi: T decode tokens per sequence in one call with
the state on chip, and the state after every token for speculative rollback.
Per-token expected states come from the oracle run one token at a time,
carrying the state (the oracle's splitting pin makes that one run)."""
import numpy as np
import pytest

import oracle
from gpu_common import (NTHREADS, assert_parity, dev, dev32, host, metrics, per_head_rel,
                        BF16_REL, F32_MAX_ABS, say, torch_mod)
from linear_attention_recurrence_04_amd import binding as gdn
from linear_attention_recurrence_04_amd import inputs as gi

pytestmark = pytest.mark.gpu


def oracle_tokens(seq, state0, gates=None):
    """(o [B,T,Hv,d], states after each token [B,T,Hv,d,d]) from the oracle."""
    lg, bt = (seq["log_g"], seq["beta"]) if gates is None else gates
    T = seq["q"].shape[1]
    h = state0
    outs, sts = [], []
    for t in range(T):
        o, h = oracle.gdn_sequential(seq["q"][:, t:t + 1], seq["k"][:, t:t + 1],
                                     seq["v"][:, t:t + 1], lg[:, t:t + 1], bt[:, t:t + 1], h,
                                     nthreads=NTHREADS)
        outs.append(o[:, 0])
        sts.append(h)
    return np.stack(outs, axis=1), np.stack(sts, axis=1)


def check(gpu, ref, dtype, label):
    m = metrics(gpu, ref)
    say(f"  {label}: {m}")
    if dtype == "f32":
        assert m["max_abs"] <= F32_MAX_ABS, (label, m)
    else:
        assert m["rel_fro"] <= BF16_REL, (label, m)


def run_multi(seq, state0, dtype, want_states=True, raw=None):
    torch = torch_mod()
    state = dev32(state0)
    kw = {}
    if raw is not None:
        lg, bt = dev32(raw["a"]), dev32(raw["b"])
        kw = {"A_log": dev32(raw["A_log"]), "dt_bias": dev32(raw["dt_bias"])}
    else:
        lg, bt = dev32(seq["log_g"]), dev32(seq["beta"])
    o, sts = gdn.gdn_decode_multi(dev(seq["q"], dtype), dev(seq["k"], dtype), dev(seq["v"], dtype),
                                  lg, bt, state, want_states=want_states, **kw)
    torch.cuda.synchronize()
    return o, state, sts


@pytest.mark.parametrize("dtype,d,Hk,Hv", [("f32", 64, 2, 2), ("bf16", 128, 2, 6)])
@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_multi_decode_matches_oracle(dtype, d, Hk, Hv, T):
    torch = torch_mod()
    B = 3
    say(f"multi decode {dtype} d={d} {Hk}x{Hv} T={T}")
    rng = np.random.default_rng(40 + T)
    state0 = (0.05 * rng.standard_normal((B, Hv, d, d))).astype(np.float32)
    seq = gi.custom_prefill(B, T, Hk, Hv, d, d, seed=41 + T, dtype=dtype, gate="qwen")
    o, state, sts = run_multi(seq, state0, dtype)
    o_ref, st_ref = oracle_tokens(seq, state0)
    check(host(o), o_ref, dtype, "o")
    check(host(state), st_ref[:, -1], dtype, "final state")
    for t in range(T):
        check(host(sts[:, t]), st_ref[:, t], dtype, f"state after token {t}")
    assert torch.equal(sts[:, -1], state)
    # the same tokens as T single decode steps agree to rounding: the two
    # kernels sum the column reductions in different orders (256 threads of 16
    # rows here, 512 or 1024 threads for a single step at head dim 128), so
    # the fp32 states agree to a few fp32 ulps and a bf16 output may round the
    # other way (one bf16 ulp, 2^-7 relative)
    state_s = dev32(state0)
    outs = []
    for t in range(T):
        outs.append(gdn.gdn_decode_step(dev(seq["q"][:, t], dtype), dev(seq["k"][:, t], dtype),
                                        dev(seq["v"][:, t], dtype), dev32(seq["log_g"][:, t]),
                                        dev32(seq["beta"][:, t]), state_s))
    torch.cuda.synchronize()
    o_rtol = 2.0 ** -7 if dtype == "bf16" else 1e-5
    assert np.allclose(host(torch.stack(outs, dim=1)), host(o), rtol=o_rtol, atol=1e-6)
    assert np.allclose(host(state_s), host(state), rtol=1e-5, atol=1e-7)


def test_multi_decode_raw_gates_and_rollback():
    """Raw gates in the kernel; then a verifier accepts 2 of 5 draft tokens,
    restores the state after token 2 and decodes one correction token."""
    torch = torch_mod()
    B, Hk, Hv, d, T = 2, 1, 3, 128, 5
    rng = np.random.default_rng(3)
    state0 = (0.05 * rng.standard_normal((B, Hv, d, d))).astype(np.float32)
    seq = gi.custom_prefill(B, T + 1, Hk, Hv, d, d, seed=5, dtype="bf16", gate="qwen")
    raw = gi.make_raw_gates((B, T + 1), Hv, seed=5)
    gates = oracle.qwen_gates(raw["a"], raw["b"], raw["A_log"], raw["dt_bias"])
    draft = {n: seq[n][:, :T] for n in ("q", "k", "v")}
    draft_raw = dict(raw, a=raw["a"][:, :T], b=raw["b"][:, :T])
    o, state, sts = run_multi(draft, state0, "bf16", raw=draft_raw)
    o_ref, st_ref = oracle_tokens(draft, state0, gates=(gates[0][:, :T], gates[1][:, :T]))
    check(host(o), o_ref, "bf16", "raw-gate o")
    check(host(sts), st_ref, "bf16", "raw-gate per-token states")
    # accept tokens 0, 1; the correction token is token T of seq
    state = sts[:, 1].contiguous()
    t = T
    o_fix = gdn.gdn_decode_step_gated(dev(seq["q"][:, t], "bf16"), dev(seq["k"][:, t], "bf16"),
                                      dev(seq["v"][:, t], "bf16"), dev32(raw["a"][:, t]),
                                      dev32(raw["b"][:, t]), dev32(raw["A_log"]),
                                      dev32(raw["dt_bias"]), state)
    torch.cuda.synchronize()
    keep = [0, 1, T]
    acc = {n: seq[n][:, keep] for n in ("q", "k", "v")}
    o_acc, st_acc = oracle_tokens(acc, state0, gates=(gates[0][:, keep], gates[1][:, keep]))
    check(host(o_fix), o_acc[:, -1], "bf16", "correction token")
    check(host(state), st_acc[:, -1], "bf16", "state after rollback + correction")


def test_multi_decode_zero_tokens_and_no_states():
    torch = torch_mod()
    B, Hv, d = 2, 2, 64
    rng = np.random.default_rng(1)
    state0 = (0.05 * rng.standard_normal((B, Hv, d, d))).astype(np.float32)
    seq = gi.custom_prefill(B, 0, 1, Hv, d, d, seed=1, dtype="f32")
    o, state, sts = run_multi(seq, state0, "f32")
    assert o.shape == (B, 0, Hv, d) and sts.shape == (B, 0, Hv, d, d)
    assert torch.equal(state.cpu(), torch.from_numpy(state0))
    seq = gi.custom_prefill(B, 3, 1, Hv, d, d, seed=2, dtype="f32", gate="qwen")
    o, state, none = run_multi(seq, state0, "f32", want_states=False)
    assert none is None
    o_ref, st_ref = oracle_tokens(seq, state0)
    check(host(o), o_ref, "f32", "o without states")
    check(host(state), st_ref[:, -1], "f32", "final state without states")


def test_qwen27b_multi_decode_full_size():
    """The 27B decode workload (B=64, 16/48 heads) with 4 tokens per call (a
    3-token draft plus one), every head against the oracle."""
    d = gi.QWEN27B_DECODE
    T = 4
    say(f"{d.name}: {T} tokens per call")
    state0 = gi.make_decode_state(d, 0)
    st = gi.make_decode_steps(d, 0, steps=T)
    seq = {n: np.ascontiguousarray(np.swapaxes(st[n], 0, 1)) for n in st}
    o, state, sts = run_multi(seq, state0, "bf16")
    o_ref, st_ref = oracle_tokens(seq, state0)
    assert_parity(host(o), o_ref, host(state), st_ref[:, -1], "bf16", f"{d.name} T={T}")
    for t in range(T - 1):
        g, r = host(sts[:, t]), st_ref[:, t]
        check(g, r, "bf16", f"state after token {t}")
        assert per_head_rel(g, r, (0, 1)) <= BF16_REL
