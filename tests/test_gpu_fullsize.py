"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, against the fp64 oracle on every (sequence, head).  Each test
prints the worst per-(sequence, head) relative error of o and of the state
beside the bar."""
import numpy as np
import pytest

import oracle
from gpu_common import (BF16_REL, NTHREADS, assert_parity, dev, dev32, host, margins, metrics,
                        per_head_rel, run_oracle, run_prefill, say, torch_mod)
from linear_attention_recurrence_04_amd import binding as gdn
from linear_attention_recurrence_04_amd import inputs as gi

pytestmark = pytest.mark.gpu


def test_qwen08b_prefill_full():
    """B=1, T=2048, 16/16 heads, d=128, bf16, chunk 64, h0 ~ N(0, 0.02): every head."""
    p = gi.QWEN08B_PREFILL
    say(f"{p.name}: generating")
    inp = gi.make_prefill(p, 0)
    o, hT = run_prefill(inp, "bf16", p.chunk)
    say("  oracle (all heads)")
    o_ref, h_ref = run_oracle(inp)
    assert_parity(host(o), o_ref, host(hT), h_ref, "bf16", p.name)
    margins(host(o), o_ref, host(hT), h_ref, p.name)


@pytest.mark.parametrize("entry", ["gdn_chunk_prefill", "gdn_chunk_prefill_onchip"])
def test_qwen27b_prefill_full_all_heads(entry):
    """B=1, T=16384, 16 key / 48 value heads, d=128, bf16, the benchmark's
    inputs (seed 0) and launch: all 48 value heads against the oracle."""
    torch = torch_mod()
    p = gi.QWEN27B_PREFILL
    say(f"{p.name} via {entry}: generating")
    inp = gi.make_prefill(p, 0)
    q, k, v = dev(inp["q"], "bf16"), dev(inp["k"], "bf16"), dev(inp["v"], "bf16")
    lg, bt, h0 = dev32(inp["log_g"]), dev32(inp["beta"]), dev32(inp["h0"])
    if entry == "gdn_chunk_prefill":
        o, hT = gdn.gdn_chunk_prefill(q, k, v, lg, bt, h0, chunk=p.chunk)
    else:
        o, hT, _ = gdn.gdn_chunk_prefill_onchip(q, k, v, lg, bt, h0, chunk=p.chunk)
    torch.cuda.synchronize()
    o, hT = host(o), host(hT)
    say("  oracle (all 48 heads)")
    o_ref, h_ref = run_oracle(inp)
    assert_parity(o, o_ref, hT, h_ref, "bf16", f"{p.name} {entry}")
    m = margins(o, o_ref, hT, h_ref, f"{p.name} {entry}")
    assert m["o"] <= BF16_REL and m["hT"] <= BF16_REL


@pytest.mark.timeout(400)
def test_qwen27b_decode_1000_steps_every_head():
    """B=64, 16/48 heads, d=128, 1000 steps of the benchmark's inputs on one
    state updated in place: every step's output and the final state of every
    (sequence, head) against the oracle.  The oracle runs the 1000 steps as
    one token-serial sequence per (sequence, head), which is what consecutive
    decode steps compute."""
    torch = torch_mod()
    p = gi.QWEN27B_DECODE
    say(f"{p.name}: generating {p.steps} steps")
    state0 = gi.make_decode_state(p, 0)
    st = gi.make_decode_steps(p, 0, steps=p.steps)
    dv = {n: (dev(st[n], "bf16") if n in ("q", "k", "v") else dev32(st[n])) for n in st}
    state = dev32(state0)
    outs = torch.empty((p.steps, p.B, p.Hv, p.dv), dtype=torch.bfloat16, device="cuda")
    for s in range(p.steps):
        gdn.gdn_decode_step(dv["q"][s], dv["k"][s], dv["v"][s], dv["log_g"][s], dv["beta"][s],
                            state, out=outs[s])
    torch.cuda.synchronize()
    del dv
    say("  oracle: 1000 tokens per (sequence, head), all 3072")
    seq = {n: np.ascontiguousarray(np.swapaxes(st[n], 0, 1)) for n in st}   # [B, steps, ...]
    o_ref, h_ref = oracle.gdn_sequential(seq["q"], seq["k"], seq["v"], seq["log_g"], seq["beta"],
                                         state0, nthreads=NTHREADS)
    del seq
    worst = 0.0
    for w0 in range(0, p.steps, 100):
        o_w = host(outs[w0:w0 + 100])                        # [w, B, Hv, dv]
        r_w = np.swapaxes(o_ref[:, w0:w0 + 100], 0, 1)       # [w, B, Hv, dv]
        w = per_head_rel(o_w, r_w, (1, 2))
        worst = max(worst, w)
        if w0 in (0, 500, 900):
            say(f"  steps {w0}..{w0 + 100}: worst per-(b,h) rel o {w:.3e}")
    h_gpu = host(state)
    m = margins(None, None, h_gpu, h_ref, f"{p.name} final state")
    say(f"  after {p.steps} steps: worst per-(b,h) rel o over all steps {worst:.3e}")
    assert worst <= BF16_REL and m["hT"] <= BF16_REL
    assert metrics(h_gpu, h_ref)["rel_fro"] <= BF16_REL


def test_qwen27b_decode_b128_state_past_the_cache():
    """B=128, 16/48 heads, d=128: 403 MB of state, more than the 256 MB Infinity
    Cache; two steps checked on every head."""
    torch = torch_mod()
    p = gi.DecodeProblem("qwen27b_decode_B128_Hk16_Hv48_d128", 128, 16, 48, 128, 128, 2)
    say("decode B=128 (state past the Infinity Cache)")
    state0 = gi.make_decode_state(p, 3)
    state = dev32(state0)
    steps = gi.make_decode_steps(p, 3)
    outs = []
    for s in range(p.steps):
        outs.append(host(gdn.gdn_decode_step(*(dev(steps[n][s], "bf16") for n in ("q", "k", "v")),
                                             dev32(steps["log_g"][s]), dev32(steps["beta"][s]), state)))
    torch.cuda.synchronize()
    h = state0
    for s in range(p.steps):
        o_r, h = oracle.gdn_sequential(*(steps[n][s][:, None] for n in ("q", "k", "v", "log_g", "beta")),
                                       h, nthreads=NTHREADS)
        m = metrics(outs[s], o_r[:, 0])
        say(f"  step {s}: o {m}")
        assert m["rel_fro"] <= BF16_REL
        assert per_head_rel(outs[s], o_r[:, 0], (0, 1)) <= BF16_REL
    h_gpu = host(state)
    mh = metrics(h_gpu, h)
    say(f"  state: {mh}")
    assert mh["rel_fro"] <= BF16_REL and per_head_rel(h_gpu, h, (0, 1)) <= BF16_REL
    margins(outs[-1], o_r[:, 0], h_gpu, h, "decode B=128 step 2", o_heads=(0, 1))


@pytest.mark.timeout(400)
def test_qwen27b_long_context_512_token_calls():
    """131072 tokens as 256 calls of 512 carrying the fp32 state through a
    bank that keeps it at every call boundary: outputs and final state bitwise
    equal to one call; every checkpoint and every output of every head
    against the oracle's single pass."""
    torch = torch_mod()
    p = gi.QWEN27B_LONG
    Tc = p.extra["call_tokens"]
    calls = p.T // Tc
    segs_dev = []
    bank = torch.empty((calls, p.B, p.Hv, p.dk, p.dv), dtype=torch.float32, device="cuda")
    say(f"{p.name}: {calls} calls")
    outs = []
    for c in range(calls):
        seg = gi.make_long_segment(p, 0, c)
        d = {n: (dev(seg[n], "bf16") if n in ("q", "k", "v") else dev32(seg[n]))
             for n in ("q", "k", "v", "log_g", "beta")}
        segs_dev.append(d)
        o_c, _ = gdn.gdn_chunk_prefill(d["q"], d["k"], d["v"], d["log_g"], d["beta"],
                                       bank[c - 1] if c else None, chunk=p.chunk, hT=bank[c])
        outs.append(o_c)
    torch.cuda.synchronize()
    say("  single call")
    cat = {n: torch.cat([s[n] for s in segs_dev], dim=1) for n in segs_dev[0]}
    del segs_dev
    o_one, h_one = gdn.gdn_chunk_prefill(cat["q"], cat["k"], cat["v"], cat["log_g"], cat["beta"],
                                         None, chunk=p.chunk)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=1), o_one)
    assert torch.equal(bank[-1], h_one)
    del cat, o_one
    say("  oracle, all 48 heads, every call")
    h_ref = None
    worst_h = 0.0
    worst_o = 0.0
    for c in range(calls):
        seg = gi.make_long_segment(p, 0, c)
        o_ref, h_ref = oracle.gdn_sequential(seg["q"], seg["k"], seg["v"], seg["log_g"],
                                             seg["beta"], h_ref, nthreads=NTHREADS)
        worst_h = max(worst_h, per_head_rel(host(bank[c]), h_ref, (0, 1)))
        worst_o = max(worst_o, per_head_rel(host(outs[c]), o_ref, (0, 2)))
        if c % 64 == 0 or c == calls - 1:
            say(f"  call {c}: worst so far o {worst_o:.3e}, checkpoint {worst_h:.3e}")
    say(f"  margins {p.name}: worst per-(b,h) rel o {worst_o:.3e}, checkpoints {worst_h:.3e} "
        f"(bar {BF16_REL:.0e})")
    assert worst_h <= BF16_REL and worst_o <= BF16_REL
