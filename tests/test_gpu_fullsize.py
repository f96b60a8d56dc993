"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.  Where the fp64 oracle cannot cover every head in seconds,
whole key-head groups (or sampled sequences) are checked one by one."""
import numpy as np
import pytest

import oracle
from gpu_common import (BF16_REL, NTHREADS, assert_parity, dev, dev32, host, metrics,
                        per_head_rel, run_oracle, run_prefill, say, torch_mod)
from linear_attention_recurrence_04_amd import binding as gdn
from linear_attention_recurrence_04_amd import inputs as gi

pytestmark = pytest.mark.gpu


def _group_slice(inp, hk, r):
    """Inputs of key head hk and its r value heads, as a 1:r problem."""
    hs = slice(hk * r, (hk + 1) * r)
    return {"q": inp["q"][:, :, hk:hk + 1], "k": inp["k"][:, :, hk:hk + 1],
            "v": inp["v"][:, :, hs], "log_g": inp["log_g"][:, :, hs],
            "beta": inp["beta"][:, :, hs],
            "h0": None if inp["h0"] is None else inp["h0"][:, hs]}


def test_qwen08b_prefill_full():
    """B=1, T=2048, 16/16 heads, d=128, bf16, chunk 64, h0 ~ N(0, 0.02): every head."""
    p = gi.QWEN08B_PREFILL
    say(f"{p.name}: generating")
    inp = gi.make_prefill(p, 0)
    o, hT = run_prefill(inp, "bf16", p.chunk)
    say("  oracle (all heads)")
    o_ref, h_ref = run_oracle(inp)
    assert_parity(host(o), o_ref, host(hT), h_ref, "bf16", p.name)


def test_qwen27b_prefill_full_sampled_groups():
    """B=1, T=16384, 16 key / 48 value heads, d=128, bf16: whole run on the GPU,
    key-head groups 7 and 15 (value heads 21-23, 45-47) checked against the oracle."""
    p = gi.QWEN27B_PREFILL
    say(f"{p.name}: generating")
    inp = gi.make_prefill(p, 0)
    o, hT = run_prefill(inp, "bf16", p.chunk)
    o, hT = host(o), host(hT)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(hT))
    r = p.Hv // p.Hk
    for hk in (7, 15):
        say(f"  oracle key head {hk}")
        sub = _group_slice(inp, hk, r)
        o_ref, h_ref = oracle.gdn_sequential(sub["q"], sub["k"], sub["v"], sub["log_g"],
                                             sub["beta"], sub["h0"], nthreads=r)
        hs = slice(hk * r, (hk + 1) * r)
        assert_parity(o[:, :, hs], o_ref, hT[:, hs], h_ref, "bf16", f"{p.name} group {hk}")


def test_qwen27b_decode_full_state_then_long_run():
    """B=64, 16/48 heads, d=128: 4 steps checked on every head, then 1000 steps
    checked on sampled (sequence, head) pairs (error must not grow)."""
    torch = torch_mod()
    p = gi.QWEN27B_DECODE
    state0 = gi.make_decode_state(p, 0)
    state = dev32(state0)
    first = gi.make_decode_steps(p, 0, steps=4)
    outs = []
    for s in range(4):
        outs.append(host(gdn.gdn_decode_step(*(dev(first[n][s], "bf16") for n in ("q", "k", "v")),
                                             dev32(first["log_g"][s]), dev32(first["beta"][s]), state)))
    torch.cuda.synchronize()
    h = state0
    for s in range(4):
        o_r, h = oracle.gdn_sequential(*(first[n][s][:, None] for n in ("q", "k", "v", "log_g", "beta")),
                                       h, nthreads=NTHREADS)
        m = metrics(outs[s], o_r[:, 0])
        say(f"  step {s}: o {m}")
        assert m["rel_fro"] <= BF16_REL
        assert per_head_rel(outs[s], o_r[:, 0], (0, 1)) <= BF16_REL
    mh = metrics(host(state), h)
    say(f"  state after 4 steps: {mh}")
    assert mh["rel_fro"] <= BF16_REL and per_head_rel(host(state), h, (0, 1)) <= BF16_REL

    # continue to 1000 steps; the oracle follows sampled sequences and heads
    seqs = [0, 37, 63]
    heads = [0, 1, 2, 23, 47]
    hk_of = [hh // (p.Hv // p.Hk) for hh in heads]
    h_s = h[np.ix_(seqs, heads)]
    worst = 0.0
    window = 100
    for w0 in range(4, p.steps, window):
        n = min(window, p.steps - w0)
        st = gi.make_decode_steps(p, 0, steps=n, first_step=w0)
        for s in range(n):
            o_d = gdn.gdn_decode_step(*(dev(st[x][s], "bf16") for x in ("q", "k", "v")),
                                      dev32(st["log_g"][s]), dev32(st["beta"][s]), state)
            # oracle: each sampled (seq, head) as its own 1:1 problem
            q = st["q"][s][np.ix_(seqs, hk_of)][:, None]
            k = st["k"][s][np.ix_(seqs, hk_of)][:, None]
            v = st["v"][s][np.ix_(seqs, heads)][:, None]
            lg = st["log_g"][s][np.ix_(seqs, heads)][:, None]
            bt = st["beta"][s][np.ix_(seqs, heads)][:, None]
            o_r = np.empty((len(seqs), len(heads), p.dv))
            for j in range(len(heads)):
                oj, hj = oracle.gdn_sequential(q[:, :, j:j + 1], k[:, :, j:j + 1], v[:, :, j:j + 1],
                                               lg[:, :, j:j + 1], bt[:, :, j:j + 1], h_s[:, j:j + 1])
                o_r[:, j] = oj[:, 0, 0]
                h_s[:, j] = hj[:, 0]
            o_g = host(o_d)[np.ix_(seqs, heads)]
            worst = max(worst, per_head_rel(o_g, o_r, (0, 1)))
        say(f"  steps {w0}..{w0 + n}: worst per-head rel o = {worst:.3e}")
    torch.cuda.synchronize()
    s_g = host(state)[np.ix_(seqs, heads)]
    rel_state = per_head_rel(s_g, h_s, (0, 1))
    say(f"  after {p.steps} steps: worst o {worst:.3e}, worst state {rel_state:.3e}")
    assert worst <= BF16_REL and rel_state <= BF16_REL



def test_qwen27b_decode_b128_state_past_the_cache():
    """B=128, 16/48 heads, d=128: 403 MB of state, more than the 256 MB Infinity
    Cache, so a single step runs the 1024-thread form of the decode kernel;
    two steps checked on every head."""
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

def test_qwen27b_long_context_512_token_calls():
    """131072 tokens as 256 calls of 512 carrying the fp32 state: outputs and
    final state bitwise equal to one call; every checkpoint of key-head group 5
    matches the oracle's single pass."""
    torch = torch_mod()
    p = gi.QWEN27B_LONG
    Tc = p.extra["call_tokens"]
    calls = p.T // Tc
    r = p.Hv // p.Hk
    hk = 5
    hs = slice(hk * r, (hk + 1) * r)
    segs_dev = []
    ckpts = []
    h = None
    say(f"{p.name}: {calls} calls")
    outs = []
    for c in range(calls):
        seg = gi.make_long_segment(p, 0, c)
        d = {n: (dev(seg[n], "bf16") if n in ("q", "k", "v") else dev32(seg[n]))
             for n in ("q", "k", "v", "log_g", "beta")}
        segs_dev.append(d)
        o_c, h = gdn.gdn_chunk_prefill(d["q"], d["k"], d["v"], d["log_g"], d["beta"], h, chunk=p.chunk)
        outs.append(o_c)
        ckpts.append(h[:, hs].clone())
    torch.cuda.synchronize()
    say("  single call")
    cat = {n: torch.cat([s[n] for s in segs_dev], dim=1) for n in segs_dev[0]}
    o_one, h_one = gdn.gdn_chunk_prefill(cat["q"], cat["k"], cat["v"], cat["log_g"], cat["beta"],
                                         None, chunk=p.chunk)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=1), o_one)
    assert torch.equal(h, h_one)
    del cat, o_one
    say("  oracle checkpoints, key head 5")
    h_ref = None
    worst_h = 0.0
    worst_o = 0.0
    for c in range(calls):
        seg = gi.make_long_segment(p, 0, c)
        sub = _group_slice(seg, hk, r)
        o_ref, h_ref = oracle.gdn_sequential(sub["q"], sub["k"], sub["v"], sub["log_g"], sub["beta"],
                                             h_ref, nthreads=r)
        worst_h = max(worst_h, per_head_rel(host(ckpts[c]), h_ref, (0, 1)))
        if c % 32 == 0 or c == calls - 1:
            worst_o = max(worst_o, per_head_rel(host(outs[c])[:, :, hs], o_ref, (0, 2)))
    say(f"  worst checkpoint rel {worst_h:.3e}, worst sampled o rel {worst_o:.3e}")
    assert worst_h <= BF16_REL and worst_o <= BF16_REL
