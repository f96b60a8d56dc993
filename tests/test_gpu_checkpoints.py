"""GPU parity of gdn_chunk_prefill_ckpt: the state stored every ckpt_every tokens
of one prefill call (the GDN checkpoint slots of hybrid prefix caching).

Expected slots come from the oracle run segment by segment, each segment
starting from the previous one's final state; the oracle's splitting pin makes
that the state of one uninterrupted run at the segment's end.  On the GPU a
slot must also be bitwise the hT of a call that stops at its token."""
import numpy as np
import pytest

import oracle
from gpu_common import (BF16_REL, F32_MAX_ABS, NTHREADS, assert_parity, dev, dev32, host,
                        metrics, per_head_rel, run_prefill, say, torch_mod)
from linear_attention_recurrence_04_amd import binding as gdn
from linear_attention_recurrence_04_amd import inputs as gi

pytestmark = pytest.mark.gpu


def _segment(inp, a, b):
    return {n: (inp[n][:, a:b] if n != "h0" else None) for n in inp}


def oracle_slots(inp, every):
    """Oracle states after min((j+1) every, T) tokens, j = 0 .. ceil(T/every)-1."""
    T = inp["q"].shape[1]
    h = inp["h0"]
    slots = []
    for a in range(0, T, every):
        b = min(a + every, T)
        s = _segment(inp, a, b)
        _, h = oracle.gdn_sequential(s["q"], s["k"], s["v"], s["log_g"], s["beta"], h,
                                     nthreads=NTHREADS)
        slots.append(h)
    return np.stack(slots, axis=1) if slots else None


def run_ckpt(inp, dtype, chunk, every):
    torch = torch_mod()
    q, k, v = dev(inp["q"], dtype), dev(inp["k"], dtype), dev(inp["v"], dtype)
    lg, bt = dev32(inp["log_g"]), dev32(inp["beta"])
    h = None if inp["h0"] is None else dev32(inp["h0"])
    o, hT, ck = gdn.gdn_chunk_prefill_ckpt(q, k, v, lg, bt, h, ckpt_every=every, chunk=chunk)
    torch.cuda.synchronize()
    return o, hT, ck


def check_slots(ck_gpu, ck_ref, dtype, label):
    for j in range(ck_ref.shape[1]):
        g, r = ck_gpu[:, j], ck_ref[:, j]
        m = metrics(g, r)
        say(f"  slot {j} {label}: {m}")
        if dtype == "f32":
            assert m["max_abs"] <= F32_MAX_ABS, (label, j, m)
        else:
            assert m["rel_fro"] <= BF16_REL, (label, j, m)
            assert per_head_rel(g, r, (0, 1)) <= BF16_REL, (label, j)


CASES = [  # (B, T, Hk, Hv, d, chunk, dtype, every)
    (1, 100, 1, 2, 64, 16, "f32", 16),      # every chunk, ragged tail
    (2, 97, 2, 4, 64, 32, "f32", 64),       # two chunks per slot, partial last slot
    (1, 200, 1, 3, 128, 64, "bf16", 64),    # MFMA path, every chunk
    (2, 300, 2, 6, 128, 64, "bf16", 128),   # MFMA path, GQA, partial last slot
    (1, 129, 1, 3, 128, 32, "bf16", 96),    # generic bf16 path
    (1, 40, 1, 2, 128, 64, "bf16", 192),    # one slot, shorter than a chunk
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_T{c[1]}_{c[2]}x{c[3]}_d{c[4]}_C{c[5]}_"
                                             f"{c[6]}_every{c[7]}" for c in CASES])
def test_checkpoints_match_oracle_and_truncated_calls(case):
    torch = torch_mod()
    B, T, Hk, Hv, d, C, dtype, every = case
    say(f"checkpoints {case}")
    inp = gi.custom_prefill(B, T, Hk, Hv, d, d, seed=21, dtype=dtype, gate="qwen", h0="normal")
    o, hT, ck = run_ckpt(inp, dtype, C, every)
    nck = -(-T // every)
    assert ck.shape == (B, nck, Hv, d, d)
    # the checkpoints change nothing else: o and hT bitwise those of the plain call
    o_plain, h_plain = run_prefill(inp, dtype, C)
    assert torch.equal(o, o_plain) and torch.equal(hT, h_plain)
    # the last slot is hT
    assert torch.equal(ck[:, -1], hT)
    # each full slot is bitwise the hT of a call that stops at its token
    for j in range(nck):
        stop = min((j + 1) * every, T)
        sub = _segment(inp, 0, stop)
        sub["h0"] = inp["h0"]
        _, h_stop = run_prefill(sub, dtype, C)
        assert torch.equal(ck[:, j], h_stop), f"slot {j} differs from a call stopping at {stop}"
    check_slots(host(ck), oracle_slots(inp, every), dtype, str(case))


def test_checkpoint_edges():
    torch = torch_mod()
    # T == 0: no slots, hT = h0
    inp = gi.custom_prefill(1, 0, 1, 2, 64, 64, seed=2, dtype="f32", h0="normal")
    o, hT, ck = run_ckpt(inp, "f32", 32, 32)
    assert ck.shape == (1, 0, 2, 64, 64)
    assert torch.equal(hT.cpu(), torch.from_numpy(inp["h0"]))
    # no initial state, every = T exactly (one slot equal to hT)
    inp = gi.custom_prefill(1, 128, 1, 1, 128, 128, seed=3, dtype="bf16", gate="qwen", h0="zero")
    inp["h0"] = None
    o, hT, ck = run_ckpt(inp, "bf16", 64, 128)
    assert ck.shape[1] == 1 and torch.equal(ck[:, 0], hT)
    # a bad interval is refused by the library before anything runs
    with pytest.raises(gdn.GdnError) as e:
        run_ckpt(inp, "bf16", 64, 96)
    assert e.value.status == 2


def test_qwen27b_checkpoints_full_size():
    """The 27B prefill workload (B=1, T=16384, 16/48 heads, bf16, MFMA path) with a
    slot every 4096 tokens: o and hT unchanged, every slot bitwise the hT of a call
    stopping there, and every slot of every head against the oracle."""
    torch = torch_mod()
    p = gi.QWEN27B_PREFILL
    every = 4096
    say(f"{p.name}: checkpoints every {every}")
    inp = gi.make_prefill(p, 0)
    o, hT, ck = run_ckpt(inp, "bf16", p.chunk, every)
    o_plain, h_plain = run_prefill(inp, "bf16", p.chunk)
    assert torch.equal(o, o_plain) and torch.equal(hT, h_plain)
    del o_plain
    assert torch.equal(ck[:, -1], hT)
    for j in range(p.T // every - 1):
        stop = (j + 1) * every
        sub = _segment(inp, 0, stop)
        sub["h0"] = inp["h0"]
        _, h_stop = run_prefill(sub, "bf16", p.chunk)
        assert torch.equal(ck[:, j], h_stop), f"slot {j}"
    say("  oracle, all 48 heads, slot by slot")
    h_ref = inp["h0"]
    refs = []
    for j in range(p.T // every):
        seg = {n: inp[n][:, j * every:(j + 1) * every] for n in ("q", "k", "v", "log_g", "beta")}
        _, h_ref = oracle.gdn_sequential(seg["q"], seg["k"], seg["v"], seg["log_g"], seg["beta"],
                                         h_ref, nthreads=NTHREADS)
        refs.append(h_ref)
    check_slots(host(ck), np.stack(refs, axis=1), "bf16", f"{p.name} all slots")
    worst = max(per_head_rel(host(ck[:, j]), refs[j], (0, 1)) for j in range(len(refs)))
    say(f"  margins {p.name} checkpoints: worst per-(b,h) rel over {len(refs)} slots {worst:.3e}")
