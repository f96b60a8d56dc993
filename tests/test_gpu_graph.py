"""Library calls captured into a HIP graph (torch.cuda.graph) and replayed:
every replay, with eager work and synchronisation between replays, must give
bitwise the eager result.  Under capture the library enqueues only kernels
on the caller's stream (no allocation, no memset, no synchronisation), which
is what makes its calls capturable."""
import numpy as np
import pytest

from gpu_common import dev, dev32, say, torch_mod
from linear_attention_recurrence_04_amd import binding as gdn
from linear_attention_recurrence_04_amd import inputs as gi

pytestmark = pytest.mark.gpu


def test_decode_steps_in_a_graph():
    torch = torch_mod()
    d = gi.DecodeProblem("graph", 8, 2, 6, 128, 128, 6)
    st = gi.make_decode_steps(d, 3)
    dv = {n: torch.from_numpy(st[n]).cuda() for n in st}
    for n in ("q", "k", "v"):
        dv[n] = dv[n].to(torch.bfloat16)
    state0 = torch.from_numpy(gi.make_decode_state(d, 3)).cuda()
    state = state0.clone()
    out = torch.empty((d.steps, d.B, d.Hv, d.dv), dtype=torch.bfloat16, device="cuda")

    def steps():
        for s in range(d.steps):
            gdn.gdn_decode_step(dv["q"][s], dv["k"][s], dv["v"][s], dv["log_g"][s], dv["beta"][s],
                                state, out=out[s])

    steps()
    torch.cuda.synchronize()
    o_ref, s_ref = out.clone(), state.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        state.copy_(state0)
        steps()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps()
    for rep in range(3):
        state.copy_(state0)            # eager work between replays
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"  decode graph replay {rep}")
        assert torch.equal(out, o_ref) and torch.equal(state, s_ref), f"replay {rep}"


# T = 16400 is 257 chunks of 64, the last one ragged
@pytest.mark.parametrize("dtype,d,C,T", [("bf16", 128, 64, 200), ("f32", 64, 32, 200),
                                         ("bf16", 128, 64, 16400)])
def test_prefill_in_a_graph(dtype, d, C, T):
    torch = torch_mod()
    inp = gi.custom_prefill(1, T, 1, 3, d, d, seed=9, dtype=dtype, gate="qwen", h0="normal")
    q, k, v = dev(inp["q"], dtype), dev(inp["k"], dtype), dev(inp["v"], dtype)
    lg, bt, h0 = dev32(inp["log_g"]), dev32(inp["beta"]), dev32(inp["h0"])
    prob = gdn.make_problem(1, T, 1, 3, d, d, chunk=C,
                            dtype=gdn.GDN_DTYPE_BF16 if dtype == "bf16" else gdn.GDN_DTYPE_F32)
    ws = torch.empty(max(gdn.gdn_chunk_prefill_workspace_bytes(prob), 1), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty(tuple(v.shape), dtype=v.dtype, device="cuda")
    hT = torch.empty_like(h0)

    def call():
        gdn.gdn_chunk_prefill(q, k, v, lg, bt, h0, chunk=C, out=o, hT=hT, workspace=ws)

    call()
    torch.cuda.synchronize()
    o_ref, h_ref = o.clone(), hT.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        o.zero_()
        hT.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"  prefill graph replay {rep} ({dtype})")
        assert torch.equal(o, o_ref) and torch.equal(hT, h_ref), f"replay {rep}"
