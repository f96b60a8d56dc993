"""gdn_chunk_prefill_noalloc: gdn_chunk_prefill with the library's fixed
per-device workspace array, called through the C ABI.  Its outputs must be
bitwise those of gdn_chunk_prefill (the same kernels, the same launch) on
calls in a row of different sizes, the array keeping the previous call's
contents; sizes beyond the array are refused before anything runs."""
import ctypes

import pytest

from gpu_common import dev, dev32, say, torch_mod
from linear_attention_recurrence_04_amd import binding as gdn
from linear_attention_recurrence_04_amd import inputs as gi

pytestmark = pytest.mark.gpu

MAX_WS = 64 << 20
REC = 13568            # workspace bytes per (sequence, value head, chunk)


def noalloc_call(prob, q, k, v, lg, bt, h0, hT, out):
    torch = torch_mod()
    st = gdn.lib().gdn_chunk_prefill_noalloc(
        ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(), lg.data_ptr(),
        bt.data_ptr(), h0.data_ptr() if h0 is not None else None, hT.data_ptr(), out.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    return st


def case(B, T, Hk, Hv, seed):
    inp = gi.custom_prefill(B, T, Hk, Hv, 128, 128, seed=seed, dtype="bf16", gate="qwen", h0="normal")
    return (dev(inp["q"], "bf16"), dev(inp["k"], "bf16"), dev(inp["v"], "bf16"),
            dev32(inp["log_g"]), dev32(inp["beta"]), dev32(inp["h0"]))


def test_noalloc_array_size_is_as_documented():
    assert gdn.gdn_chunk_prefill_noalloc_max_workspace() == MAX_WS


def test_noalloc_matches_prefill_on_calls_in_a_row():
    """A 27B-shaped call longer than the array holds in one piece (B=1,
    20,000 tokens, 16/48 heads: pieces of 98 chunks), then a smaller ragged
    call (one piece), then 35 sequences of 650 tokens over 4/20 heads (B * Hv
    = 700: pieces of 2 chunks), then the long one again: each bitwise equal
    to gdn_chunk_prefill on the same inputs (pieces of 256 chunks)."""
    torch = torch_mod()
    shapes = [(1, 20000, 16, 48, 1), (2, 1100, 2, 6, 2), (35, 650, 4, 20, 5), (1, 20000, 16, 48, 3)]
    for (B, T, Hk, Hv, seed) in shapes:
        say(f"noalloc B={B} T={T} {Hk}x{Hv} seed={seed}")
        prob = gdn.make_problem(B, T, Hk, Hv, 128, 128)
        chunks = -(-T // 64)
        one_piece = B * Hv * chunks * REC
        assert (one_piece > MAX_WS) == (T != 1100)
        assert B * Hv * REC + (B * Hv * 65536 if chunks > 1 else 0) <= MAX_WS
        q, k, v, lg, bt, h0 = case(B, T, Hk, Hv, seed)
        out = torch.full((B, T, Hv, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        hT = torch.full((B, Hv, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
        assert noalloc_call(prob, q, k, v, lg, bt, h0, hT, out) == 0
        o_ref, h_ref = gdn.gdn_chunk_prefill(q, k, v, lg, bt, h0)
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref), (B, T, Hk, Hv)
        assert torch.equal(hT, h_ref), (B, T, Hk, Hv)
        del q, k, v, lg, bt, h0, out, hT, o_ref, h_ref


def test_noalloc_refuses_beyond_the_array():
    """One chunk's records and the carried state do not fit (B * Hv = 864):
    GDN_ERR_WORKSPACE, nothing enqueued (the pointers are never used)."""
    prob = gdn.make_problem(18, 6593, 16, 48, 128, 128)
    assert 18 * 48 * (REC + 65536) > MAX_WS
    fake = 1 << 20
    st = gdn.lib().gdn_chunk_prefill_noalloc(ctypes.byref(prob), fake, fake, fake, fake, fake,
                                             None, fake, fake, None)
    assert st == 5


def test_noalloc_in_a_graph():
    """Captured in a HIP graph and replayed three times with eager work in
    between: bitwise the eager gdn_chunk_prefill result every time."""
    torch = torch_mod()
    B, T, Hk, Hv = 1, 777, 2, 6
    prob = gdn.make_problem(B, T, Hk, Hv, 128, 128)
    q, k, v, lg, bt, h0 = case(B, T, Hk, Hv, 4)
    out = torch.empty((B, T, Hv, 128), dtype=torch.bfloat16, device="cuda")
    hT = torch.empty((B, Hv, 128, 128), dtype=torch.float32, device="cuda")
    o_ref, h_ref = gdn.gdn_chunk_prefill(q, k, v, lg, bt, h0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert noalloc_call(prob, q, k, v, lg, bt, h0, hT, out) == 0
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert noalloc_call(prob, q, k, v, lg, bt, h0, hT, out) == 0
    for rep in range(3):
        out.zero_()
        hT.zero_()
        # other work on the array between replays: a smaller call of its own
        q2, k2, v2, lg2, bt2, h02 = case(1, 300, 1, 3, 10 + rep)
        gdn.gdn_chunk_prefill_noalloc(q2, k2, v2, lg2, bt2, h02)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref) and torch.equal(hT, h_ref), rep
