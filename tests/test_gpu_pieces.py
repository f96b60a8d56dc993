"""Long bf16 MFMA prefill calls run in pieces of chunks that reuse one set of
workspace records (256 chunks with the documented workspace, longer with a
larger one; gdn_chunk_prefill_noalloc runs pieces as short as its array
requires, tested with the no-allocation entry point).  Every chunk computes
the same whatever the pieces, so a call must give bitwise the same outputs,
final state and checkpoints for every workspace size it accepts, and match
the oracle."""
import numpy as np
import pytest

import oracle
from gpu_common import NTHREADS, assert_parity, dev, dev32, host, margins, say, torch_mod
from linear_attention_recurrence_04_amd import binding as gdn
from linear_attention_recurrence_04_amd import inputs as gi

pytestmark = pytest.mark.gpu

REC = 13568        # workspace bytes per (sequence, value head, chunk)
CARRY = 65536      # bytes of one head's carried state


def ws_for_piece(B, Hv, chunks, piece):
    """Workspace that runs a call of `chunks` chunks in pieces of `piece`."""
    torch = torch_mod()
    if piece >= chunks:
        n = B * Hv * chunks * REC
    else:
        n = ((B * Hv * piece * REC + 255) // 256) * 256 + B * Hv * CARRY
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def tensors(inp):
    return ([dev(inp[n], "bf16") for n in ("q", "k", "v")]
            + [dev32(inp["log_g"]), dev32(inp["beta"]), dev32(inp["h0"])])


def test_long_call_bitwise_for_every_piece_length():
    """T = 40,000 (625 chunks), 2/6 heads: one piece, the documented 256 +
    256 + 113 and pieces of 300 give bitwise the same o and hT, with and
    without a final state, and match the oracle on every head."""
    torch = torch_mod()
    B, T, Hk, Hv = 1, 40000, 2, 6
    inp = gi.custom_prefill(B, T, Hk, Hv, 128, 128, seed=31, dtype="bf16", gate="qwen", h0="normal")
    q, k, v, lg, bt, h0 = tensors(inp)
    chunks = -(-T // 64)
    runs = {}
    for name, ws in [("one piece", ws_for_piece(B, Hv, chunks, chunks)), ("documented", None),
                     ("300", ws_for_piece(B, Hv, chunks, 300))]:
        say(f"pieces: {name}")
        runs[name] = gdn.gdn_chunk_prefill(q, k, v, lg, bt, h0, workspace=ws)
        o_ns, none = gdn.gdn_chunk_prefill(q, k, v, lg, bt, h0, workspace=ws, want_state=False)
        torch.cuda.synchronize()
        assert none is None and torch.equal(o_ns, runs[name][0]), name
    o1, h1 = runs["one piece"]
    for name, (o, h) in runs.items():
        assert torch.equal(o, o1) and torch.equal(h, h1), name
    say("  oracle, all 6 heads")
    o_ref, h_ref = oracle.gdn_sequential(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["beta"],
                                         inp["h0"], nthreads=NTHREADS)
    assert_parity(host(o1), o_ref, host(h1), h_ref, "bf16", "625 chunks in pieces")
    margins(host(o1), o_ref, host(h1), h_ref, "625 chunks in pieces")


def test_in_place_state_across_pieces():
    """hT == h0 (in-place carry) over two pieces (266 chunks) equals a separate hT."""
    torch = torch_mod()
    B, T, Hk, Hv = 2, 17000, 1, 3
    inp = gi.custom_prefill(B, T, Hk, Hv, 128, 128, seed=32, dtype="bf16", gate="qwen", h0="normal")
    q, k, v, lg, bt, h0 = tensors(inp)
    o_sep, h_sep = gdn.gdn_chunk_prefill(q, k, v, lg, bt, h0.clone())
    h = h0.clone()
    o_inp, h_inp = gdn.gdn_chunk_prefill(q, k, v, lg, bt, h, hT=h)
    torch.cuda.synchronize()
    assert h_inp.data_ptr() == h.data_ptr()
    assert torch.equal(o_sep, o_inp) and torch.equal(h_sep, h_inp)


def test_varlen_with_a_sequence_longer_than_a_piece():
    """Packed lengths 17,000 / 500 / 12,500 (the longest 266 chunks): the
    documented workspace (256 + 10 chunks) and one piece give bitwise the same
    results; the short sequences pass through the second piece unchanged."""
    torch = torch_mod()
    lengths = [17000, 500, 12500]
    Hk, Hv = 1, 3
    seqs = [gi.custom_prefill(1, L, Hk, Hv, 128, 128, seed=40 + i, dtype="bf16", gate="qwen",
                              h0="normal") for i, L in enumerate(lengths)]
    cat = {n: np.concatenate([s[n][0] for s in seqs], axis=0) for n in ("q", "k", "v", "log_g", "beta")}
    h0 = dev32(np.concatenate([s["h0"] for s in seqs], axis=0))
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)).cuda()
    q, k, v = (dev(cat[n], "bf16") for n in ("q", "k", "v"))
    lg, bt = dev32(cat["log_g"]), dev32(cat["beta"])
    chunks = -(-max(lengths) // 64)
    o1, h1 = gdn.gdn_chunk_prefill_varlen(q, k, v, lg, bt, cu, max(lengths), h0,
                                          workspace=ws_for_piece(3, Hv, chunks, chunks))
    o2, h2 = gdn.gdn_chunk_prefill_varlen(q, k, v, lg, bt, cu, max(lengths), h0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    # the 500-token sequence alone, bitwise
    s = seqs[1]
    o_s, h_s = gdn.gdn_chunk_prefill(*tensors(s))
    torch.cuda.synchronize()
    assert torch.equal(o2[17000:17500], o_s[0]) and torch.equal(h2[1], h_s[0])


@pytest.mark.parametrize("raw_gates", [False, True], ids=["gates", "raw_gates"])
def test_checkpoints_across_pieces(raw_gates):
    """A slot every 1,024 tokens over 17,000 tokens (slots on both sides of the
    piece boundary at chunk 256): bitwise the same for pieces of 256 chunks
    and for one piece, with given or raw gates."""
    torch = torch_mod()
    B, T, Hk, Hv = 1, 17000, 1, 3
    inp = gi.custom_prefill(B, T, Hk, Hv, 128, 128, seed=33, dtype="bf16", gate="qwen", h0="normal")
    q, k, v, lg, bt, h0 = tensors(inp)
    chunks = -(-T // 64)
    rng = np.random.default_rng(5)
    a_raw = dev32(rng.normal(0.0, 1.0, (B, T, Hv)).astype(np.float32))
    b_raw = dev32(rng.normal(0.0, 1.0, (B, T, Hv)).astype(np.float32))
    A_log = dev32(np.log(rng.uniform(1.0, 16.0, Hv)).astype(np.float32))
    dt_bias = dev32(rng.normal(0.0, 0.5, Hv).astype(np.float32))
    res = []
    for ws in (ws_for_piece(B, Hv, chunks, chunks), None):
        if raw_gates:
            res.append(gdn.gdn_chunk_prefill_gated(q, k, v, a_raw, b_raw, A_log, dt_bias, h0,
                                                   ckpt_every=1024, workspace=ws))
        else:
            res.append(gdn.gdn_chunk_prefill_ckpt(q, k, v, lg, bt, h0, ckpt_every=1024, workspace=ws))
    torch.cuda.synchronize()
    for r in res[1:]:
        for x, y in zip(r, res[0]):
            assert torch.equal(x, y)
    assert res[0][2].shape[1] == -(-T // 1024)
