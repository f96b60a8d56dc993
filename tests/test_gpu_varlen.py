"""GPU parity of gdn_chunk_prefill_varlen: a packed batch of sequences of
different lengths.  Each sequence must match the oracle run on it alone, and
bitwise the plain prefill call on it alone (same chunks, same order)."""
import numpy as np
import pytest

import oracle
from gpu_common import (margins, NTHREADS, assert_parity, dev, dev32, host, run_prefill, say, torch_mod)
from linear_attention_recurrence_04_amd import binding as gdn
from linear_attention_recurrence_04_amd import inputs as gi

pytestmark = pytest.mark.gpu


def packed(lengths, Hk, Hv, d, dtype, seed):
    """Per-sequence inputs (each with its own h0) and their packed concatenation."""
    seqs = [gi.custom_prefill(1, L, Hk, Hv, d, d, seed=seed + i, dtype=dtype, gate="qwen",
                              h0="normal") for i, L in enumerate(lengths)]
    cat = {n: np.concatenate([s[n][0] for s in seqs], axis=0) for n in ("q", "k", "v", "log_g", "beta")}
    h0 = np.concatenate([s["h0"] for s in seqs], axis=0)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return seqs, cat, h0, cu


def run_varlen(cat, h0, cu, dtype, chunk, max_len=None, total_extra=0, fill=None):
    torch = torch_mod()
    pad = lambda x: np.concatenate([x, np.zeros((total_extra,) + x.shape[1:], x.dtype)])  # noqa: E731
    q, k, v = (dev(pad(cat[n]), dtype) for n in ("q", "k", "v"))
    lg, bt = dev32(pad(cat["log_g"])), dev32(pad(cat["beta"]))
    out = None
    if fill is not None:
        out = torch.full(tuple(v.shape), fill, dtype=v.dtype, device="cuda")
    o, hT = gdn.gdn_chunk_prefill_varlen(q, k, v, lg, bt, torch.from_numpy(cu).cuda(), max_len,
                                         None if h0 is None else dev32(h0), chunk=chunk, out=out)
    torch.cuda.synchronize()
    return o, hT


CASES = [  # (lengths, Hk, Hv, d, chunk, dtype)
    ([130, 1, 64, 0, 257], 1, 3, 128, 64, "bf16"),     # MFMA path, empty and 1-token sequences
    ([64, 128, 192], 2, 6, 128, 64, "bf16"),           # MFMA path, whole chunks only
    ([50, 33, 97, 2], 2, 4, 64, 32, "f32"),            # generic fp32
    ([100, 7, 129], 1, 2, 128, 32, "bf16"),            # generic bf16
]


@pytest.mark.parametrize("case", CASES, ids=[f"{'-'.join(map(str, c[0]))}_{c[1]}x{c[2]}_d{c[3]}_C{c[4]}_{c[5]}"
                                             for c in CASES])
def test_varlen_matches_single_calls_and_oracle(case):
    torch = torch_mod()
    lengths, Hk, Hv, d, C, dtype = case
    say(f"varlen {case}")
    seqs, cat, h0, cu = packed(lengths, Hk, Hv, d, dtype, seed=60)
    o, hT = run_varlen(cat, h0, cu, dtype, C)
    for i, s in enumerate(seqs):
        a, b = int(cu[i]), int(cu[i + 1])
        o1, h1 = run_prefill(s, dtype, C)
        assert torch.equal(o[a:b], o1[0]), f"sequence {i}: o differs from its own call"
        assert torch.equal(hT[i], h1[0]), f"sequence {i}: hT differs from its own call"
        o_ref, h_ref = oracle.gdn_sequential(s["q"], s["k"], s["v"], s["log_g"], s["beta"],
                                             s["h0"], nthreads=NTHREADS)
        if lengths[i] == 0:
            assert np.array_equal(host(hT[i]), s["h0"][0].astype(np.float64))
            continue
        assert_parity(host(o[a:b])[None], o_ref, host(hT[i])[None], h_ref, dtype,
                      f"varlen sequence {i} (length {lengths[i]})")


def test_varlen_edges():
    torch = torch_mod()
    # rows past the last sequence are left as they were; a launch sized for a
    # longer maximum than any sequence changes nothing
    seqs, cat, h0, cu = packed([70, 20], 1, 2, 128, "bf16", seed=70)
    o, hT = run_varlen(cat, h0, cu, "bf16", 64, max_len=300, total_extra=9, fill=7.0)
    assert torch.all(o[90:] == 7.0)
    o2, h2 = run_varlen(cat, h0, cu, "bf16", 64)
    assert torch.equal(o[:90], o2) and torch.equal(hT, h2)
    # no initial states; all sequences empty (hT = 0)
    o3, h3 = run_varlen(cat, None, np.zeros(3, np.int32), "bf16", 64, total_extra=0)
    assert torch.count_nonzero(h3).item() == 0
    # no sequences at all
    o4, h4 = run_varlen(cat, None, np.zeros(1, np.int32), "bf16", 64)
    assert h4.shape[0] == 0


def test_qwen27b_varlen_mix_full_size():
    """A continuous-batching mix at the 27B head shape: 8 sequences totalling
    16384 tokens; every sequence bitwise its own call, and every sequence
    and head against the oracle."""
    torch = torch_mod()
    p = gi.QWEN27B_PREFILL
    lengths = [4096, 3000, 2500, 2048, 1800, 1500, 900, 540]
    assert sum(lengths) == p.T
    say(f"varlen 27B mix {lengths}")
    seqs = [gi.make_prefill(p, 100 + i, T=L) for i, L in enumerate(lengths)]
    cat = {n: np.concatenate([s[n][0] for s in seqs], axis=0) for n in ("q", "k", "v", "log_g", "beta")}
    h0 = np.concatenate([s["h0"] for s in seqs], axis=0)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    o, hT = run_varlen(cat, h0, cu, "bf16", p.chunk)
    for i, s in enumerate(seqs):
        a, b = int(cu[i]), int(cu[i + 1])
        o1, h1 = run_prefill(s, "bf16", p.chunk)
        assert torch.equal(o[a:b], o1[0]) and torch.equal(hT[i], h1[0]), f"sequence {i}"
    worst = {"o": 0.0, "hT": 0.0}
    for i, s in enumerate(seqs):
        o_ref, h_ref = oracle.gdn_sequential(s["q"], s["k"], s["v"], s["log_g"], s["beta"],
                                             s["h0"], nthreads=NTHREADS)
        a, b = int(cu[i]), int(cu[i + 1])
        og, hg = host(o[a:b])[None], host(hT[i])[None]
        assert_parity(og, o_ref, hg, h_ref, "bf16", f"27B varlen sequence {i}")
        m = margins(og, o_ref, hg, h_ref, f"27B varlen sequence {i} (T={lengths[i]})")
        worst = {x: max(worst[x], m[x]) for x in worst}
    say(f"  margins 27B varlen mix: worst per-(b,h) rel o {worst['o']:.3e}, hT {worst['hT']:.3e}")
