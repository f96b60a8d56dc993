"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments before touching the GPU (no compute calls here)."""
import ctypes
import glob
import os
import re

import pytest

from linear_attention_recurrence_04_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    assert {os.path.basename(h) for h in HEADERS} >= {"gdn.h", "gdn_calib.h"}
    for n in ("gdn_chunk_prefill", "gdn_decode_step", "gdn_chunk_prefill_workspace_bytes",
              "gdn_status_string", "gdn_abi_version", "gdn_calib_copy", "gdn_calib_mfma_loop"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIBRARY)
    for name in declared_functions():
        assert hasattr(lib, name), f"libgdn.so does not export {name}"


def test_version_and_status_strings():
    assert B.gdn_abi_version() == 1
    for s in range(8):
        assert B.gdn_status_string(s)
    assert "unknown" in B.gdn_status_string(99)


# Fake, 16-byte-aligned, non-overlapping "device" addresses: the library must
# reject the call during validation, before any HIP call.
BASE = 1 << 40


def fake(i, off=0):
    return BASE + i * (1 << 34) + off


def prefill(prob, q=fake(0), k=fake(1), v=fake(2), lg=fake(3), bt=fake(4), h0=None, hT=fake(6),
            o=fake(7), ws=None, wsb=0):
    return B.lib().gdn_chunk_prefill(ctypes.byref(prob), q, k, v, lg, bt, h0, hT, o, ws, wsb, None)


def decode(prob, q=fake(0), k=fake(1), v=fake(2), lg=fake(3), bt=fake(4), st=fake(5), o=fake(7)):
    return B.lib().gdn_decode_step(ctypes.byref(prob), q, k, v, lg, bt, st, o, None)


def P(**kw):
    base = dict(B=1, T=128, Hk=2, Hv=2, dk=64, dv=64, chunk=32, dtype=0)
    base.update(kw)
    return B.make_problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), 2), (dict(T=-1), 2), (dict(Hk=0), 2), (dict(Hv=3, Hk=2), 2),
    (dict(dk=64, dv=128), 3), (dict(dk=96, dv=96), 3), (dict(dk=256, dv=256), 3),
    (dict(chunk=48), 3), (dict(chunk=128), 3), (dict(dtype=2), 3),
])
def test_prefill_rejects_bad_problem(kw, status):
    assert prefill(P(**kw)) == status


def test_prefill_rejects_null_and_misaligned_and_alias():
    assert B.lib().gdn_chunk_prefill(None, fake(0), fake(1), fake(2), fake(3), fake(4), None,
                                     fake(6), fake(7), None, 0, None) == 1
    assert prefill(P(), q=None) == 1
    assert prefill(P(), o=None) == 1
    assert prefill(P(), lg=None) == 1
    assert prefill(P(), k=fake(1, 8)) == 4
    assert prefill(P(), hT=fake(6, 4)) == 4
    assert prefill(P(), o=fake(0, 256)) == 7           # o overlaps q
    assert prefill(P(), hT=fake(2, 1024)) == 7         # hT overlaps v
    assert prefill(P(), h0=fake(6), hT=fake(6, 64)) == 7   # partial h0/hT overlap
    assert prefill(P(), o=fake(6), hT=fake(6)) == 7    # o overlaps hT


def test_decode_rejects_bad_arguments():
    assert decode(P(T=2)) == 2
    assert decode(P(T=0)) == 2
    assert decode(P(T=1, dk=32, dv=32)) == 3
    assert decode(P(T=1), st=None) == 1
    assert decode(P(T=1), st=fake(5, 4)) == 4
    assert decode(P(T=1), o=fake(5, 512)) == 7         # o inside the state
    assert decode(P(T=1), st=fake(2)) == 7             # state over v


def test_workspace_query():
    assert B.gdn_chunk_prefill_workspace_bytes(P()) == 0
    assert B.gdn_chunk_prefill_workspace_bytes(P(Hv=3)) == 0   # invalid -> 0 as documented


@pytest.mark.parametrize("Bn,T,Hk,Hv", [(1, 1, 1, 1), (2, 200, 1, 3), (1, 768, 16, 48),
                                        (1, 769, 16, 48), (1, 16384, 16, 48), (1, 16385, 16, 48),
                                        (3, 16400, 2, 6), (1, 131072, 16, 48)])
def test_mfma_workspace_bytes_as_documented(Bn, T, Hk, Hv):
    """bf16, d = 128, chunk 64 takes the MFMA path, whose workspace is 13568
    bytes per (sequence, value head, chunk of 64) for up to 256 chunks; a
    longer call runs in pieces of 256 chunks and also holds the carried
    state (65536 bytes per head) at the next multiple of 256 bytes."""
    prob = P(B=Bn, T=T, Hk=Hk, Hv=Hv, dk=128, dv=128, chunk=64, dtype=1)
    assert B.gdn_chunk_prefill_variant(prob) == "mfma_bf16"
    chunks = -(-T // 64)
    want = (Bn * Hv * chunks * 13568 if chunks <= 256
            else ((Bn * Hv * 256 * 13568 + 255) // 256) * 256 + Bn * Hv * 65536)
    assert B.gdn_chunk_prefill_workspace_bytes(prob) == want


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 64)
    with pytest.raises(ValueError):
        B.gdn_chunk_prefill(x, x, x, torch.zeros(1, 4, 1), torch.zeros(1, 4, 1))


def prefill_ckpt(prob, every, ck=fake(8), q=fake(0), k=fake(1), v=fake(2), lg=fake(3),
                 bt=fake(4), h0=None, hT=fake(6), o=fake(7)):
    return B.lib().gdn_chunk_prefill_ckpt(ctypes.byref(prob), q, k, v, lg, bt, h0, hT, o, ck,
                                          every, None, 0, None)


def test_checkpointed_prefill_rejects_bad_arguments():
    # ckpt_every must be a positive multiple of the chunk in use (chunk 0 means 64)
    assert prefill_ckpt(P(), 0) == 2
    assert prefill_ckpt(P(), -32) == 2
    assert prefill_ckpt(P(), 48) == 2                  # chunk 32
    assert prefill_ckpt(P(chunk=0), 32) == 2           # chunk 64
    assert prefill_ckpt(P(Hv=3), 64) == 2              # the problem is checked first
    assert prefill_ckpt(P(), 64, ck=None) == 1         # T > 0 needs the slots
    assert prefill_ckpt(P(), 64, ck=fake(8, 4)) == 4
    assert prefill_ckpt(P(), 64, ck=fake(7, 512)) == 7      # slots inside o
    assert prefill_ckpt(P(), 64, ck=fake(6, 0)) == 7        # slots over hT
    assert prefill_ckpt(P(), 32, ck=fake(0, 4096)) == 7     # slots inside q
    # 4 slots of 1*2*64*64 fp32 = 131072 bytes: one byte short of hT's start
    # still overlaps; the call is then rejected before any launch
    assert prefill_ckpt(P(), 32, ck=fake(6, -131072 + 16)) == 7


def prefill_gated(prob, every=0, ck=None, A_log=fake(9), dt_bias=fake(10), o=fake(7), a=fake(3)):
    return B.lib().gdn_chunk_prefill_gated(ctypes.byref(prob), fake(0), fake(1), fake(2), a,
                                           fake(4), A_log, dt_bias, None, fake(6), o, ck, every,
                                           None, 0, None)


def decode_gated(prob, A_log=fake(9), dt_bias=fake(10), st=fake(5)):
    return B.lib().gdn_decode_step_gated(ctypes.byref(prob), fake(0), fake(1), fake(2), fake(3),
                                         fake(4), A_log, dt_bias, st, fake(7), None)


def test_gated_entry_points_reject_bad_arguments():
    assert prefill_gated(P(Hv=3)) == 2
    assert prefill_gated(P(), A_log=None) == 1
    assert prefill_gated(P(), dt_bias=None) == 1
    assert prefill_gated(P(), a=None) == 1
    assert prefill_gated(P(), every=-32) == 2
    assert prefill_gated(P(), every=48) == 2            # not a multiple of chunk 32
    assert prefill_gated(P(), every=0, ck=fake(8)) == 2  # slots without an interval
    assert prefill_gated(P(), every=32, ck=None) == 1
    assert prefill_gated(P(), A_log=fake(9, 4)) == 4
    assert prefill_gated(P(), A_log=fake(7, 64)) == 7   # gate parameters inside o
    assert prefill_gated(P(), o=fake(10)) == 7          # o over dt_bias
    assert decode_gated(P(T=1), A_log=None) == 1
    assert decode_gated(P(T=1), dt_bias=fake(10, 8)) == 4
    assert decode_gated(P(T=1), st=fake(9)) == 7        # state over A_log
    assert decode_gated(P(T=2)) == 2


def decode_multi(prob, A_log=None, dt_bias=None, st=fake(5), sts=None, o=fake(7)):
    return B.lib().gdn_decode_multi(ctypes.byref(prob), fake(0), fake(1), fake(2), fake(3),
                                    fake(4), A_log, dt_bias, st, o, sts, None)


def test_multi_token_decode_rejects_bad_arguments():
    assert decode_multi(P(T=-1)) == 2
    assert decode_multi(P(Hv=3)) == 2
    assert decode_multi(P(T=4), A_log=fake(9)) == 1     # A_log without dt_bias
    assert decode_multi(P(T=4), st=None) == 1
    assert decode_multi(P(T=4), sts=fake(8, 8)) == 4
    assert decode_multi(P(T=4), sts=fake(5, 4096)) == 7  # per-token states over the state
    assert decode_multi(P(T=4), o=fake(8), sts=fake(8)) == 7
    assert decode_multi(P(T=4, dk=32, dv=32)) == 3
    # the chunk field is ignored by decode
    assert decode_multi(P(T=4, chunk=48), st=None) == 1


def prefill_varlen(prob, cu=fake(11), total=300, q=fake(0), o=fake(7), hT=fake(6), h0=None):
    return B.lib().gdn_chunk_prefill_varlen(ctypes.byref(prob), cu, total, q, fake(1), fake(2),
                                            fake(3), fake(4), h0, hT, o, None, 0, None)


def test_varlen_prefill_rejects_bad_arguments():
    assert prefill_varlen(P(B=3, T=128), total=-1) == 2
    assert prefill_varlen(P(B=3, T=128), total=1 << 31) == 2
    assert prefill_varlen(P(B=3, T=128), cu=None) == 1
    assert prefill_varlen(P(B=3, T=128), cu=fake(11, 4)) == 4
    assert prefill_varlen(P(B=3, T=128), cu=fake(7, 64)) == 7     # offsets inside o
    assert prefill_varlen(P(B=3, T=128), q=None) == 1
    assert prefill_varlen(P(B=3, T=128, Hv=3)) == 2
    # o sized by total_tokens: an hT just past a 300-token o does not overlap it,
    # one starting inside it does (2 heads x 64 x 4 bytes per token)
    assert prefill_varlen(P(B=3, T=128), hT=fake(7, 300 * 2 * 64 * 4 - 16)) == 7


def onchip(prob, every=0, ck=None, q=fake(0), k=fake(1), v=fake(2), lg=fake(3), bt=fake(4),
           h0=None, hT=fake(6), o=fake(7)):
    return B.lib().gdn_chunk_prefill_onchip(ctypes.byref(prob), q, k, v, lg, bt, h0, hT, o, ck,
                                            every, None)


def test_onchip_prefill_rejects_bad_arguments():
    """The workspace-free prefill checks its arguments like the others: the
    checkpoint spacing, null and misaligned pointers, overlapping outputs."""
    assert onchip(P(), every=48) == 2                  # not a multiple of chunk 32
    assert onchip(P(), every=-32) == 2
    assert onchip(P(), every=0, ck=fake(8)) == 2       # slots without a spacing
    assert onchip(P(), every=32) == 1                  # spacing without slots
    assert onchip(P(), q=None) == 1
    assert onchip(P(), q=fake(0, 4)) == 4
    big = P(T=128, dk=128, dv=128, chunk=64, dtype=1)
    assert onchip(big, o=fake(0)) == 7                 # o over q
    assert onchip(P(chunk=48)) == 3


def test_calibration_kernels_reject_bad_arguments():
    """The copy and matrix-core calibration calls check their arguments on the
    host and enqueue nothing when they refuse (only refusals are called here)."""
    L = B.lib()
    a, b = 1 << 20, 1 << 21          # fake 16-byte-aligned device addresses (never launched)
    assert L.gdn_calib_copy(a, b, 4096, 3, None) == 3          # variant
    assert L.gdn_calib_copy(a, b, 4100, 0, None) == 2          # bytes % 16
    assert L.gdn_calib_copy(None, b, 4096, 0, None) == 1
    assert L.gdn_calib_copy(a, None, 4096, 0, None) == 1
    assert L.gdn_calib_copy(a + 8, b, 4096, 0, None) == 4
    assert L.gdn_calib_copy(a, a + 2048, 4096, 0, None) == 2   # overlapping ranges
    assert L.gdn_calib_copy(None, None, 0, 0, None) == 0       # nothing to do
    assert L.gdn_calib_mfma_loop(None, 4, 4, 0, None) == 1
    assert L.gdn_calib_mfma_loop(a + 4, 4, 4, 0, None) == 4
    assert L.gdn_calib_mfma_loop(a, 0, 4, 0, None) == 2
    assert L.gdn_calib_mfma_loop(a, 4, 0, 0, None) == 2
    assert L.gdn_calib_mfma_loop(a, 4, 4, 2, None) == 3


def test_noalloc_prefill_refuses_before_any_device_call():
    """gdn_chunk_prefill_noalloc checks the problem and the size of its fixed
    array on the host: a NULL problem, a bad problem and a problem whose
    workspace exceeds the 64 MiB array are refused without touching a GPU."""
    L = B.lib()
    assert L.gdn_chunk_prefill_noalloc_max_workspace() == 64 << 20
    fake = 1 << 20
    args = [fake, fake, fake, fake, fake, None, fake, fake, None]
    assert L.gdn_chunk_prefill_noalloc(None, *args) == 1
    # more than one chunk: one chunk's records and the carried state must fit,
    # B * Hv <= 848; one chunk: the records alone, B * Hv <= 4946
    big = B.make_problem(18, 6593, 16, 48, 128, 128)       # B * Hv = 864
    assert L.gdn_chunk_prefill_noalloc(ctypes.byref(big), *args) == 5
    big2 = B.make_problem(104, 64, 16, 48, 128, 128)       # one chunk, B * Hv = 4992
    assert L.gdn_chunk_prefill_noalloc(ctypes.byref(big2), *args) == 5
    bad = B.make_problem(1, 64, 16, 40, 128, 128)          # Hv % Hk != 0
    assert L.gdn_chunk_prefill_noalloc(ctypes.byref(bad), *args) == 2


def test_conv1d_and_rmsnorm_reject_bad_arguments():
    """The conv1d and gated RMS norm entry points check on the host and
    enqueue nothing when they refuse (fake addresses, never dereferenced)."""
    L = B.lib()
    a, w, y, s1, s2 = 1 << 20, 2 << 20, 3 << 20, 4 << 20, 5 << 20
    bf16, f32 = 1, 0
    conv = L.gdn_causal_conv1d
    assert conv(1, 10, 64, 4, 7, a, w, None, None, None, y, 1, None) == 3       # dtype
    assert conv(1, 10, 64, 5, bf16, a, w, None, None, None, y, 1, None) == 3    # K
    assert conv(1, 10, 60, 4, bf16, a, w, None, None, None, y, 1, None) == 3    # C * 2 % 16
    assert conv(1, 10, 6, 4, f32, a, w, None, None, None, y, 1, None) == 3      # C * 4 % 16
    assert conv(-1, 10, 64, 4, bf16, a, w, None, None, None, y, 1, None) == 2
    assert conv(1, 65535 * 64 + 1, 64, 4, bf16, a, w, None, None, None, y, 1, None) == 2
    assert conv(1, 10, 64, 4, bf16, None, w, None, None, None, y, 1, None) == 1
    assert conv(1, 10, 64, 4, bf16, a, None, None, None, None, y, 1, None) == 1
    assert conv(1, 10, 64, 4, bf16, a + 8, w, None, None, None, y, 1, None) == 4
    assert conv(1, 10, 64, 4, bf16, a, w, None, None, None, a + 256, 1, None) == 7   # y over x
    assert conv(1, 10, 64, 4, bf16, a, w, None, s1, s1 + 64, y, 1, None) == 7      # states overlap
    assert conv(1, 10, 64, 4, bf16, a, w, None, s1, y + 64, y, 1, None) == 7       # state_out inside y
    assert conv(0, 10, 64, 4, bf16, None, w, None, None, None, None, 1, None) == 0  # nothing to do
    norm = L.gdn_gated_rmsnorm
    assert norm(10, 128, 7, a, None, w, 1e-6, y, None) == 3
    assert norm(10, 120, bf16, a, None, w, 1e-6, y, None) == 3     # D / 8 not a power of two
    assert norm(10, 1024, bf16, a, None, w, 1e-6, y, None) == 3    # D / 8 > 64
    assert norm(10, 8, bf16, a, None, w, 1e-6, y, None) == 3       # one lane per row
    assert norm(-1, 128, bf16, a, None, w, 1e-6, y, None) == 2
    assert norm(10, 128, bf16, a, None, w, -1.0, y, None) == 2
    assert norm(10, 128, bf16, a, None, None, 1e-6, y, None) == 1
    assert norm(10, 128, bf16, None, None, w, 1e-6, y, None) == 1
    assert norm(10, 128, bf16, a, s1, w, 1e-6, s1 + 16, None) == 7  # y over z
    assert norm(10, 128, bf16, a, None, w, 1e-6, a + 16, None) == 7  # y partly over x
    assert norm(10, 128, bf16, a + 4, None, w, 1e-6, y, None) == 4
    assert norm(0, 128, bf16, None, None, w, 1e-6, None, None) == 0
