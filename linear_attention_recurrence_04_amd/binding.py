"""Thin ctypes binding of libgdn.so (include/gdn.h).

Argument marshalling only: checks that torch tensors have the layout the C ABI
expects, allocates outputs with torch's caching allocator, and passes raw
device pointers plus torch's current HIP stream.  Every step of the
computation runs in the HIP kernels; there is no CPU or PyTorch fallback --
a missing library raises.
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libgdn.so")

GDN_DTYPE_F32 = 0
GDN_DTYPE_BF16 = 1
GDN_OK = 0
STATUS_NAMES = {0: "GDN_OK", 1: "GDN_ERR_NULL_POINTER", 2: "GDN_ERR_BAD_SHAPE",
                3: "GDN_ERR_UNSUPPORTED", 4: "GDN_ERR_MISALIGNED", 5: "GDN_ERR_WORKSPACE",
                6: "GDN_ERR_HIP", 7: "GDN_ERR_ALIAS"}


class GdnProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hk", ctypes.c_int32),
                ("Hv", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("qk_l2norm", ctypes.c_int32), ("q_scale", ctypes.c_float)]


class GdnError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {text}")
        self.status = status


_lib = None


def lib():
    """Load libgdn.so once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise RuntimeError(f"{LIBRARY} is missing: build it with "
                           "`python -m linear_attention_recurrence_04_amd.build`")
    # torch first: its HIP runtime (which it loads under the name
    # libamdhip64.so) must be the one libgdn.so binds to (libamdhip64.so.7).
    # Loaded the other way round, the process ends up with two HIP runtimes
    # and the library's own one sees no device and none of torch's streams.
    import torch  # noqa: F401
    _lib = _declare(ctypes.CDLL(LIBRARY))
    return _lib


def _declare(L):
    """Argument and result types of every exported call (include/*.h)."""
    vp, fp, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t
    pp = ctypes.POINTER(GdnProblem)
    L.gdn_abi_version.restype = ctypes.c_int
    L.gdn_abi_version.argtypes = []
    L.gdn_status_string.restype = ctypes.c_char_p
    L.gdn_status_string.argtypes = [ctypes.c_int]
    L.gdn_chunk_prefill_workspace_bytes.restype = sz
    L.gdn_chunk_prefill_workspace_bytes.argtypes = [pp]
    L.gdn_chunk_prefill_variant.restype = ctypes.c_char_p
    L.gdn_chunk_prefill_variant.argtypes = [pp]
    L.gdn_chunk_prefill.restype = ctypes.c_int
    L.gdn_chunk_prefill.argtypes = [pp, vp, vp, vp, fp, fp, fp, fp, vp, vp, sz, vp]
    L.gdn_chunk_prefill_ckpt.restype = ctypes.c_int
    L.gdn_chunk_prefill_ckpt.argtypes = [pp, vp, vp, vp, fp, fp, fp, fp, vp, fp, ctypes.c_int32,
                                         vp, sz, vp]
    L.gdn_chunk_prefill_gated.restype = ctypes.c_int
    L.gdn_chunk_prefill_gated.argtypes = [pp, vp, vp, vp, fp, fp, fp, fp, fp, fp, vp, fp,
                                          ctypes.c_int32, vp, sz, vp]
    L.gdn_decode_step_gated.restype = ctypes.c_int
    L.gdn_decode_step_gated.argtypes = [pp, vp, vp, vp, fp, fp, fp, fp, fp, vp, vp]
    L.gdn_decode_multi.restype = ctypes.c_int
    L.gdn_decode_multi.argtypes = [pp, vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, vp]
    L.gdn_chunk_prefill_varlen.restype = ctypes.c_int
    L.gdn_chunk_prefill_varlen.argtypes = [pp, vp, ctypes.c_int64, vp, vp, vp, fp, fp, fp, fp, vp,
                                           vp, sz, vp]
    L.gdn_chunk_prefill_onchip.restype = ctypes.c_int
    L.gdn_chunk_prefill_onchip.argtypes = [pp, vp, vp, vp, fp, fp, fp, fp, vp, fp, ctypes.c_int32,
                                           vp]
    L.gdn_decode_step.restype = ctypes.c_int
    L.gdn_decode_step.argtypes = [pp, vp, vp, vp, fp, fp, fp, vp, vp]
    L.gdn_chunk_prefill_noalloc.restype = ctypes.c_int
    L.gdn_chunk_prefill_noalloc.argtypes = [pp, vp, vp, vp, fp, fp, fp, fp, vp, vp]
    L.gdn_chunk_prefill_noalloc_max_workspace.restype = sz
    L.gdn_chunk_prefill_noalloc_max_workspace.argtypes = []
    L.gdn_causal_conv1d.restype = ctypes.c_int
    L.gdn_causal_conv1d.argtypes = [ctypes.c_int32] * 5 + [vp, fp, fp, vp, vp, vp, ctypes.c_int32, vp]
    L.gdn_gated_rmsnorm.restype = ctypes.c_int
    L.gdn_gated_rmsnorm.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, vp, fp,
                                    ctypes.c_float, vp, vp]
    # calibration kernels (include/gdn_calib.h)
    L.gdn_calib_copy.restype = ctypes.c_int
    L.gdn_calib_copy.argtypes = [vp, vp, sz, ctypes.c_int32, vp]
    L.gdn_calib_mfma_loop.restype = ctypes.c_int
    L.gdn_calib_mfma_loop.argtypes = [fp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp]
    return L


def gdn_abi_version() -> int:
    return lib().gdn_abi_version()


def gdn_status_string(status: int) -> str:
    return lib().gdn_status_string(int(status)).decode()


def _check(status: int):
    if status != GDN_OK:
        raise GdnError(status, gdn_status_string(status))


def make_problem(B, T, Hk, Hv, dk, dv, *, chunk=64, dtype=GDN_DTYPE_BF16, qk_l2norm=True,
                 q_scale=1.0) -> GdnProblem:
    return GdnProblem(int(B), int(T), int(Hk), int(Hv), int(dk), int(dv), int(chunk),
                      int(dtype), int(bool(qk_l2norm)), float(q_scale))


def gdn_chunk_prefill_workspace_bytes(problem: GdnProblem) -> int:
    return int(lib().gdn_chunk_prefill_workspace_bytes(ctypes.byref(problem)))


def gdn_chunk_prefill_variant(problem: GdnProblem) -> str:
    return lib().gdn_chunk_prefill_variant(ctypes.byref(problem)).decode()


# kernel variant -> (kernel symbol, arithmetic, source files under csrc/)
VARIANTS = {
    "generic_f32": ("prefill_generic_kernel", "fp32-valu", ("prefill_generic.hip", "gdn_device.h")),
    "mfma_bf16": ("chunk_prep_kernel+chunk_scan_kernel", "bf16-mfma",
                  ("prefill_mfma.hip", "prefill_mfma_common.h", "prefill_prep.inc", "gdn_device.h")),
}

# the single-pass kernel of gdn_chunk_prefill_onchip (bf16, d = 128, chunk 64)
ONCHIP_KERNEL = {"name": "chunk_fused_kernel<false>", "arith": "bf16-mfma",
                 "sources": ("prefill_fused.hip", "prefill_mfma_common.h", "gdn_device.h")}


def selected_prefill_kernel(problem: GdnProblem) -> dict:
    v = gdn_chunk_prefill_variant(problem)
    if v not in VARIANTS:
        raise ValueError(f"problem rejected ({v})")
    name, arith, srcs = VARIANTS[v]
    return {"variant": v, "name": name, "arith": arith, "sources": srcs}


# ---------------------------------------------------------------------------
# torch-facing calls
# ---------------------------------------------------------------------------


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return GDN_DTYPE_BF16
    if t.dtype == torch.float32:
        return GDN_DTYPE_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _need(t, name, dtype=None, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _on_stream(fn):
    """Run a wrapper with ``stream`` (when given) as torch's current stream, so
    that every tensor it allocates (outputs, workspace) belongs to the stream
    the kernels run on: the caching allocator then reuses such memory only
    for work ordered after those kernels, also once the wrapper's local
    workspace is released."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kwargs):
        if stream is None:
            return fn(*args, **kwargs)
        with _torch().cuda.stream(stream):
            return fn(*args, stream=stream, **kwargs)
    return wrapper


@_on_stream
def gdn_chunk_prefill(q, k, v, log_g, beta, h0=None, *, chunk: int = 64,
                      qk_l2norm: bool = True, q_scale: float = 1.0, out=None, hT=None,
                      want_state: bool = True, workspace=None,
                      stream=None) -> Tuple[object, object]:
    """Chunked prefill.  q, k [B,T,Hk,d]; v [B,T,Hv,d]; log_g, beta [B,T,Hv] fp32;
    h0 [B,Hv,d,d] fp32 or None.  Returns (o [B,T,Hv,d], hT or None).
    ``hT`` may be passed (even ``hT is h0``) to receive the state in place."""
    torch = _torch()
    _need(q, "q")
    dt = _dtype_code(q)
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    _need(k, "k", q.dtype, q.shape)
    _need(v, "v", q.dtype, (B, T, Hv, dv))
    _need(log_g, "log_g", torch.float32, (B, T, Hv))
    _need(beta, "beta", torch.float32, (B, T, Hv))
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, Hv, dk, dv))
    if out is None:
        out = torch.empty((B, T, Hv, dv), dtype=q.dtype, device=q.device)
    else:
        _need(out, "out", q.dtype, (B, T, Hv, dv))
    if hT is None and want_state:
        hT = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=q.device)
    elif hT is not None:
        _need(hT, "hT", torch.float32, (B, Hv, dk, dv))
    prob = make_problem(B, T, Hk, Hv, dk, dv, chunk=chunk, dtype=dt, qk_l2norm=qk_l2norm,
                        q_scale=q_scale)
    need = gdn_chunk_prefill_workspace_bytes(prob)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().gdn_chunk_prefill(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g),
                                 _ptr(beta), _ptr(h0), _ptr(hT), _ptr(out), _ptr(workspace),
                                 ws_bytes, _stream(stream))
    _check(st)
    return out, hT


@_on_stream
def gdn_chunk_prefill_ckpt(q, k, v, log_g, beta, h0=None, *, ckpt_every: int,
                           chunk: int = 64, qk_l2norm: bool = True, q_scale: float = 1.0,
                           out=None, hT=None, h_ckpt=None, workspace=None, stream=None):
    """Chunked prefill that also stores the state every ``ckpt_every`` tokens.
    Returns (o, hT, h_ckpt) with h_ckpt [B, ceil(T/ckpt_every), Hv, d, d] fp32:
    slot j is the state after min((j+1) ckpt_every, T) tokens."""
    torch = _torch()
    _need(q, "q")
    dt = _dtype_code(q)
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    _need(k, "k", q.dtype, q.shape)
    _need(v, "v", q.dtype, (B, T, Hv, dv))
    _need(log_g, "log_g", torch.float32, (B, T, Hv))
    _need(beta, "beta", torch.float32, (B, T, Hv))
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, Hv, dk, dv))
    every = int(ckpt_every)
    nck = -(-T // every) if every > 0 else 0
    if out is None:
        out = torch.empty((B, T, Hv, dv), dtype=q.dtype, device=q.device)
    else:
        _need(out, "out", q.dtype, (B, T, Hv, dv))
    if hT is None:
        hT = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=q.device)
    else:
        _need(hT, "hT", torch.float32, (B, Hv, dk, dv))
    if h_ckpt is None:
        h_ckpt = torch.empty((B, max(nck, 0), Hv, dk, dv), dtype=torch.float32, device=q.device)
    else:
        _need(h_ckpt, "h_ckpt", torch.float32, (B, nck, Hv, dk, dv))
    prob = make_problem(B, T, Hk, Hv, dk, dv, chunk=chunk, dtype=dt, qk_l2norm=qk_l2norm,
                        q_scale=q_scale)
    need = gdn_chunk_prefill_workspace_bytes(prob)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ck_ptr = _ptr(h_ckpt) if h_ckpt.numel() else None
    st = lib().gdn_chunk_prefill_ckpt(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(log_g), _ptr(beta), _ptr(h0), _ptr(hT), _ptr(out),
                                      ck_ptr, every, _ptr(workspace), ws_bytes, _stream(stream))
    _check(st)
    return out, hT, h_ckpt


@_on_stream
def gdn_decode_step(q, k, v, log_g, beta, state, *, qk_l2norm: bool = True,
                    q_scale: float = 1.0, out=None, stream=None):
    """One decode step.  q, k [B,Hk,d]; v [B,Hv,d]; log_g, beta [B,Hv] fp32;
    state [B,Hv,d,d] fp32 is updated in place.  Returns o [B,Hv,d]."""
    torch = _torch()
    _need(q, "q")
    dt = _dtype_code(q)
    B, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    _need(k, "k", q.dtype, q.shape)
    _need(v, "v", q.dtype, (B, Hv, dv))
    _need(log_g, "log_g", torch.float32, (B, Hv))
    _need(beta, "beta", torch.float32, (B, Hv))
    _need(state, "state", torch.float32, (B, Hv, dk, dv))
    if out is None:
        out = torch.empty((B, Hv, dv), dtype=q.dtype, device=q.device)
    else:
        _need(out, "out", q.dtype, (B, Hv, dv))
    prob = make_problem(B, 1, Hk, Hv, dk, dv, chunk=0, dtype=dt, qk_l2norm=qk_l2norm,
                        q_scale=q_scale)
    st = lib().gdn_decode_step(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g),
                               _ptr(beta), _ptr(state), _ptr(out), _stream(stream))
    _check(st)
    return out


@_on_stream
def gdn_chunk_prefill_gated(q, k, v, a, b, A_log, dt_bias, h0=None, *, ckpt_every: int = 0,
                            chunk: int = 64, qk_l2norm: bool = True, q_scale: float = 1.0,
                            out=None, hT=None, h_ckpt=None, workspace=None, stream=None):
    """Chunked prefill with the gates formed in the kernels from the raw
    projections a, b [B,T,Hv] fp32 and per-head A_log, dt_bias [Hv] fp32:
    log g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b).
    Returns (o, hT, h_ckpt); h_ckpt is None unless ckpt_every > 0."""
    torch = _torch()
    _need(q, "q")
    dt = _dtype_code(q)
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    _need(k, "k", q.dtype, q.shape)
    _need(v, "v", q.dtype, (B, T, Hv, dv))
    _need(a, "a", torch.float32, (B, T, Hv))
    _need(b, "b", torch.float32, (B, T, Hv))
    _need(A_log, "A_log", torch.float32, (Hv,))
    _need(dt_bias, "dt_bias", torch.float32, (Hv,))
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, Hv, dk, dv))
    every = int(ckpt_every)
    if out is None:
        out = torch.empty((B, T, Hv, dv), dtype=q.dtype, device=q.device)
    else:
        _need(out, "out", q.dtype, (B, T, Hv, dv))
    if hT is None:
        hT = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=q.device)
    else:
        _need(hT, "hT", torch.float32, (B, Hv, dk, dv))
    ck_ptr = None
    if every > 0:
        nck = -(-T // every)
        if h_ckpt is None:
            h_ckpt = torch.empty((B, nck, Hv, dk, dv), dtype=torch.float32, device=q.device)
        else:
            _need(h_ckpt, "h_ckpt", torch.float32, (B, nck, Hv, dk, dv))
        ck_ptr = _ptr(h_ckpt) if h_ckpt.numel() else None
    prob = make_problem(B, T, Hk, Hv, dk, dv, chunk=chunk, dtype=dt, qk_l2norm=qk_l2norm,
                        q_scale=q_scale)
    need = gdn_chunk_prefill_workspace_bytes(prob)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().gdn_chunk_prefill_gated(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                       _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(h0), _ptr(hT),
                                       _ptr(out), ck_ptr, every, _ptr(workspace), ws_bytes,
                                       _stream(stream))
    _check(st)
    return out, hT, (h_ckpt if every > 0 else None)


@_on_stream
def gdn_decode_step_gated(q, k, v, a, b, A_log, dt_bias, state, *, qk_l2norm: bool = True,
                          q_scale: float = 1.0, out=None, stream=None):
    """One decode step with the gates formed in the kernel from a, b [B,Hv] fp32
    and A_log, dt_bias [Hv] fp32; state [B,Hv,d,d] is updated in place."""
    torch = _torch()
    _need(q, "q")
    dt = _dtype_code(q)
    B, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    _need(k, "k", q.dtype, q.shape)
    _need(v, "v", q.dtype, (B, Hv, dv))
    _need(a, "a", torch.float32, (B, Hv))
    _need(b, "b", torch.float32, (B, Hv))
    _need(A_log, "A_log", torch.float32, (Hv,))
    _need(dt_bias, "dt_bias", torch.float32, (Hv,))
    _need(state, "state", torch.float32, (B, Hv, dk, dv))
    if out is None:
        out = torch.empty((B, Hv, dv), dtype=q.dtype, device=q.device)
    else:
        _need(out, "out", q.dtype, (B, Hv, dv))
    prob = make_problem(B, 1, Hk, Hv, dk, dv, chunk=0, dtype=dt, qk_l2norm=qk_l2norm,
                        q_scale=q_scale)
    st = lib().gdn_decode_step_gated(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                     _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(state), _ptr(out),
                                     _stream(stream))
    _check(st)
    return out


@_on_stream
def gdn_decode_multi(q, k, v, log_g, beta, state, *, A_log=None, dt_bias=None,
                     want_states: bool = False, qk_l2norm: bool = True, q_scale: float = 1.0,
                     out=None, states=None, stream=None):
    """T decode tokens per sequence in one call.  q, k [B,T,Hk,d]; v [B,T,Hv,d];
    log_g, beta [B,T,Hv] fp32 (raw projections a, b when A_log and dt_bias
    [Hv] are given); state [B,Hv,d,d] fp32 updated in place.  Returns
    (o [B,T,Hv,d], states [B,T,Hv,d,d] or None): the state after every token."""
    torch = _torch()
    _need(q, "q")
    dt = _dtype_code(q)
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    _need(k, "k", q.dtype, q.shape)
    _need(v, "v", q.dtype, (B, T, Hv, dv))
    _need(log_g, "log_g", torch.float32, (B, T, Hv))
    _need(beta, "beta", torch.float32, (B, T, Hv))
    _need(state, "state", torch.float32, (B, Hv, dk, dv))
    if (A_log is None) != (dt_bias is None):
        raise ValueError("A_log and dt_bias go together")
    if A_log is not None:
        _need(A_log, "A_log", torch.float32, (Hv,))
        _need(dt_bias, "dt_bias", torch.float32, (Hv,))
    if out is None:
        out = torch.empty((B, T, Hv, dv), dtype=q.dtype, device=q.device)
    else:
        _need(out, "out", q.dtype, (B, T, Hv, dv))
    if states is None and want_states:
        states = torch.empty((B, T, Hv, dk, dv), dtype=torch.float32, device=q.device)
    elif states is not None:
        _need(states, "states", torch.float32, (B, T, Hv, dk, dv))
    prob = make_problem(B, T, Hk, Hv, dk, dv, chunk=0, dtype=dt, qk_l2norm=qk_l2norm,
                        q_scale=q_scale)
    st = lib().gdn_decode_multi(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g),
                                _ptr(beta), _ptr(A_log), _ptr(dt_bias), _ptr(state), _ptr(out),
                                _ptr(states) if states is not None and states.numel() else None,
                                _stream(stream))
    _check(st)
    return out, states


@_on_stream
def gdn_chunk_prefill_varlen(q, k, v, log_g, beta, cu_seqlens, max_seqlen: Optional[int] = None,
                             h0=None, *, chunk: int = 64, qk_l2norm: bool = True,
                             q_scale: float = 1.0, out=None, hT=None, workspace=None,
                             stream=None):
    """Chunked prefill of a packed batch of sequences of different lengths.
    q, k [total, Hk, d]; v [total, Hv, d]; log_g, beta [total, Hv] fp32;
    cu_seqlens int32 [N+1] on the GPU (sequence b = tokens cu[b] .. cu[b+1]-1);
    h0 [N, Hv, d, d] fp32 or None.  ``max_seqlen`` (the longest sequence) sizes
    the launch; when omitted it is read from cu_seqlens, which synchronises.
    Returns (o [total, Hv, d], hT [N, Hv, d, d])."""
    torch = _torch()
    _need(q, "q")
    dt = _dtype_code(q)
    total, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    _need(k, "k", q.dtype, q.shape)
    _need(v, "v", q.dtype, (total, Hv, dv))
    _need(log_g, "log_g", torch.float32, (total, Hv))
    _need(beta, "beta", torch.float32, (total, Hv))
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of N+1 offsets")
    N = cu_seqlens.numel() - 1
    if max_seqlen is None:
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if N > 0 else 0
    if h0 is not None:
        _need(h0, "h0", torch.float32, (N, Hv, dk, dv))
    if out is None:
        out = torch.empty((total, Hv, dv), dtype=q.dtype, device=q.device)
    else:
        _need(out, "out", q.dtype, (total, Hv, dv))
    if hT is None:
        hT = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=q.device)
    else:
        _need(hT, "hT", torch.float32, (N, Hv, dk, dv))
    prob = make_problem(N, max_seqlen, Hk, Hv, dk, dv, chunk=chunk, dtype=dt,
                        qk_l2norm=qk_l2norm, q_scale=q_scale)
    need = gdn_chunk_prefill_workspace_bytes(prob)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().gdn_chunk_prefill_varlen(ctypes.byref(prob), _ptr(cu_seqlens), int(total), _ptr(q),
                                        _ptr(k), _ptr(v), _ptr(log_g), _ptr(beta), _ptr(h0),
                                        _ptr(hT), _ptr(out), _ptr(workspace), ws_bytes,
                                        _stream(stream))
    _check(st)
    return out, hT


@_on_stream
def gdn_chunk_prefill_onchip(q, k, v, log_g, beta, h0=None, *, ckpt_every: int = 0,
                             chunk: int = 64, qk_l2norm: bool = True, q_scale: float = 1.0,
                             out=None, hT=None, h_ckpt=None, want_state: bool = True,
                             stream=None):
    """Chunked prefill in a single pass with every intermediate on chip (no
    workspace).  Arguments as gdn_chunk_prefill_ckpt; returns (o, hT, h_ckpt),
    h_ckpt None unless ckpt_every > 0."""
    torch = _torch()
    _need(q, "q")
    dt = _dtype_code(q)
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    _need(k, "k", q.dtype, q.shape)
    _need(v, "v", q.dtype, (B, T, Hv, dv))
    _need(log_g, "log_g", torch.float32, (B, T, Hv))
    _need(beta, "beta", torch.float32, (B, T, Hv))
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, Hv, dk, dv))
    every = int(ckpt_every)
    if out is None:
        out = torch.empty((B, T, Hv, dv), dtype=q.dtype, device=q.device)
    else:
        _need(out, "out", q.dtype, (B, T, Hv, dv))
    if hT is None and want_state:
        hT = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=q.device)
    elif hT is not None:
        _need(hT, "hT", torch.float32, (B, Hv, dk, dv))
    ck_ptr = None
    if every > 0:
        nck = -(-T // every)
        if h_ckpt is None:
            h_ckpt = torch.empty((B, nck, Hv, dk, dv), dtype=torch.float32, device=q.device)
        else:
            _need(h_ckpt, "h_ckpt", torch.float32, (B, nck, Hv, dk, dv))
        ck_ptr = _ptr(h_ckpt) if h_ckpt.numel() else None
    prob = make_problem(B, T, Hk, Hv, dk, dv, chunk=chunk, dtype=dt, qk_l2norm=qk_l2norm,
                        q_scale=q_scale)
    st = lib().gdn_chunk_prefill_onchip(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(log_g), _ptr(beta), _ptr(h0), _ptr(hT), _ptr(out),
                                        ck_ptr, every, _stream(stream))
    _check(st)
    return out, hT, (h_ckpt if every > 0 else None)


def gdn_chunk_prefill_noalloc_max_workspace() -> int:
    return int(lib().gdn_chunk_prefill_noalloc_max_workspace())


@_on_stream
def gdn_chunk_prefill_noalloc(q, k, v, log_g, beta, h0=None, *, chunk: int = 64,
                              qk_l2norm: bool = True, q_scale: float = 1.0, out=None, hT=None,
                              want_state: bool = True, stream=None):
    """gdn_chunk_prefill with the library's fixed per-device workspace array
    (the C call allocates nothing; pass ``out`` and ``hT`` to allocate nothing
    here either).  Returns (o, hT or None)."""
    torch = _torch()
    _need(q, "q")
    dt = _dtype_code(q)
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    _need(k, "k", q.dtype, q.shape)
    _need(v, "v", q.dtype, (B, T, Hv, dv))
    _need(log_g, "log_g", torch.float32, (B, T, Hv))
    _need(beta, "beta", torch.float32, (B, T, Hv))
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, Hv, dk, dv))
    if out is None:
        out = torch.empty((B, T, Hv, dv), dtype=q.dtype, device=q.device)
    else:
        _need(out, "out", q.dtype, (B, T, Hv, dv))
    if hT is None and want_state:
        hT = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=q.device)
    elif hT is not None:
        _need(hT, "hT", torch.float32, (B, Hv, dk, dv))
    prob = make_problem(B, T, Hk, Hv, dk, dv, chunk=chunk, dtype=dt, qk_l2norm=qk_l2norm,
                        q_scale=q_scale)
    st = lib().gdn_chunk_prefill_noalloc(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(log_g), _ptr(beta), _ptr(h0), _ptr(hT), _ptr(out),
                                         _stream(stream))
    _check(st)
    return out, hT


@_on_stream
def gdn_causal_conv1d(x, weight, bias=None, state_in=None, *, silu: bool = True, out=None,
                      state_out=None, want_state: bool = True, stream=None):
    """Causal depthwise conv1d over the channel axis.  x [B, T, C] (bf16 or
    fp32), weight [C, K] fp32, bias [C] fp32 or None, state_in [B, K-1, C] or
    None (zeros).  Returns (y [B, T, C], state_out [B, K-1, C] or None);
    ``state_out`` may be ``state_in`` to update it in place."""
    torch = _torch()
    _need(x, "x")
    dt = _dtype_code(x)
    B, T, C = x.shape
    _need(weight, "weight", torch.float32)
    if weight.dim() != 2 or weight.shape[0] != C:
        raise ValueError("weight must be [C, K]")
    K = weight.shape[1]
    if bias is not None:
        _need(bias, "bias", torch.float32, (C,))
    if state_in is not None:
        _need(state_in, "state_in", x.dtype, (B, K - 1, C))
    if out is None:
        out = torch.empty_like(x)
    else:
        _need(out, "out", x.dtype, (B, T, C))
    if state_out is None and want_state:
        state_out = torch.empty((B, K - 1, C), dtype=x.dtype, device=x.device)
    elif state_out is not None:
        _need(state_out, "state_out", x.dtype, (B, K - 1, C))
    st_ptr = _ptr(state_out) if state_out is not None and state_out.numel() else None
    _check(lib().gdn_causal_conv1d(B, T, C, K, dt, _ptr(x) if x.numel() else None, _ptr(weight),
                                   _ptr(bias), _ptr(state_in) if state_in is not None and state_in.numel() else None,
                                   st_ptr, _ptr(out) if out.numel() else None, int(bool(silu)),
                                   _stream(stream)))
    return out, state_out


@_on_stream
def gdn_gated_rmsnorm(x, z, weight, eps: float = 1e-6, *, out=None, stream=None):
    """y = x / sqrt(mean(x^2) + eps) * weight * silu(z) over the last axis of x
    (bf16 or fp32); z like x or None (no gate); weight fp32 [D].  ``out`` may
    be x itself."""
    torch = _torch()
    _need(x, "x")
    dt = _dtype_code(x)
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    if z is not None:
        _need(z, "z", x.dtype, tuple(x.shape))
    _need(weight, "weight", torch.float32, (D,))
    if out is None:
        out = torch.empty_like(x)
    else:
        _need(out, "out", x.dtype, tuple(x.shape))
    _check(lib().gdn_gated_rmsnorm(rows, D, dt, _ptr(x) if rows else None, _ptr(z) if z is not None and rows else None,
                                   _ptr(weight), float(eps), _ptr(out) if rows else None, _stream(stream)))
    return out


# ---------------------------------------------------------------------------
# calibration kernels (include/gdn_calib.h): achieved peaks of this GPU
# ---------------------------------------------------------------------------

CALIB_MFMA_FLOPS = {0: 2 * 16 * 16 * 32, 1: 2 * 32 * 32 * 16}   # per instruction
CALIB_MFMA_CHAINS = 8


def gdn_calib_copy(src, dst, *, variant: int = 0, stream=None):
    """Copy src into dst (same byte size, contiguous device tensors) with the
    in-library streaming copy kernel."""
    _need(src, "src")
    _need(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same size in bytes")
    _check(lib().gdn_calib_copy(_ptr(src), _ptr(dst), nbytes, int(variant), _stream(stream)))


def gdn_calib_mfma_loop(out, workgroups: int, iters: int, *, variant: int = 0, stream=None) -> float:
    """Run the bf16 matrix-core loop; out holds workgroups * 4 floats.  Returns
    the flops the launch performs."""
    torch = _torch()
    _need(out, "out", torch.float32)
    if out.numel() < 4 * int(workgroups):
        raise ValueError("out must hold 4 floats per workgroup")
    _check(lib().gdn_calib_mfma_loop(_ptr(out), int(workgroups), int(iters), int(variant),
                                     _stream(stream)))
    return float(workgroups) * 4 * iters * CALIB_MFMA_CHAINS * CALIB_MFMA_FLOPS[int(variant)]
