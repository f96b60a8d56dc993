"""fp64 CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never loads it and the
two share no code; the only common module is the seeded input generator.

The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, sequential loops);
this file only compiles it with gcc and marshals numpy arrays through ctypes.

Page citations for what is computed:
  * "Qwen3.5 Gated Delta Net NKI Kernel for AWS Neuron" (model card),
    section "How It Works" -- the five per-token steps (decay, read, delta,
    write, output from the updated state);
  * same card, "Correctness Contract" -- log g <= 0, no clamping, heads
    independent;
  * "Qwen3.6: Fused DeltaNet Direct-Solve Follow-Up" (PR comment), sections
    "Why This Exists" / "Implementation Details" -- the chunked form with a
    direct triangular solve, and the Neumann power-doubling it replaced.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "gdn_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_lib = None
_lib_path = None


def build(src: str = SOURCE, out: str = LIBRARY) -> str:
    """Compile the oracle with gcc into a shared library and return its path."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-I", _HERE, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _declare(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.oracle_gdn_sequential.restype = i
    lib.oracle_gdn_sequential.argtypes = [i, i, i, i, i, i, i, ctypes.c_double,
                                          dp, dp, dp, dp, dp, dp, dp, dp, i]
    lib.oracle_gdn_chunked.restype = i
    lib.oracle_gdn_chunked.argtypes = [i, i, i, i, i, i, i, i, ctypes.c_double,
                                       dp, dp, dp, dp, dp, dp, dp, dp]
    lib.oracle_unit_lower_inverse.restype = i
    lib.oracle_unit_lower_inverse.argtypes = [i, dp, dp]
    lib.oracle_neumann_inverse.restype = i
    lib.oracle_neumann_inverse.argtypes = [i, dp, dp]
    lib.oracle_qwen_gates.restype = i
    lib.oracle_qwen_gates.argtypes = [ctypes.c_long, i, dp, dp, dp, dp, dp, dp]
    lib.oracle_causal_conv1d.restype = i
    lib.oracle_causal_conv1d.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp, i]
    lib.oracle_gated_rmsnorm.restype = i
    lib.oracle_gated_rmsnorm.argtypes = [ctypes.c_long, i, dp, dp, dp, ctypes.c_double, dp]
    return lib


def load(path: Optional[str] = None):
    """Load (building first if absent) the oracle library.

    ``path`` selects another build of the same source (the mutation tests
    compile deliberately broken copies into a temporary directory)."""
    global _lib, _lib_path
    if path is None:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIBRARY):
            build()
        _lib = _declare(ctypes.CDLL(LIBRARY))
        _lib_path = LIBRARY
        return _lib
    return _declare(ctypes.CDLL(path))


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _shapes(q, k, v, log_g, beta):
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or log_g.shape != (B, T, Hv) \
            or beta.shape != (B, T, Hv):
        raise ValueError("inconsistent oracle input shapes")
    return B, T, Hk, Hv, dk, dv


def gdn_sequential(q, k, v, log_g, beta, h0=None, *, qk_l2norm: bool = True,
                   q_scale: float = 1.0, nthreads: int = 1,
                   lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """Token-serial definition.  Returns (o [B,T,Hv,dv], hT [B,Hv,dk,dv]) in fp64."""
    lib = lib or load()
    q, k, v, log_g, beta = map(_f64, (q, k, v, log_g, beta))
    B, T, Hk, Hv, dk, dv = _shapes(q, k, v, log_g, beta)
    h0a = None if h0 is None else _f64(h0)
    if h0a is not None and h0a.shape != (B, Hv, dk, dv):
        raise ValueError("h0 must be [B,Hv,dk,dv]")
    o = np.zeros((B, T, Hv, dv))
    hT = np.zeros((B, Hv, dk, dv))
    rc = lib.oracle_gdn_sequential(B, T, Hk, Hv, dk, dv, int(bool(qk_l2norm)),
                                   float(q_scale), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(log_g), _ptr(beta), _ptr(h0a), _ptr(o),
                                   _ptr(hT), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_gdn_sequential failed ({rc})")
    return o, hT


def gdn_chunked(q, k, v, log_g, beta, h0=None, *, chunk: int, qk_l2norm: bool = True,
                q_scale: float = 1.0, lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """Chunked (WY, direct solve) form; equal to gdn_sequential up to rounding."""
    lib = lib or load()
    q, k, v, log_g, beta = map(_f64, (q, k, v, log_g, beta))
    B, T, Hk, Hv, dk, dv = _shapes(q, k, v, log_g, beta)
    h0a = None if h0 is None else _f64(h0)
    o = np.zeros((B, T, Hv, dv))
    hT = np.zeros((B, Hv, dk, dv))
    rc = lib.oracle_gdn_chunked(B, T, Hk, Hv, dk, dv, int(chunk), int(bool(qk_l2norm)),
                                float(q_scale), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g),
                                _ptr(beta), _ptr(h0a), _ptr(o), _ptr(hT))
    if rc != 0:
        raise ValueError(f"oracle_gdn_chunked failed ({rc})")
    return o, hT


def unit_lower_inverse(A, lib=None) -> np.ndarray:
    """(I + strictly_lower(A))^-1 by forward substitution."""
    lib = lib or load()
    A = _f64(A)
    n = A.shape[0]
    out = np.zeros((n, n))
    if lib.oracle_unit_lower_inverse(n, _ptr(A), _ptr(out)) != 0:
        raise ValueError("oracle_unit_lower_inverse failed")
    return out


def neumann_inverse(A, lib=None) -> np.ndarray:
    """(I + strictly_lower(A))^-1 by Neumann power doubling."""
    lib = lib or load()
    A = _f64(A)
    n = A.shape[0]
    out = np.zeros((n, n))
    if lib.oracle_neumann_inverse(n, _ptr(A), _ptr(out)) != 0:
        raise ValueError("oracle_neumann_inverse failed")
    return out


def qwen_gates(a, b, A_log, dt_bias, lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """(log_g, beta) from raw projections a, b [..., Hv] and per-head A_log,
    dt_bias [Hv]: log g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b)."""
    lib = lib or load()
    a, b, A_log, dt_bias = map(_f64, (a, b, A_log, dt_bias))
    Hv = A_log.shape[0]
    if a.shape != b.shape or a.shape[-1] != Hv or dt_bias.shape != (Hv,):
        raise ValueError("inconsistent gate shapes")
    n = a.size // Hv
    log_g = np.zeros(a.shape)
    beta = np.zeros(a.shape)
    rc = lib.oracle_qwen_gates(n, Hv, _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
                               _ptr(log_g), _ptr(beta))
    if rc != 0:
        raise ValueError(f"oracle_qwen_gates failed ({rc})")
    return log_g, beta


def causal_conv1d(x, w, bias=None, state_in=None, *, silu: bool = True,
                  lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """Causal depthwise conv1d over the channel axis (the operations around
    the recurrence, "Qwen3.5 Gated Delta Net NKI Kernel for AWS Neuron",
    section "How It Works"; the carried convolution state of "Add Qwen3.6-27B
    hybrid DeltaNet/GQA contrib model and vLLM serving path", "Summary").
    x [B, T, C], w [C, K], bias [C] or None, state_in [B, K-1, C] or None
    (zeros).  Returns (y [B, T, C], state_out [B, K-1, C]) in fp64."""
    lib = lib or load()
    x, w = _f64(x), _f64(w)
    if x.ndim != 3 or w.ndim != 2 or w.shape[0] != x.shape[2]:
        raise ValueError("x must be [B, T, C] and w [C, K]")
    B, T, C = x.shape
    K = w.shape[1]
    bias_a = None if bias is None else _f64(bias)
    st = None if state_in is None else _f64(state_in)
    if st is not None and st.shape != (B, K - 1, C):
        raise ValueError("state_in must be [B, K-1, C]")
    y = np.zeros((B, T, C))
    st_out = np.zeros((B, K - 1, C))
    rc = lib.oracle_causal_conv1d(B, T, C, K, _ptr(x), _ptr(w), _ptr(bias_a), _ptr(st),
                                  _ptr(st_out), _ptr(y), int(bool(silu)))
    if rc != 0:
        raise ValueError(f"oracle_causal_conv1d failed ({rc})")
    return y, st_out


def gated_rmsnorm(x, z, w, eps: float = 1e-6, lib=None) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * w * silu(z) over the last axis (the RMS
    norm and gating around the recurrence, same section); z None: no gate."""
    lib = lib or load()
    x, w = _f64(x), _f64(w)
    D = x.shape[-1]
    if w.shape != (D,):
        raise ValueError("w must hold one value per element of the last axis")
    za = None if z is None else _f64(z)
    if za is not None and za.shape != x.shape:
        raise ValueError("z must have the shape of x")
    rows = x.size // D if D else 0
    y = np.zeros(x.shape)
    rc = lib.oracle_gated_rmsnorm(rows, D, _ptr(x), _ptr(za), _ptr(w), float(eps), _ptr(y))
    if rc != 0:
        raise ValueError(f"oracle_gated_rmsnorm failed ({rc})")
    return y
