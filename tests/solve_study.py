"""Direct solve against Neumann power doubling for the chunk system (I + A) T = I.

A diagnostic study on the CPU.  "Qwen3.6: Fused DeltaNet Direct-Solve
Follow-Up" (sections "Why This Exists", "Implementation Details") reports that
the Neumann power-doubling solve, which forms full matrix powers of A, gave
unstable output under realistic Qwen gate scales, and that a direct triangular
solve fixed it at some cost in speed.  This module rebuilds that comparison
for the chunk matrices of the 27B workload:

  A_rs = beta_r exp(gamma_r - gamma_s) (k_r . k_s),  s < r,  unit-norm keys,

with the 27B gate law (log g = -exp(A_log) softplus(dt), A_log ~ U(-2, 1),
dt ~ N(0, 1), beta = sigmoid(N(0, 1))) and keys of a chosen mutual cosine
(real keys are far from orthogonal).  Each solve runs in two emulated
precisions, fp32 throughout and bf16 operands with fp32 accumulation (what a
bf16 matrix engine does); the error is measured against the fp64 inverse of
the oracle (forward substitution, pinned separately).

Solves compared:
  direct_fp32       forward substitution, fp32
  blocked_bf16      the GPU kernel's scheme: 16x16 diagonal blocks by fp32
                    forward substitution, then T_ij = -T_ii sum_k A_ik T_kj
                    with bf16 operands and fp32 accumulation
  neumann_fp32      prod_j (I + (-A)^(2^j)), fp32
  neumann_bf16      the same product with bf16 operands, fp32 accumulation

Run ``python tests/solve_study.py`` for the table.
"""
from __future__ import annotations

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402

C = 64
D = 128


def bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def chunk_matrix(rng: np.random.Generator, cos: float, beta_hi: bool = False) -> np.ndarray:
    """One 64x64 strictly lower A of the 27B gate law with keys of mutual cosine ~cos."""
    a_log = rng.uniform(-2.0, 1.0)
    dt = rng.standard_normal(C)
    log_g = -np.exp(a_log) * np.logaddexp(0.0, dt)
    gam = np.cumsum(log_g)
    beta = np.ones(C) if beta_hi else 1.0 / (1.0 + np.exp(-rng.standard_normal(C)))
    shared = rng.standard_normal(D)
    shared /= np.linalg.norm(shared)
    noise = rng.standard_normal((C, D))
    noise /= np.linalg.norm(noise, axis=1, keepdims=True)
    K = np.sqrt(cos) * shared[None, :] + np.sqrt(1.0 - cos) * noise
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    G = K @ K.T
    dec = np.exp(np.minimum(gam[:, None] - gam[None, :], 0.0))
    return np.tril(beta[:, None] * dec * G, -1)


def direct_fp32(A: np.ndarray) -> np.ndarray:
    A = A.astype(np.float32)
    n = A.shape[0]
    T = np.eye(n, dtype=np.float32)
    for i in range(1, n):
        T[i, :i] = -(A[i, :i] @ T[:i, :i])
    return T


def blocked_bf16(A: np.ndarray, b: int = 16) -> np.ndarray:
    A = A.astype(np.float32)
    n = A.shape[0]
    nb = n // b
    T = np.zeros((n, n), dtype=np.float32)
    blk = lambda M, i, j: M[i * b:(i + 1) * b, j * b:(j + 1) * b]  # noqa: E731
    for i in range(nb):
        T[i * b:(i + 1) * b, i * b:(i + 1) * b] = direct_fp32(blk(A, i, i))
    for j in range(nb):
        for i in range(j + 1, nb):
            R = np.zeros((b, b), dtype=np.float32)
            for k in range(j, i):
                R += bf16(blk(A, i, k)) @ bf16(blk(T, k, j))
            T[i * b:(i + 1) * b, j * b:(j + 1) * b] = bf16(blk(T, i, i)) @ bf16(-R)
    return T


def neumann(A: np.ndarray, operands_bf16: bool) -> tuple:
    """Returns (T, largest |entry| of the powers formed on the way)."""
    rnd = bf16 if operands_bf16 else (lambda x: x.astype(np.float32))
    n = A.shape[0]
    P = (-A).astype(np.float32)
    R = np.eye(n, dtype=np.float32)
    growth = float(np.max(np.abs(P)))
    span = 1
    while span < n:
        R = (rnd(R) @ rnd(np.eye(n, dtype=np.float32) + P)).astype(np.float32)
        P = (rnd(P) @ rnd(P)).astype(np.float32)
        growth = max(growth, float(np.max(np.abs(P))))
        span *= 2
    return R, growth


def rel(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def study(cosines=(0.0, 0.5, 0.9, 0.99), trials: int = 12, seed: int = 0, beta_hi=(False, True)):
    """Rows: dict(cos, beta_hi, norm_A, growth, err_<solve> median / max)."""
    rng = np.random.default_rng(seed)
    rows = []
    for bh in beta_hi:
        for cos in cosines:
            errs = {k: [] for k in ("direct_fp32", "blocked_bf16", "neumann_fp32", "neumann_bf16")}
            growth, norms, tnorm = [], [], []
            for _ in range(trials):
                A = chunk_matrix(rng, cos, bh)
                T = oracle.unit_lower_inverse(A)
                errs["direct_fp32"].append(rel(direct_fp32(A), T))
                errs["blocked_bf16"].append(rel(blocked_bf16(A), T))
                tn, g = neumann(A, False)
                errs["neumann_fp32"].append(rel(tn, T))
                tb, _ = neumann(A, True)
                errs["neumann_bf16"].append(rel(tb, T))
                growth.append(g)
                norms.append(float(np.linalg.norm(A, 2)))
                tnorm.append(float(np.max(np.abs(T))))
            row = {"cos": cos, "beta_hi": bh, "norm_A": float(np.median(norms)),
                   "max_T": float(np.max(tnorm)), "power_growth": float(np.max(growth))}
            for k, v in errs.items():
                row[k + "_med"] = float(np.median(v))
                row[k + "_max"] = float(np.max(v))
            rows.append(row)
    return rows


def flop_counts(n: int = C, b: int = 16) -> dict:
    """Multiply-adds of each solve for one n x n chunk system."""
    steps = int(np.ceil(np.log2(n)))
    nb = n // b
    off = sum((i - j) for j in range(nb) for i in range(j + 1, nb)) * b ** 3 + \
        nb * (nb - 1) // 2 * b ** 3
    return {"direct": n * (n - 1) * (n + 1) // 6,
            "blocked (diag fp32 + off-diag products)": nb * b * (b - 1) * (b + 1) // 6 + off,
            "neumann (dense products)": 2 * steps * n ** 3,
            "neumann dependent steps": 2 * steps, "direct dependent steps": n - 1}


if __name__ == "__main__":
    print("solve error ||T_hat - T||_F / ||T||_F against the fp64 inverse, 64x64 chunks")
    hdr = ("cos", "beta=1", "|A|_2", "max|T|", "max|A^2^j|", "direct32", "blocked16",
           "neumann32", "neumann16")
    print(" | ".join(hdr))
    for r in study():
        print(f"{r['cos']:.2f} | {str(r['beta_hi']):5s} | {r['norm_A']:7.2f} | {r['max_T']:9.3g} | "
              f"{r['power_growth']:10.3g} | {r['direct_fp32_max']:.2e} | {r['blocked_bf16_max']:.2e} | "
              f"{r['neumann_fp32_max']:.2e} | {r['neumann_bf16_max']:.2e}")
    print(flop_counts())
