"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each ``pin_*`` function takes an oracle library handle and raises
AssertionError when the oracle disagrees with:
  * the expanded matrix form of the recurrence, S_t = g_t (I - b_t k_t k_t^T)
    S_{t-1} + b_t k_t v_t^T, o_t = S_t^T q_t (evaluated here with numpy
    matrices, a different expression from the oracle's five-step loop);
  * closed forms (no write when beta = 0; exact overwrite with orthonormal
    keys; the scalar recurrence at d = 1; a small exact example);
  * invariants (identity plumbing, unit-key read-back, split invariance,
    linearity, non-expansiveness, GQA grouping, normalisation scale
    invariance);
  * library routines (numpy's matrix inverse for the triangular solve).

The same list is run against deliberately broken builds of the oracle
(tests/test_oracle_mutants.py) to show that each plausible mistake is caught.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _inputs(rng, B, T, Hk, Hv, dk, dv, gate="uniform"):
    q = rng.standard_normal((B, T, Hk, dk))
    k = rng.standard_normal((B, T, Hk, dk))
    v = rng.standard_normal((B, T, Hv, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hv))))
    if gate == "uniform":
        log_g = rng.uniform(-0.5, -0.01, size=(B, T, Hv))
    else:  # Qwen-scale gates: -exp(A_log) softplus(dt)
        a_log = rng.uniform(-2.0, 1.0, size=(Hv,))
        log_g = -np.exp(a_log) * np.logaddexp(0.0, rng.standard_normal((B, T, Hv)))
    h0 = 0.02 * rng.standard_normal((B, Hv, dk, dv))
    return q, k, v, log_g, beta, h0


def _unit(x):
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    return x / np.maximum(n, 1e-6)


def _rel(a, b):
    den = max(np.linalg.norm(b), 1e-300)
    return np.linalg.norm(a - b) / den


# --------------------------------------------------------------------------


def pin_identity_plumbing(lib):
    """beta = 0, g = 1: state untouched (bitwise), o_t = S0^T q_hat_t."""
    rng = _rng(1)
    B, T, Hk, Hv, d = 2, 9, 2, 4, 6
    q, k, v, _, _, h0 = _inputs(rng, B, T, Hk, Hv, d, d)
    log_g = np.zeros((B, T, Hv))
    beta = np.zeros((B, T, Hv))
    o, hT = oracle.gdn_sequential(q, k, v, log_g, beta, h0, lib=lib)
    assert np.array_equal(hT, h0), "state changed although beta=0 and g=1"
    qh = _unit(q)
    r = Hv // Hk
    for h in range(Hv):
        exp_o = np.einsum("btk,bkv->btv", qh[:, :, h // r, :], h0[:, h])
        assert _rel(o[:, :, h], exp_o) < 1e-13


def pin_matrix_form(lib):
    """Oracle equals the expanded matrix recurrence (numpy), several shapes."""
    for seed, (B, T, Hk, Hv, dk, dv, qs, gate) in enumerate([
            (1, 17, 1, 1, 5, 5, 1.0, "uniform"),
            (2, 11, 2, 4, 4, 4, 0.75, "qwen"),
            (1, 13, 1, 3, 3, 7, 1.0, "uniform"),
            (1, 9, 2, 2, 6, 3, 1.25, "qwen")]):
        rng = _rng(100 + seed)
        q, k, v, log_g, beta, h0 = _inputs(rng, B, T, Hk, Hv, dk, dv, gate)
        o, hT = oracle.gdn_sequential(q, k, v, log_g, beta, h0, q_scale=qs, lib=lib)
        qh, kh = _unit(q), _unit(k)
        r = Hv // Hk
        I = np.eye(dk)
        for b in range(B):
            for h in range(Hv):
                S = h0[b, h].copy()
                for t in range(T):
                    kk = kh[b, t, h // r][:, None]
                    g = np.exp(log_g[b, t, h])
                    bt = beta[b, t, h]
                    S = g * (I - bt * kk @ kk.T) @ S + bt * kk @ v[b, t, h][None, :]
                    exp_o = qs * (S.T @ qh[b, t, h // r])
                    assert _rel(o[b, t, h], exp_o) < 1e-12, (seed, b, h, t)
                assert _rel(hT[b, h], S) < 1e-12, (seed, b, h)


def pin_unit_key_readback(lib):
    """g = 1, beta = 1, unit k: S_t^T k_t = v_t (read with q_t = k_t)."""
    rng = _rng(2)
    B, T, H, d = 1, 12, 2, 8
    _, _, v, _, _, h0 = _inputs(rng, B, T, H, H, d, d)
    # basis keys, normalisation off
    idx = rng.integers(0, d, size=(B, T, H))
    k = np.zeros((B, T, H, d))
    for t in range(T):
        for h in range(H):
            k[0, t, h, idx[0, t, h]] = 1.0
    ones = np.ones((B, T, H))
    o, _ = oracle.gdn_sequential(k, k, v, np.zeros((B, T, H)), ones, h0,
                                 qk_l2norm=False, lib=lib)
    assert np.max(np.abs(o - v)) < 1e-14 * max(1.0, np.max(np.abs(v)))
    # random unit keys, normalisation on
    k = _unit(rng.standard_normal((B, T, H, d)))
    o, _ = oracle.gdn_sequential(k, k, v, np.zeros((B, T, H)), ones, h0, lib=lib)
    assert np.max(np.abs(o - v)) < 1e-12


def pin_no_write_closed_form(lib):
    """beta = 0: o_t = exp(sum_{s<=t} log g_s) S0^T q_hat_t."""
    rng = _rng(3)
    B, T, Hk, Hv, d = 1, 20, 1, 2, 5
    q, k, v, log_g, _, h0 = _inputs(rng, B, T, Hk, Hv, d, d, "qwen")
    beta = np.zeros((B, T, Hv))
    o, hT = oracle.gdn_sequential(q, k, v, log_g, beta, h0, lib=lib)
    qh = _unit(q)
    for h in range(Hv):
        G = np.exp(np.cumsum(log_g[0, :, h]))
        exp_o = G[:, None] * (qh[0, :, 0] @ h0[0, h])
        assert _rel(o[0, :, h], exp_o) < 1e-13
        assert _rel(hT[0, h], G[-1] * h0[0, h]) < 1e-13



def pin_closed_gate(lib):
    """g = 0 (log g = -inf) forgets the state before the write.  All gates
    closed: S_t = beta_t k_hat_t v_t^T, so o_t = beta_t (k_hat_t . q_hat_t) v_t.
    One closed token at t0: the run from t0 on is a fresh run from a zero
    state (bitwise)."""
    rng = _rng(17)
    B, T, Hk, Hv, d = 1, 12, 1, 2, 5
    q, k, v, log_g, beta, h0 = _inputs(rng, B, T, Hk, Hv, d, d, "qwen")
    closed = np.full_like(log_g, -np.inf)
    o, hT = oracle.gdn_sequential(q, k, v, closed, beta, h0, lib=lib)
    qh, kh = _unit(q), _unit(k)
    kq = np.sum(kh[0, :, 0] * qh[0, :, 0], axis=-1)
    for h in range(Hv):
        assert _rel(o[0, :, h], (beta[0, :, h] * kq)[:, None] * v[0, :, h]) < 1e-14
        assert _rel(hT[0, h], beta[0, -1, h] * np.outer(kh[0, -1, 0], v[0, -1, h])) < 1e-14
    t0 = 5
    lg = log_g.copy()
    lg[:, t0, :] = -np.inf
    o, hT = oracle.gdn_sequential(q, k, v, lg, beta, h0, lib=lib)
    o2, hT2 = oracle.gdn_sequential(q[:, t0:], k[:, t0:], v[:, t0:], lg[:, t0:], beta[:, t0:], None,
                                    lib=lib)
    assert np.array_equal(o[:, t0:], o2) and np.array_equal(hT, hT2)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(hT))

def pin_orthonormal_overwrite(lib):
    """k_t = e_t, g = 1, beta = 1: after d steps the state's rows are the v_t."""
    rng = _rng(4)
    d = 6
    T = d
    k = np.zeros((1, T, 1, d))
    for t in range(T):
        k[0, t, 0, t] = 1.0
    q = rng.standard_normal((1, T, 1, d))
    v = rng.standard_normal((1, T, 1, d))
    h0 = rng.standard_normal((1, 1, d, d))
    _, hT = oracle.gdn_sequential(q, k, v, np.zeros((1, T, 1)), np.ones((1, T, 1)), h0, lib=lib)
    assert np.max(np.abs(hT[0, 0] - v[0, :, 0, :])) < 1e-14 * 8


def pin_scalar_recurrence(lib):
    """d = 1: s_t = g (1 - beta) s_{t-1} + beta sign(k) v_t; o_t = s_t sign(q)."""
    rng = _rng(5)
    T = 40
    q, k, v, log_g, beta, h0 = _inputs(rng, 1, T, 1, 1, 1, 1, "qwen")
    o, hT = oracle.gdn_sequential(q, k, v, log_g, beta, h0, q_scale=0.5, lib=lib)
    s = h0[0, 0, 0, 0]
    for t in range(T):
        g = np.exp(log_g[0, t, 0])
        bt = beta[0, t, 0]
        s = g * (1.0 - bt) * s + bt * np.sign(k[0, t, 0, 0]) * v[0, t, 0, 0]
        assert abs(o[0, t, 0, 0] - 0.5 * s * np.sign(q[0, t, 0, 0])) < 1e-14 * max(1, abs(s))
    assert abs(hT[0, 0, 0, 0] - s) < 1e-14 * max(1, abs(s))


def pin_exact_example(lib):
    """A two-step, two-dimensional example worked in exact rational arithmetic.

    k_1 = (3, 4) -> (3/5, 4/5); k_2 = (0, 2) -> (0, 1); q_t = (1, 0) raw;
    g_1 = 1, g_2 = 1/2 (log g = -ln 2), beta = (1/2, 1); S0 = [[1, 2], [0, 1]].
    """
    F = Fraction
    S = [[F(1), F(2)], [F(0), F(1)]]
    ks = [(F(3, 5), F(4, 5)), (F(0), F(1))]
    vs = [(F(1), F(-1)), (F(2), F(3))]
    gs = [F(1), F(1, 2)]
    bs = [F(1, 2), F(1)]
    outs = []
    for t in range(2):
        kk, vv, g, b = ks[t], vs[t], gs[t], bs[t]
        # S <- g (I - b k k^T) S + b k v^T, written entry by entry
        M = [[(1 if i == j else 0) - b * kk[i] * kk[j] for j in range(2)] for i in range(2)]
        S = [[g * sum(M[i][l] * S[l][j] for l in range(2)) + b * kk[i] * vv[j]
              for j in range(2)] for i in range(2)]
        outs.append([S[0][j] for j in range(2)])  # q = e_1 -> o = first row
    q = np.array([[[[1.0, 0.0]], [[1.0, 0.0]]]])
    k = np.array([[[[3.0, 4.0]], [[0.0, 2.0]]]])
    v = np.array([[[[1.0, -1.0]], [[2.0, 3.0]]]])
    log_g = np.array([[[0.0], [-np.log(2.0)]]])
    beta = np.array([[[0.5], [1.0]]])
    h0 = np.array([[[[1.0, 2.0], [0.0, 1.0]]]])
    o, hT = oracle.gdn_sequential(q, k, v, log_g, beta, h0, lib=lib)
    for t in range(2):
        for j in range(2):
            assert abs(o[0, t, 0, j] - float(outs[t][j])) < 1e-14
    for i in range(2):
        for j in range(2):
            assert abs(hT[0, 0, i, j] - float(S[i][j])) < 1e-14


def pin_split_invariance(lib):
    """Carrying the final state across calls changes nothing (bitwise), incl. one token per call."""
    rng = _rng(6)
    B, T, Hk, Hv, d = 2, 23, 1, 3, 5
    q, k, v, log_g, beta, h0 = _inputs(rng, B, T, Hk, Hv, d, d, "qwen")
    o_ref, h_ref = oracle.gdn_sequential(q, k, v, log_g, beta, h0, lib=lib)
    for cuts in ([0, 7, 23], [0, 1, 2, 16, 22, 23], list(range(T + 1))):
        h = h0
        parts = []
        for a, b in zip(cuts[:-1], cuts[1:]):
            o_p, h = oracle.gdn_sequential(q[:, a:b], k[:, a:b], v[:, a:b], log_g[:, a:b],
                                           beta[:, a:b], h, lib=lib)
            parts.append(o_p)
        assert np.array_equal(np.concatenate(parts, axis=1), o_ref)
        assert np.array_equal(h, h_ref)


def pin_linearity(lib):
    """o and S are jointly linear in (S0, V): f(S0, V) = f(S0, 0) + f(0, V)."""
    rng = _rng(7)
    B, T, Hk, Hv, d = 1, 15, 1, 2, 4
    q, k, v, log_g, beta, h0 = _inputs(rng, B, T, Hk, Hv, d, d)
    o, hT = oracle.gdn_sequential(q, k, v, log_g, beta, h0, lib=lib)
    o1, h1 = oracle.gdn_sequential(q, k, np.zeros_like(v), log_g, beta, h0, lib=lib)
    o2, h2 = oracle.gdn_sequential(q, k, v, log_g, beta, None, lib=lib)
    assert _rel(o1 + o2, o) < 1e-12
    assert _rel(h1 + h2, hT) < 1e-12
    o3, h3 = oracle.gdn_sequential(q, k, 3.0 * v, log_g, beta, 3.0 * h0, lib=lib)
    assert _rel(o3, 3.0 * o) < 1e-12 and _rel(h3, 3.0 * hT) < 1e-12


def pin_nonexpansive(lib):
    """beta in [0, 2], g <= 1: ||S_t||_2 <= g ||S_{t-1}||_2 + |beta| ||v_t||."""
    rng = _rng(8)
    T, d = 30, 6
    q, k, v, log_g, _, h0 = _inputs(rng, 1, T, 1, 1, d, d, "qwen")
    beta = rng.uniform(0.0, 2.0, size=(1, T, 1))
    h = 5.0 * h0
    for t in range(T):
        _, h_new = oracle.gdn_sequential(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1],
                                         log_g[:, t:t + 1], beta[:, t:t + 1], h, lib=lib)
        lhs = np.linalg.norm(h_new[0, 0], 2)
        rhs = np.exp(log_g[0, t, 0]) * np.linalg.norm(h[0, 0], 2) + \
            abs(beta[0, t, 0]) * np.linalg.norm(v[0, t, 0])
        assert lhs <= rhs * (1 + 1e-12)
        h = h_new


def pin_gqa_grouping(lib):
    """Value head h reads key head h // (Hv/Hk); other key heads do not touch it."""
    rng = _rng(9)
    B, T, Hk, Hv, d = 1, 8, 2, 4, 5
    q, k, v, log_g, beta, h0 = _inputs(rng, B, T, Hk, Hv, d, d)
    o, hT = oracle.gdn_sequential(q, k, v, log_g, beta, h0, lib=lib)
    q2, k2 = q.copy(), k.copy()
    q2[:, :, 1] = rng.standard_normal(q2[:, :, 1].shape)
    k2[:, :, 1] = rng.standard_normal(k2[:, :, 1].shape)
    o2, h2 = oracle.gdn_sequential(q2, k2, v, log_g, beta, h0, lib=lib)
    assert np.array_equal(o2[:, :, :2], o[:, :, :2]) and np.array_equal(h2[:, :2], hT[:, :2])
    assert not np.allclose(o2[:, :, 2:], o[:, :, 2:])
    # and value heads 0..1 equal a 1:1 run on key head 0 alone
    o3, h3 = oracle.gdn_sequential(q[:, :, :1], k[:, :, :1], v[:, :, :2], log_g[:, :, :2],
                                   beta[:, :, :2], h0[:, :2], lib=lib)
    assert np.array_equal(o3, o[:, :, :2]) and np.array_equal(h3, hT[:, :2])


def pin_normalisation(lib):
    """q, k normalised: power-of-two rescaling is bitwise invisible; zero k writes nothing;
    q_scale scales o only."""
    rng = _rng(10)
    B, T, Hk, Hv, d = 1, 10, 1, 2, 7
    q, k, v, log_g, beta, h0 = _inputs(rng, B, T, Hk, Hv, d, d)
    o, hT = oracle.gdn_sequential(q, k, v, log_g, beta, h0, lib=lib)
    o2, h2 = oracle.gdn_sequential(8.0 * q, 0.25 * k, v, log_g, beta, h0, lib=lib)
    assert np.array_equal(o, o2) and np.array_equal(hT, h2)
    o3, h3 = oracle.gdn_sequential(q, k, v, log_g, beta, h0, q_scale=0.5, lib=lib)
    assert np.array_equal(o3, 0.5 * o) and np.array_equal(h3, hT)
    kz = np.zeros_like(k)
    _, h4 = oracle.gdn_sequential(q, kz, v, log_g, beta, h0, lib=lib)
    G = np.exp(np.sum(log_g[0], axis=0))
    assert _rel(h4[0], G[:, None, None] * h0[0]) < 1e-13


def pin_chunked_equals_sequential(lib):
    """Chunked WY form with direct solve == token-serial form (tiny brute force)."""
    rng = _rng(11)
    cases = [(1, 1, 1, 1, 3), (4, 10, 2, 2, 3), (8, 15, 1, 3, 8), (16, 16, 2, 4, 1),
             (32, 51, 1, 3, 8), (4, 37, 1, 1, 5), (64, 129, 1, 2, 8), (2, 7, 1, 1, 2)]
    for C, T, Hk, Hv, d in cases:
        for gate in ("uniform", "qwen"):
            q, k, v, log_g, beta, h0 = _inputs(rng, 1, T, Hk, Hv, d, d, gate)
            o_s, h_s = oracle.gdn_sequential(q, k, v, log_g, beta, h0, q_scale=0.75, lib=lib)
            o_c, h_c = oracle.gdn_chunked(q, k, v, log_g, beta, h0, chunk=C, q_scale=0.75, lib=lib)
            assert _rel(o_c, o_s) < 1e-12, (C, T, Hk, Hv, d, gate)
            assert _rel(h_c, h_s) < 1e-12, (C, T, Hk, Hv, d, gate)


def pin_triangular_inverse(lib):
    """Forward substitution and Neumann doubling both invert I + A (A strictly lower)."""
    rng = _rng(12)
    for n in (1, 2, 3, 5, 8, 16, 33):
        A = np.tril(rng.standard_normal((n, n)) * 0.3, -1)
        junk = A + np.triu(rng.standard_normal((n, n)))  # upper part must be ignored
        Ti = oracle.unit_lower_inverse(junk, lib=lib)
        Tn = oracle.neumann_inverse(junk, lib=lib)
        I = np.eye(n)
        assert np.max(np.abs(Ti @ (I + A) - I)) < 1e-13
        assert np.max(np.abs(Ti - np.linalg.inv(I + A))) < 1e-12
        assert np.max(np.abs(Tn - Ti)) < 1e-12


def pin_qwen_gates(lib):
    """Closed forms of log g = -exp(A_log) softplus(a + dt_bias) and beta = sigmoid(b)
    ("Qwen3.5 Gated Delta Net NKI Kernel for AWS Neuron", "Correctness Contract")."""
    A_log = np.array([0.0, 0.5, -2.0, 1.0])
    dt_bias = np.array([0.3, -1.0, 2.0, 0.0])
    # a + dt_bias = 0: softplus = ln 2
    a = -dt_bias[None, :].copy()
    b = np.zeros((1, 4))
    lg, bt = oracle.qwen_gates(a, b, A_log, dt_bias, lib=lib)
    assert np.allclose(lg[0], -np.exp(A_log) * np.log(2.0), rtol=1e-15, atol=0)
    assert np.all(bt == 0.5)
    # a + dt_bias = ln(e - 1): softplus = 1, so log g = -exp(A_log)
    a = (np.log(np.e - 1.0) - dt_bias)[None, :]
    b = np.array([[np.log(3.0), -np.log(3.0), 0.0, 0.0]])
    lg, bt = oracle.qwen_gates(a, b, A_log, dt_bias, lib=lib)
    assert np.allclose(lg[0], -np.exp(A_log), rtol=1e-14, atol=0)
    assert np.allclose(bt[0, :2], [0.75, 0.25], rtol=1e-15, atol=0)
    # far tails: softplus(x) -> x (x >> 0) and -> e^x (x << 0); no overflow
    a = np.array([[60.0, -60.0, 800.0, -800.0]]) - dt_bias[None, :]
    b = np.array([[800.0, -800.0, 40.0, -40.0]])
    lg, bt = oracle.qwen_gates(a, b, A_log, dt_bias, lib=lib)
    assert np.allclose(lg[0, [0, 2]], -np.exp(A_log[[0, 2]]) * np.array([60.0, 800.0]), rtol=1e-15)
    assert np.allclose(lg[0, 1], -np.exp(A_log[1]) * np.exp(-60.0), rtol=1e-12)
    assert lg[0, 3] <= 0.0 and lg[0, 3] > -1e-300
    assert bt[0, 0] == 1.0 and 0.0 <= bt[0, 1] < 1e-300
    assert np.isclose(bt[0, 2] + bt[0, 3], 1.0, rtol=0, atol=1e-16)
    # random rows: log g <= 0, decreasing in a; beta in (0, 1), sigma(-b) = 1 - sigma(b)
    rng = np.random.default_rng(7)
    a = rng.standard_normal((50, 4)) * 4
    b = rng.standard_normal((50, 4)) * 4
    lg, bt = oracle.qwen_gates(a, b, A_log, dt_bias, lib=lib)
    lg2, bt2 = oracle.qwen_gates(a + 0.25, -b, A_log, dt_bias, lib=lib)
    assert np.all(lg < 0) and np.all(lg2 < lg)
    assert np.all((bt > 0) & (bt < 1)) and np.allclose(bt + bt2, 1.0, rtol=0, atol=1e-15)
    # matches an independent formulation of softplus (numpy's logaddexp(0, x))
    x = a + dt_bias[None, :]
    assert np.allclose(lg, -np.exp(A_log)[None, :] * np.logaddexp(0.0, x), rtol=1e-14, atol=0)


def _silu(x):
    return x / (1.0 + np.exp(-x))


def pin_conv_closed_forms(lib):
    """Causal conv1d: the identity and pure-delay kernels reproduce the input
    exactly (the delay reads the carried state for the first K-1 tokens);
    a constant input through a full state gives act(bias + c sum w); the
    carried state is the last K-1 inputs, mixing old state and input when
    T < K-1; SiLU at 0, +-1 and 30 against x / (1 + e^-x)."""
    rng = _rng(41)
    for K in (2, 3, 4):
        B, T, C = 2, 9, 5
        x = rng.standard_normal((B, T, C))
        st = rng.standard_normal((B, K - 1, C))
        w = np.zeros((C, K))
        w[:, K - 1] = 1.0
        y, so = oracle.causal_conv1d(x, w, None, st, silu=False, lib=lib)
        assert np.array_equal(y, x) and np.array_equal(so, x[:, T - (K - 1):]), K
        w = np.zeros((C, K))
        w[:, 0] = 1.0
        y, _ = oracle.causal_conv1d(x, w, None, st, silu=False, lib=lib)
        assert np.array_equal(y[:, :K - 1], st) and np.array_equal(y[:, K - 1:], x[:, :T - (K - 1)]), K
        c = 0.37
        w = rng.standard_normal((C, K))
        bias = rng.standard_normal(C)
        y, _ = oracle.causal_conv1d(np.full((B, T, C), c), w, bias, np.full((B, K - 1, C), c),
                                    silu=True, lib=lib)
        z = bias + c * w.sum(axis=1)
        assert np.allclose(y, (z / (1.0 + np.exp(-z)))[None, None, :], rtol=1e-14, atol=1e-15), K
        if K > 2:   # fewer tokens than the carried state
            xs = x[:, :1]
            _, so = oracle.causal_conv1d(xs, w, None, st, silu=False, lib=lib)
            assert np.array_equal(so, np.concatenate([st, xs], axis=1)[:, 1:]), K
    x = np.array([[[0.0], [1.0], [-1.0], [30.0]]])
    w = np.array([[0.0, 0.0, 0.0, 1.0]])
    y, _ = oracle.causal_conv1d(x, w, None, None, silu=True, lib=lib)
    assert np.allclose(y[0, :, 0], [0.0, 1.0 / (1.0 + np.exp(-1.0)), -1.0 / (1.0 + np.e),
                                    30.0 / (1.0 + np.exp(-30.0))], rtol=1e-15, atol=0)


def pin_conv_library_correlation(lib):
    """Every channel against numpy's correlate (an independent routine) over
    the input with its carried prefix, plus the bias."""
    rng = _rng(42)
    B, T, C, K = 2, 23, 4, 4
    x = rng.standard_normal((B, T, C))
    st = rng.standard_normal((B, K - 1, C))
    w = rng.standard_normal((C, K))
    bias = rng.standard_normal(C)
    y, _ = oracle.causal_conv1d(x, w, bias, st, silu=False, lib=lib)
    for b in range(B):
        for c in range(C):
            u = np.concatenate([st[b, :, c], x[b, :, c]])
            ref = np.correlate(u, w[c], mode="valid") + bias[c]
            assert np.allclose(y[b, :, c], ref, rtol=1e-13, atol=1e-13), (b, c)


def pin_conv_split_and_linearity(lib):
    """Carrying the state across calls gives bitwise one call's result (any
    split, one token per call included); without the activation the
    convolution is linear in (input, state)."""
    rng = _rng(43)
    B, T, C, K = 2, 17, 6, 4
    x = rng.standard_normal((B, T, C))
    st0 = rng.standard_normal((B, K - 1, C))
    w = rng.standard_normal((C, K))
    bias = rng.standard_normal(C)
    y1, s1 = oracle.causal_conv1d(x, w, bias, st0, silu=True, lib=lib)
    for splits in ([5, 12], [1] * T, [2, 1, 14]):
        st, ys, t0 = st0, [], 0
        for n in splits:
            y, st = oracle.causal_conv1d(x[:, t0:t0 + n], w, bias, st, silu=True, lib=lib)
            ys.append(y)
            t0 += n
        assert np.array_equal(np.concatenate(ys, axis=1), y1) and np.array_equal(st, s1), splits
    x2 = rng.standard_normal((B, T, C))
    st2 = rng.standard_normal((B, K - 1, C))
    a, b = 0.7, -1.3
    ya, _ = oracle.causal_conv1d(x, w, None, st0, silu=False, lib=lib)
    yb, _ = oracle.causal_conv1d(x2, w, None, st2, silu=False, lib=lib)
    yab, _ = oracle.causal_conv1d(a * x + b * x2, w, None, a * st0 + b * st2, silu=False, lib=lib)
    assert np.allclose(yab, a * ya + b * yb, rtol=1e-12, atol=1e-12)


def pin_rmsnorm_closed_forms(lib):
    """Gated RMS norm: a constant row normalises to its sign; a row of +-1
    (unit RMS) passes through times w * silu(z); z = 0 gives zero; [3, 4]
    has RMS sqrt(12.5); scaling a row leaves it unchanged (eps = 0); a zero
    row stays zero for eps > 0; no gate when z is None."""
    rng = _rng(44)
    D = 8
    w = rng.uniform(0.5, 1.5, D)
    x = np.array([[-2.5] * D, [4.0] * D])
    y = oracle.gated_rmsnorm(x, None, np.ones(D), eps=0.0, lib=lib)
    assert np.allclose(y, np.sign(x), rtol=1e-15, atol=0)
    x = rng.choice([-1.0, 1.0], size=(3, D))
    z = rng.standard_normal((3, D))
    y = oracle.gated_rmsnorm(x, z, w, eps=0.0, lib=lib)
    assert np.allclose(y, x * w * z / (1.0 + np.exp(-z)), rtol=1e-14, atol=0)
    assert np.array_equal(oracle.gated_rmsnorm(x, np.zeros_like(z), w, eps=1e-6, lib=lib),
                          np.zeros_like(x))
    y = oracle.gated_rmsnorm(np.array([[3.0, 4.0]]), None, np.ones(2), eps=0.0, lib=lib)
    assert np.allclose(y, [[3.0 / np.sqrt(12.5), 4.0 / np.sqrt(12.5)]], rtol=1e-15, atol=0)
    x = rng.standard_normal((4, D))
    z = rng.standard_normal((4, D))
    assert np.allclose(oracle.gated_rmsnorm(37.0 * x, z, w, eps=0.0, lib=lib),
                       oracle.gated_rmsnorm(x, z, w, eps=0.0, lib=lib), rtol=1e-13, atol=0)
    assert np.array_equal(oracle.gated_rmsnorm(np.zeros((2, D)), None, w, eps=1e-6, lib=lib),
                          np.zeros((2, D)))
    # eps enters under the root: a row of RMS r reads r / sqrt(r^2 + eps)
    y = oracle.gated_rmsnorm(np.full((1, D), 0.01), None, np.ones(D), eps=1e-4, lib=lib)
    assert np.allclose(y, 0.01 / np.sqrt(1e-4 + 1e-4), rtol=1e-14, atol=0)


PINS = [
    pin_identity_plumbing,
    pin_matrix_form,
    pin_unit_key_readback,
    pin_no_write_closed_form,
    pin_closed_gate,
    pin_orthonormal_overwrite,
    pin_scalar_recurrence,
    pin_exact_example,
    pin_split_invariance,
    pin_linearity,
    pin_nonexpansive,
    pin_gqa_grouping,
    pin_normalisation,
    pin_chunked_equals_sequential,
    pin_triangular_inverse,
    pin_qwen_gates,
    pin_conv_closed_forms,
    pin_conv_library_correlation,
    pin_conv_split_and_linearity,
    pin_rmsnorm_closed_forms,
]
