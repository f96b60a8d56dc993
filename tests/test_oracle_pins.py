"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle_pins import PINS, _inputs


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


# Chunked == sequential over the seq-len sweep the model card's parity table
# uses (2, 10, 15, 16, 51, 100, 127, 129, 200) plus 1, chunk sizes 1..64,
# GQA ratios 1, 2 (as 2:4) and 3, head dims 1, 3, 8, 64.
_T = [1, 2, 10, 15, 16, 51, 100, 127, 129, 200]
_C = [1, 2, 4, 8, 16, 32, 64]
_H = [(1, 1), (2, 2), (1, 3), (2, 4)]


@pytest.mark.parametrize("d", [1, 3, 8])
@pytest.mark.parametrize("heads", _H, ids=[f"{a}x{b}" for a, b in _H])
def test_chunked_equals_sequential_grid(d, heads, oracle_lib):
    Hk, Hv = heads
    rng = np.random.default_rng(1000 + 10 * d + Hv)
    for T in _T:
        q, k, v, log_g, beta, h0 = _inputs(rng, 1, T, Hk, Hv, d, d, "qwen" if T % 2 else "uniform")
        o_s, h_s = oracle.gdn_sequential(q, k, v, log_g, beta, h0, lib=oracle_lib)
        for C in _C:
            o_c, h_c = oracle.gdn_chunked(q, k, v, log_g, beta, h0, chunk=C, lib=oracle_lib)
            den_o = max(np.linalg.norm(o_s), 1e-300)
            assert np.linalg.norm(o_c - o_s) / den_o < 1e-12, (T, C)
            assert np.linalg.norm(h_c - h_s) / np.linalg.norm(h_s) < 1e-12, (T, C)


@pytest.mark.parametrize("C,T", [(16, 51), (32, 129), (64, 200), (64, 127)])
def test_chunked_equals_sequential_d64(C, T, oracle_lib):
    rng = np.random.default_rng(77 + C + T)
    q, k, v, log_g, beta, h0 = _inputs(rng, 1, T, 1, 3, 64, 64, "qwen")
    o_s, h_s = oracle.gdn_sequential(q, k, v, log_g, beta, h0, lib=oracle_lib)
    o_c, h_c = oracle.gdn_chunked(q, k, v, log_g, beta, h0, chunk=C, lib=oracle_lib)
    assert np.linalg.norm(o_c - o_s) / np.linalg.norm(o_s) < 1e-12
    assert np.linalg.norm(h_c - h_s) / np.linalg.norm(h_s) < 1e-12


def test_threads_do_not_change_results(oracle_lib):
    rng = np.random.default_rng(5)
    q, k, v, log_g, beta, h0 = _inputs(rng, 2, 33, 2, 6, 8, 8, "qwen")
    a = oracle.gdn_sequential(q, k, v, log_g, beta, h0, nthreads=1, lib=oracle_lib)
    b = oracle.gdn_sequential(q, k, v, log_g, beta, h0, nthreads=5, lib=oracle_lib)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_empty_and_degenerate(oracle_lib):
    rng = np.random.default_rng(6)
    q, k, v, log_g, beta, h0 = _inputs(rng, 1, 0, 1, 2, 4, 4)
    o, hT = oracle.gdn_sequential(q, k, v, log_g, beta, h0, lib=oracle_lib)
    assert o.shape == (1, 0, 2, 4) and np.array_equal(hT, h0)
    o, hT = oracle.gdn_sequential(q, k, v, log_g, beta, None, lib=oracle_lib)
    assert np.array_equal(hT, np.zeros_like(h0))
    # zero batch
    q, k, v, log_g, beta, h0 = _inputs(rng, 0, 5, 1, 2, 4, 4)
    o, hT = oracle.gdn_sequential(q, k, v, log_g, beta, h0, lib=oracle_lib)
    assert o.shape == (0, 5, 2, 4) and hT.shape == (0, 2, 4, 4)


def test_bad_gqa_ratio_rejected(oracle_lib):
    rng = np.random.default_rng(7)
    q, k, v, log_g, beta, _ = _inputs(rng, 1, 3, 2, 3, 4, 4)
    with pytest.raises(ValueError):
        oracle.gdn_sequential(q, k, v, log_g, beta, None, lib=oracle_lib)

