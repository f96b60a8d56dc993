"""The direct / Neumann solve study (tests/solve_study.py) on the CPU: the direct
solves stay at rounding level for every gate and key regime of the 27B law,
while Neumann power doubling breaks down once keys are correlated -- the
instability "Qwen3.6: Fused DeltaNet Direct-Solve Follow-Up" reports ("Why This
Exists", "Implementation Details")."""
import solve_study as S


def test_direct_solves_stable_neumann_not():
    rows = {(r["cos"], r["beta_hi"]): r for r in S.study(trials=8, seed=1)}
    for r in rows.values():
        assert r["direct_fp32_max"] < 1e-6, r              # fp32 rounding level
        assert r["blocked_bf16_max"] < 4e-3, r             # bf16 operand rounding level
    # uncorrelated keys: A is small and every solve agrees
    assert rows[(0.0, False)]["neumann_fp32_max"] < 1e-6
    # correlated keys: the powers of A blow up and Neumann loses all accuracy,
    # already in fp32 and far worse with bf16 operands
    bad = rows[(0.9, True)]
    assert bad["power_growth"] > 1e6
    assert bad["neumann_fp32_max"] > 1e-2 and bad["neumann_bf16_max"] > 1.0
    assert bad["neumann_bf16_max"] > 1e3 * bad["blocked_bf16_max"]


def test_solve_costs():
    f = S.flop_counts()
    assert f["direct"] == 64 * 63 * 65 // 6
    assert f["neumann (dense products)"] > 30 * f["direct"]   # the price of log depth
    assert f["neumann dependent steps"] == 12 and f["direct dependent steps"] == 63


def test_bf16_rounding_helper():
    import numpy as np
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0], dtype=np.float32)
    y = S.bf16(x)
    assert list(y) == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 0.0]   # ties to even
