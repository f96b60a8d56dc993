"""Plant plausible mistakes in copies of the oracle and check that a pin catches each.

Every mutant is a textual edit of oracle/gdn_oracle.c compiled into a
temporary directory (CPU only).  The real oracle is never modified.
"""
import os

import pytest

import oracle
from oracle_pins import PINS

MUTANTS = {
    "no_decay": [("S[i * dv + j] *= g;", "S[i * dv + j] *= 1.0;")],
    "exp_linearised": [("const double g = exp(J->log_g[g_off]);",
                        "const double g = 1.0 + J->log_g[g_off];")],
    "delta_sign": [("delta[j] = bt * (J->v[v_off + j] - a[j]);",
                    "delta[j] = bt * (a[j] - J->v[v_off + j]);")],
    "delta_no_beta": [("delta[j] = bt * (J->v[v_off + j] - a[j]);",
                       "delta[j] = (J->v[v_off + j] - a[j]);")],
    "read_transposed": [("for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * kh[i];",
                         "for (int i = 0; i < dk; ++i) acc += S[j * dv + i] * kh[i];")],
    "output_from_old_state": [
        ("            /* 4. write: S += k delta^T */\n"
         "            for (int i = 0; i < dk; ++i)\n"
         "                for (int j = 0; j < dv; ++j) S[i * dv + j] += kh[i] * delta[j];\n", ""),
        ("                J->o[v_off + j] = J->q_scale * acc;\n            }\n",
         "                J->o[v_off + j] = J->q_scale * acc;\n            }\n"
         "            for (int i = 0; i < dk; ++i)\n"
         "                for (int j = 0; j < dv; ++j) S[i * dv + j] += kh[i] * delta[j];\n")],
    "decay_after_read": [
        ("            /* 1. decay */\n"
         "            for (int i = 0; i < dk; ++i)\n"
         "                for (int j = 0; j < dv; ++j) S[i * dv + j] *= g;\n", ""),
        ("            /* 3. delta = beta (v - a) */\n",
         "            for (int i = 0; i < dk; ++i)\n"
         "                for (int j = 0; j < dv; ++j) S[i * dv + j] *= g;\n"
         "            /* 3. delta = beta (v - a) */\n")],
    "gqa_interleaved": [("        const int hk = h / r;\n        const size_t state_off",
                         "        const int hk = h % Hk;\n        const size_t state_off")],
    "q_not_normalised": [("normalise(J->q + qk_off, dk, J->qk_l2norm, qh);",
                          "normalise(J->q + qk_off, dk, 0, qh);")],
    "q_scale_ignored": [("J->o[v_off + j] = J->q_scale * acc;", "J->o[v_off + j] = acc;")],
    "norm_without_sqrt": [("double nrm = sqrt(ss);", "double nrm = ss;")],
    "state_not_carried": [("        if (J->h0)\n            memcpy(S, J->h0 + state_off",
                           "        if (0)\n            memcpy(S, J->h0 + state_off")],
    "chunk_mask_without_decay": [("val = br * exp(gam[rr] - gam[s]) * dot;", "val = br * dot;")],
    "chunk_solve_off_by_one": [("for (int s = 0; s < rr; ++s) {\n                        const double ars",
                                "for (int s = 0; s + 1 < rr; ++s) {\n                        const double ars")],
    "chunk_handoff_no_decay": [("double acc = GL * S[(size_t)i * dv + j];",
                                "double acc = S[(size_t)i * dv + j];")],
    "chunk_output_strict_mask": [("for (int s = 0; s <= rr; ++s) {\n                            double dot",
                                  "for (int s = 0; s < rr; ++s) {\n                            double dot")],
    "tri_inverse_sign": [("Tinv[i * n + c] -= aij * Tinv[j * n + c];",
                          "Tinv[i * n + c] += aij * Tinv[j * n + c];")],
    "gate_no_dt_bias": [("softplus(a[e] + dt_bias[h])", "softplus(a[e])")],
    "gate_A_log_not_exponentiated": [("-exp(A_log[h]) * softplus", "-A_log[h] * softplus")],
    "gate_softplus_overflow_branch": [("return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));",
                                       "return log1p(exp(x));")],
    "gate_beta_sign": [("beta[e] = 1.0 / (1.0 + exp(-b[e]));", "beta[e] = 1.0 / (1.0 + exp(b[e]));")],
    "neumann_one_factor_short": [("for (int span = 1; span < n; span *= 2) {",
                                  "for (int span = 2; span < n; span *= 2) {")],
    "conv_kernel_reversed": [("acc += w[(size_t)c * K + j] * u[(size_t)(t + j) * C + c];",
                              "acc += w[(size_t)c * K + (K - 1 - j)] * u[(size_t)(t + j) * C + c];")],
    "conv_no_activation": [("y[((size_t)b * T + t) * C + c] = silu_on ? silu(acc) : acc;",
                            "y[((size_t)b * T + t) * C + c] = acc;")],
    "conv_state_not_carried": [("u[(size_t)i * C + c] = state_in ? state_in[((size_t)b * P + i) * C + c] : 0.0;",
                                "u[(size_t)i * C + c] = 0.0;")],
    "conv_state_out_shifted": [("state_out[((size_t)b * P + i) * C + c] = u[(size_t)(T + i) * C + c];",
                                "state_out[((size_t)b * P + i) * C + c] = u[(size_t)(T - 1 + i) * C + c];")],
    "conv_bias_dropped": [("double acc = bias ? bias[c] : 0.0;", "double acc = 0.0;")],
    "silu_sign": [("static double silu(double x) { return x / (1.0 + exp(-x)); }",
                   "static double silu(double x) { return x / (1.0 + exp(x)); }")],
    "rmsnorm_sum_not_mean": [("const double inv = 1.0 / sqrt(ss / D + eps);",
                              "const double inv = 1.0 / sqrt(ss + eps);")],
    "rmsnorm_eps_outside_root": [("const double inv = 1.0 / sqrt(ss / D + eps);",
                                  "const double inv = 1.0 / (sqrt(ss / D) + eps);")],
    "rmsnorm_gate_ignored": [("const double g = z ? silu(z[r * D + i]) : 1.0;", "const double g = 1.0;")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, oracle_lib):
    with open(oracle.SOURCE) as f:
        src = f.read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
        src = src.replace(old, new)
    path = tmp_path / "gdn_oracle.c"
    path.write_text(src)
    lib_path = oracle.build(str(path), str(tmp_path / f"liboracle_{name}.so"))
    lib = oracle.load(lib_path)
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"
    print(f"{name}: caught by {', '.join(caught)}")
    os.remove(lib_path)
