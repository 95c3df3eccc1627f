"""Plant plausible mistakes in a copy of the oracle source (on the CPU) and check that every one of
them fails at least one pin: evidence that the pins would catch such a mistake in the oracle."""
import os
import shutil

import pytest

import oracle
from oracle.build import build
from pins import PINS

SRC = open(oracle.SRC).read()

# (name, exact text in oracle.c, replacement)
MUTANTS = [
    ("recurrent_no_decay", "Si[j - j0] = g * Si[j - j0] + kn[i] * vn[j];", "Si[j - j0] = Si[j - j0] + kn[i] * vn[j];"),
    ("recurrent_read_before_update",
     "for (int j = j0; j < j1; ++j) Si[j - j0] = g * Si[j - j0] + kn[i] * vn[j];\n                if (on)\n"
     "                    for (int j = j0; j < j1; ++j) on[j] += qn[i] * Si[j - j0];",
     "if (on)\n                    for (int j = j0; j < j1; ++j) on[j] += qn[i] * Si[j - j0];\n"
     "                for (int j = j0; j < j1; ++j) Si[j - j0] = g * Si[j - j0] + kn[i] * vn[j];"),
    ("recurrent_state_in_transposed", "state_in[((size_t)bh * dk + i) * dv + j]", "state_in[((size_t)bh * dv + j) * dk + i]"),
    ("recurrent_k_q_swapped_roles", "on[j] += qn[i] * Si[j - j0];", "on[j] += kn[i] * Si[j - j0];"),
    ("parallel_no_diagonal", "for (int m = 0; m <= n; ++m)", "for (int m = 0; m < n; ++m)"),
    ("parallel_decay_sign", "pow(g, (double)(n - m))", "pow(g, (double)(m - n))"),
    ("parallel_wrong_key_index", "const double* km = k + ((size_t)bh * N + m) * dk;",
     "const double* km = k + ((size_t)bh * N + n) * dk;"),
    ("chunk_xi_off_by_one", "pow(g, (double)(j + 1))", "pow(g, (double)j)"),
    ("chunk_zeta_off_by_one", "pow(g, (double)(L - 1 - t))", "pow(g, (double)(L - t))"),
    ("chunk_decay_uses_C_for_tail", "const double gL = pow(g, (double)L);", "const double gL = pow(g, (double)C);"),
    ("chunk_intra_no_diagonal", "for (int t = 0; t <= j; ++t)", "for (int t = 0; t < j; ++t)"),
    ("chunk_intra_decay_sign", "pow(g, (double)(j - t))", "pow(g, (double)(t - j))"),
    ("chunk_ignores_state_in", "if (state_in) memcpy(R,", "if (0) memcpy(R,"),
    ("chunk_cross_term_dropped", "oj[col] += xi * qj[i] * Ri[col];", "oj[col] += 0.0 * xi * qj[i] * Ri[col];"),
    ("groupnorm_unbiased_variance", "var /= dv;", "var /= (dv - 1);"),
    ("groupnorm_eps_outside_sqrt", "1.0 / sqrt(var + eps)", "1.0 / (sqrt(var) + eps)"),
    ("groupnorm_wrong_head_index", "const int h = (int)((r / N) % H);", "const int h = (int)(r % H);"),
    ("groupnorm_bias_not_added", "yr[c] = (xr[c] - mu) * inv * w + b;", "yr[c] = (xr[c] - mu) * inv * w;"),
    ("bwd_dual_no_decay", "U[(size_t)i * dv + j] = g * U[(size_t)i * dv + j] + qn[i] * gn[j];",
     "U[(size_t)i * dv + j] = U[(size_t)i * dv + j] + qn[i] * gn[j];"),
    ("bwd_dstate_no_gamma", "dstate_in[(size_t)bh * dk * dv + e] = g * U[e];", "dstate_in[(size_t)bh * dk * dv + e] = U[e];"),
    ("bwd_dk_uses_dout", "a += U[(size_t)i * dv + j] * vn[j];", "a += U[(size_t)i * dv + j] * gn[j];"),
    ("bwd_dv_uses_q", "a += kn[i] * U[(size_t)i * dv + j];", "a += qn[i] * U[(size_t)i * dv + j];"),
    ("bwd_dq_ignores_state_in", "S[e] = state_in ? state_in[(size_t)bh * dk * dv + e] : 0.0;\n        for (int n = 0; n < N; ++n) {",
     "S[e] = 0.0;\n        for (int n = 0; n < N; ++n) {"),
    ("gate_sigmoid_not_swish", "yr[c] *= g / (1.0 + exp(-g));", "yr[c] *= 1.0 / (1.0 + exp(-g));"),
    ("gate_sigmoid_sign", "yr[c] *= g / (1.0 + exp(-g));", "yr[c] *= g / (1.0 + exp(g));"),
    ("gate_wrong_index", "const double g = gate[(size_t)r * dv + c];", "const double g = gate[c];"),
    ("gate_before_bias", "yr[c] = (xr[c] - mu) * inv * w + b;\n            if (gate) {\n                const double g = gate[(size_t)r * dv + c];\n                yr[c] *= g / (1.0 + exp(-g));",
     "yr[c] = (xr[c] - mu) * inv * w;\n            if (gate) {\n                const double g = gate[(size_t)r * dv + c];\n                yr[c] *= g / (1.0 + exp(-g));\n            }\n            yr[c] += b;\n            {"),
    ("rot_sin_sign_first", "yn[2 * i] = a * c - b * s;", "yn[2 * i] = a * c + b * s;"),
    ("rot_turns_backwards", "yn[2 * i] = a * c - b * s;\n                yn[2 * i + 1] = a * s + b * c;",
     "yn[2 * i] = a * c + b * s;\n                yn[2 * i + 1] = -a * s + b * c;"),
    ("rot_theta_exponent_halved", "pow(base, -2.0 * i / d)", "pow(base, -1.0 * i / d)"),
    ("rot_theta_per_feature_count", "pow(base, -2.0 * i / d)", "pow(base, -2.0 * i / (d - 2 > 0 ? d - 2 : 1))"),
    ("rot_ignores_offset", "(double)(offset + n)", "(double)(n)"),
    ("rot_position_one_based", "(double)(offset + n)", "(double)(offset + n + 1)"),
    ("rot_half_split_pairs", "const double a = xn[2 * i], b = xn[2 * i + 1];\n                yn[2 * i] = a * c - b * s;\n                yn[2 * i + 1] = a * s + b * c;",
     "const double a = xn[i], b = xn[i + d / 2];\n                yn[i] = a * c - b * s;\n                yn[i + d / 2] = a * s + b * c;"),
    ("rot_inverse_not_negated", "(direction < 0 ? -1.0 : 1.0)", "1.0"),
    ("rla_reads_one_token_late", "const int p = t - P;", "const int p = t - P + 1;"),
    ("rla_reads_one_token_early", "const int p = t - P;", "const int p = t - P - 1;"),
    ("rla_softmax_unnormalised", "for (int i = 0; i < d; ++i) y[i] /= s;", "(void)s;"),
    ("rla_softmax_sign", "y[i] = exp(x[i] - m);", "y[i] = exp(m - x[i]);"),
    ("rla_q_not_mapped", "rla_phi(fmap, dk, q + ((size_t)bh * N + t) * dk, fq);",
     "rla_phi(0, dk, q + ((size_t)bh * N + t) * dk, fq);"),
    ("rla_k_not_mapped", "rla_phi(fmap, dk, kt, fk);", "rla_phi(0, dk, kt, fk);"),
    ("rla_prev_window_ignored", "if (kp && p >= -prev_len) {", "if (0) {"),
    ("rla_prev_len_ignored", "if (kp && p >= -prev_len) {", "if (kp) {"),
    ("rla_prev_rows_reversed", "kt = kp + ((size_t)bh * P + (p + P)) * dk;", "kt = kp + ((size_t)bh * P + (-1 - p)) * dk;"),
    ("rla_ignores_state_in", "S[e] = state_in ? state_in[(size_t)bh * dk * dv + e] : 0.0;\n        for (int t = 0; t < N; ++t) {",
     "S[e] = 0.0;\n        for (int t = 0; t < N; ++t) {"),
]


def _fails_some_pin(orc):
    for pin in PINS:
        try:
            pin(orc)
        except AssertionError:
            return pin.__name__
    return None


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    assert SRC.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    src = tmp_path / "oracle_mut.c"
    src.write_text(SRC.replace(old, new))
    lib = build(str(src), str(tmp_path / "liboracle_mut.so"), quiet=True)
    orc = oracle.Oracle(oracle.load(lib))
    caught = _fails_some_pin(orc)
    assert caught is not None, f"planted mistake {name} passed every pin"
