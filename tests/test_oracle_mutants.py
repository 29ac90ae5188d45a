"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is a one-spot textual edit of oracle/dlrm_oracle.c (a dropped
term, a wrong sign, index or operand, a wrong loop bound or order), compiled
with gcc into a temporary library and run through the whole pin battery on
the CPU.  This shows the pins can tell a wrong oracle from a right one.
"""
import os

import pytest

import oracle
import pins

MUTANTS = {
    "embbag_keeps_last_row_only": [("o[d] += (double)row[d];", "o[d] = (double)row[d];")],
    "embbag_last_bag_empty": [("*e = (b + 1 < B) ? off[b + 1] : n_idx;", "*e = (b + 1 < B) ? off[b + 1] : off[b];")],
    "embbag_skips_first_index": [("for (int64_t k = s; k < e; ++k) {\n                const float* row = W[t] + idx[t][k]",
                                  "for (int64_t k = s + (e > s); k < e; ++k) {\n                const float* row = W[t] + idx[t][k]")],
    "interact_squares_left_vector": [("acc += u[d] * v[d];\n                Z", "acc += u[d] * u[d];\n                Z")],
    "interact_reversed_pair_order": [("Z[b * ldz + p] = acc;", "Z[b * ldz + (P - 1 - p)] = acc;")],
    "interact_drops_last_feature": [("for (int32_t i = 1; i < F; ++i) {\n            for (int32_t j = 0; j < i; ++j) {\n                const double* u",
                                     "for (int32_t i = 1; i < F; ++i) {\n            for (int32_t j = 0; j < i; ++j) {\n                if (i == F - 1) { Z[b * ldz + p] = 0.0; ++p; continue; }\n                const double* u")],
    "interact_x_from_wrong_table": [("if (f == 0) return x + b * ldx;", "if (f == 0) return E + b * T * (int64_t)D;")],
    "closed_form_missing_one": [("int64_t i = (1 + isqrt_floor(1 + 8 * p)) / 2;", "int64_t i = (1 + isqrt_floor(8 * p)) / 2;")],
    "linear_transposed_weight": [("a += x[m * ldx + k] * (double)W[n * K + k];", "a += x[m * ldx + k] * (double)W[(k * N + n) % (N * K)];")],
    "linear_drops_bias": [("double a = bias ? (double)bias[n] : 0.0;", "double a = 0.0;")],
    "relu_wrong_sign": [("a = a > 0.0 ? a : 0.0;", "a = a < 0.0 ? a : 0.0;")],
    "sigmoid_wrong_sign": [("a = 1.0 / (1.0 + exp(-a));", "a = 1.0 / (1.0 + exp(a));")],
    "no_relu_on_last_bottom_layer": [("m->bot_w[l], m->bot_b[l], ORACLE_ACT_RELU", "m->bot_w[l], m->bot_b[l], (l + 2 == m->n_bot) ? ORACLE_ACT_NONE : ORACLE_ACT_RELU")],
    "r_is_z_then_x": [("h1[b * wr + d] = h0[b * D + d];", "h1[b * wr + P + d] = h0[b * D + d];"),
                      ("h1[b * wr + D + p] = Z[b * P + p];", "h1[b * wr + p] = Z[b * P + p];")],
    "top_last_layer_relu": [("last ? ORACLE_ACT_SIGMOID : ORACLE_ACT_RELU", "ORACLE_ACT_RELU")],
    "validate_ignores_pair_count": [("if (m->ln_top[0] != m->D + oracle_n_pairs(m->T + 1)) return ORACLE_E_SHAPE;", "")],
    "bag_mean_counts_padding": [("if (pad && pad[t] >= 0 && r == pad[t]) continue;",
                                 "if (pad && pad[t] >= 0 && r == pad[t]) { ++count; continue; }")],
    "bag_max_keeps_first_row": [("if (mode == 2) o[d] = (count == 0 || v > o[d]) ? v : o[d];",
                                 "if (mode == 2) o[d] = (count == 0) ? v : o[d];")],
    "bag_ignores_sample_weights": [("const double w = psw ? (double)psw[t][k] : 1.0;", "const double w = 1.0;")],
    "bag_ignores_last_offset": [("            const int64_t e = include_last_offset ? off[t][b + 1] : ((b + 1 < B) ? off[t][b + 1] : n_idx[t]);",
                                 "            const int64_t e = (b + 1 < B) ? off[t][b + 1] : n_idx[t];")],
    "pair_count_off_by_one": [("return n_feat * (n_feat - 1) / 2;", "return n_feat * (n_feat + 1) / 2 - n_feat + (n_feat > 40);")],
}


def _build_mutant(name, edits, tmp_path):
    src = open(oracle.SOURCE).read()
    for old, new in edits:
        assert src.count(old) == 1, f"mutant {name}: pattern not unique/found: {old!r}"
        src = src.replace(old, new)
    path = tmp_path / f"{name}.c"
    path.write_text(src)
    lib = str(tmp_path / f"lib_{name}.so")
    oracle.compile_library(str(path), lib)
    return oracle.Oracle(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    o = _build_mutant(name, MUTANTS[name], tmp_path)
    o.set_threads(2)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, oracle.OracleError, ValueError) as e:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
