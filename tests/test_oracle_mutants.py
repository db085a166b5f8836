"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of the oracle's C source (on the CPU),
builds it, routes the oracle's Python wrapper through that build and runs the
pin tests: at least one pin must fail.  A mutant that survives means the pins
leave that part of the oracle unchecked.
"""
import subprocess
from pathlib import Path

import pytest

import oracle
import test_oracle_pins as pins
import test_oracle_overlap as ovl
import test_oracle_tree as tree
import test_oracle_typical as typ
import test_oracle_stats as stats

SRC = Path(oracle.__file__).resolve().parent / "spec_verify_ref.c"

# (name, original text, planted mistake)
MUTANTS = [
    ("strict_acceptance", "accept = (u <= alpha);", "accept = (u < alpha);"),
    ("ratio_inverted", "exp(fmin(0.0, log_px - log_qx))", "exp(fmin(0.0, log_qx - log_px))"),
    ("no_positive_part", "W[v] = fmax(P[v] - Q[v], 0.0);", "W[v] = P[v] - Q[v];"),
    ("residual_sign", "W[v] = fmax(P[v] - Q[v], 0.0);", "W[v] = fmax(Q[v] - P[v], 0.0);"),
    ("correct_from_p", "int y = ref_invcdf(W, V,", "int y = ref_invcdf(P, V,"),
    ("bonus_from_draft_row", "load_row(J->target, J->dtype, trow0 + G, V, zt);",
     "load_row(J->draft, J->dtype, drow0 + G - 1, V, zt);"),
    ("draft_row_shifted", "load_row(J->draft, J->dtype, drow0 + i, V, zd);\n    double logZp",
     "load_row(J->draft, J->dtype, drow0 + (i + 1) % G, V, zd);\n    double logZp"),
    ("cdf_closed_interval", "if (F > t) {", "if (F >= t) {"),
    ("temperature_multiplies", "double e = kept ? exp(z[v] / T - m) : 0.0;",
     "double e = kept ? exp(z[v] * T - m * T * T) : 0.0;"),
    ("topk_drops_ties", "int kept = (z[v] >= tau) && (z[v] > -INFINITY);\n    double e",
     "int kept = (z[v] > tau || v == 0) && (z[v] > -INFINITY);\n    double e"),
    ("topk_off_by_one", "double tau = tmp[k - 1];", "double tau = tmp[k];"),
    ("argmax_highest_index", "if (z[v] > z[a]) a = v;", "if (z[v] >= z[a]) a = v;"),
    ("uniform_closed", "float u = J->u_accept[(size_t)b * G + i];\n      if (!(u >= 0.0f && u < 1.0f))",
     "float u = J->u_accept[(size_t)b * G + i];\n      if (!(u >= 0.0f && u <= 1.0f))"),
    ("no_p_support_test", "accept = 0; /* p(x) = 0", "accept = (u <= 1.0); /* p(x) = 0"),
    ("greedy_keeps_draft_token", "out[i] = a; /* greedy correction", "out[i] = x[i]; /* greedy correction"),
    ("no_padding", "fill_tokens(out + i + 1, G - i, -1);\n    return;\n  }\n\n  /* Every",
     "return;\n  }\n\n  /* Every"),
    ("accept_len_off_by_one", "J->accepted_len[b] = i;\n    fill_tokens(out + i + 1, G - i, -1);\n    return;\n  }\n\n  /* Every",
     "J->accepted_len[b] = i + 1;\n    fill_tokens(out + i + 1, G - i, -1);\n    return;\n  }\n\n  /* Every"),
    ("overlap_max_for_min", "sb += fmin(P[v], Q[v]);", "sb += fmax(P[v], Q[v]);"),
    ("overlap_tv_absolute", "st += fmax(P[v] - Q[v], 0.0);", "st += fabs(P[v] - Q[v]);"),
    ("overlap_target_stride", "load_row(target, dtype, (size_t)b * target_rows + i, V, zt);",
     "load_row(target, dtype, (size_t)b * G + i, V, zt);"),
    ("overlap_next_draft_row", "load_row(draft, dtype, (size_t)b * G + i, V, zd);",
     "load_row(draft, dtype, (size_t)b * G + (i + 1) % G, V, zd);"),
    ("overlap_topk_target_only", "policy(zd, V, temperature, top_k, NULL, Q);",
     "policy(zd, V, temperature, 0, NULL, Q);"),
    ("overlap_draft_unscaled", "policy(zd, V, temperature, top_k, NULL, Q);",
     "policy(zd, V, 1.0, top_k, NULL, Q);"),
    ("overlap_skips_draft_check", "if (!row_is_valid(zt, V) || !row_is_valid(zd, V)) {",
     "if (!row_is_valid(zt, V)) {"),
    ("tree_naive_siblings", "for (int v = 0; v < V; ++v) cur[v] = fmax(cur[v] - Q[v], 0.0) / Z;",
     "for (int v = 0; v < V; ++v) cur[v] = P[v];"),
    ("tree_first_child_only", "if (par[s] != u) continue;\n          const int xs", "if (par[s] != u || rejected) continue;\n          const int xs"),
    ("tree_parent_row", "load_row(target, dtype, row0 + u, V, zt);\n        if (greedy)",
     "load_row(target, dtype, row0 + (u ? par[u] : 0), V, zt);\n        if (greedy)"),
    ("tree_draw_from_p", "out[depth] = ref_invcdf(cur, V,", "out[depth] = ref_invcdf(P, V,"),
    ("tree_greedy_last_match", "for (int s = u + 1; s < N && next < 0; ++s)\n            if (par[s] == u && x[s] == a) next = s;",
     "for (int s = u + 1; s < N; ++s)\n            if (par[s] == u && x[s] == a) next = s;"),
    ("tree_uniform_index", "const double us = (double)u_accept[row0 + s];", "const double us = (double)u_accept[row0 + s - 1];"),
    ("tree_leaf_draft_checked", "if (!nchild[n]) continue;\n          load_row(draft", "load_row(draft"),
    ("r4_no_fallback", "if (y < 0) y = ref_invcdf(P, V, (double)J->u_sample[b], &d); /* R4 */",
     "/* no fallback */"),
    ("r4_fallback_accept_uniform", "if (y < 0) y = ref_invcdf(P, V, (double)J->u_sample[b], &d); /* R4 */",
     "if (y < 0) y = ref_invcdf(P, V, (double)J->u_accept[(size_t)b * G + i], &d);"),
    ("tree_zero_residual_no_reset", "for (int v = 0; v < V; ++v) cur[v] = P[v];\n          ++rejected;",
     "for (int v = 0; v < V; ++v) cur[v] = 0.0;\n          ++rejected;"),
    ("tree_zero_residual_divides", "if (Z > 0.0)\n            for (int v = 0; v < V; ++v) cur[v] = fmax(cur[v] - Q[v], 0.0) / Z;",
     "if (1)\n            for (int v = 0; v < V; ++v) cur[v] = fmax(cur[v] - Q[v], 0.0) / Z;"),
    ("typical_non_strict", "if (!(px > thr)) {", "if (!(px >= thr)) {"),
    ("typical_max_threshold", "const double thr = fmin(eps, delta * exp(-H));", "const double thr = fmax(eps, delta * exp(-H));"),
    ("typical_exp_sign", "const double thr = fmin(eps, delta * exp(-H));", "const double thr = fmin(eps, delta * exp(H));"),
    ("typical_entropy_bits", "if (P[v] > 0.0) h -= P[v] * log(P[v]);", "if (P[v] > 0.0) h -= P[v] * log2(P[v]);"),
    ("typical_next_from_previous_row", "load_row(target, dtype, row0 + j, V, z);\n      out[j] = argmax_lowest(z, V);",
     "load_row(target, dtype, row0 + (j ? j - 1 : 0), V, z);\n      out[j] = argmax_lowest(z, V);"),
    ("typical_wrong_token", "const double px = P[x[i]];", "const double px = P[x[i ? i - 1 : 0]];"),
]

PIN_TESTS = [
    lambda: pins.test_four_token_table_alpha_and_acceptance_mass(),
    lambda: pins.test_four_token_table_residual(),
    lambda: pins.test_three_token_example(),
    lambda: pins.test_single_position_reference_checks(),
    lambda: pins.test_acceptance_boundary_is_inclusive(),
    lambda: pins.test_check_row_of_tiny_chain_config(),
    lambda: pins.test_policy_matches_scipy_softmax("bf16", 0.7),
    lambda: pins.test_topk_threshold_and_kept_set(5),
    lambda: pins.test_topk_brute_force_tiny(),
    lambda: pins.test_argmax_lowest_index(),
    lambda: pins.test_invcdf_matches_searchsorted(),
    lambda: pins.test_invcdf_boundary_distance(),
    lambda: pins.test_p_equals_q_accepts_every_legal_token("f32", 0),
    lambda: pins.test_disjoint_supports_correct_from_p(),
    lambda: pins.test_chain_structure("f32", 1.0, 0),
    lambda: pins.test_chain_structure("f32", 0.0, 0),
    lambda: pins.test_g_zero_is_plain_target_sampling(),
    lambda: pins.test_row_error_codes("u_one", oracle.ERR_UNIFORM),
    lambda: pins.test_zero_residual_fallback_draws_from_p("f32"),
    lambda: pins.test_zero_residual_fallback_draws_from_p("bf16"),
    lambda: stats.test_monte_carlo_law_matches_target(1.0, 0),
    lambda: stats.test_expected_tokens_constant_rate(0.6, 4),
    lambda: ovl.test_worked_examples(),
    lambda: ovl.test_two_point_closed_form(),
    lambda: ovl.test_identities_and_scipy(2.0, 5),
    lambda: ovl.test_target_layout_with_or_without_bonus_row(),
    lambda: ovl.test_row_checks(),
    lambda: tree.test_chain_tree_equals_chain_oracle("f32", 1.0, 0),
    lambda: tree.test_chain_tree_equals_chain_oracle("bf16", 0.0, 0),
    lambda: tree.test_second_sibling_is_tested_against_the_residual(),
    lambda: tree.test_third_sibling_threshold_and_final_draw(),
    lambda: tree.test_greedy_tree_walk(),
    lambda: tree.test_zero_residual_resets_to_p("f32"),
    lambda: tree.test_tree_checks("nan_draft_leaf", 0),
    lambda: tree.test_monte_carlo_tree_law_matches_target((3,), 1.0, 0),
    lambda: typ.test_entropy_matches_scipy(1.0, 0),
    lambda: typ.test_uniform_rows_closed_form(),
    lambda: typ.test_equality_rejects(),
    lambda: typ.test_threshold_sides(1),
    lambda: typ.test_threshold_sides(-1),
    lambda: typ.test_near_one_hot_is_greedy_chain(),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_kill_mutant(name, old, new, tmp_path):
    src = SRC.read_text()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mutated = tmp_path / f"{name}.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / f"lib_{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(lib),
                    str(mutated), "-lm"], check=True)
    saved = oracle._swap_library(lib)
    failures = 0
    try:
        for t in PIN_TESTS:
            try:
                t()
            except Exception:  # an assertion (or any error) means the mistake was seen
                failures += 1
                break
    finally:
        oracle._lib = saved
    assert failures, f"no pin detects the planted mistake '{name}'"
