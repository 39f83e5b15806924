"""The pins must catch plausible mistakes: each case compiles a copy of the oracle with one
planted mistake (on the CPU, in a temporary directory) and checks that a pin test fails."""
import ctypes
import functools
import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_draft_options_pins as op
import test_oracle_draft_pins as dp
import test_oracle_plan_pins as pp
import test_oracle_rnn_pins as rp
import test_oracle_tree_pins as tp
import test_oracle_verify_pins as vp

SRC = os.path.join(os.path.dirname(oracle.__file__), "dspark_oracle.cpp")

MUTATIONS = [
    ("residual sign", "std::max(0.0, pt[v] - pd[v])", "std::max(0.0, pd[v] - pt[v])",
     [vp.test_ab_worked_example_exact_grid]),
    ("bias from anchor at every position", "prev = cond;", "prev = anchor[b];",
     [dp.test_markov_chain_probabilities_closed_form]),
    ("confidence reads x_k", "(k == 0) ? anchor[b] : tokens[b * gamma + k - 1]",
     "tokens[b * gamma + k]", [dp.test_confidence_closed_forms]),
    ("survival order ascending", "if (x.a != y.a) return x.a > y.a;",
     "if (x.a != y.a) return x.a < y.a;", [pp.test_brute_force_planner_optimality]),
    ("early stop keeps going on a tie", "if (!(theta[k + 1] > theta[k])) break;",
     "if (!(theta[k + 1] >= theta[k] - 0.2)) break;", [pp.test_appendix_a_theta_values_and_choices]),
    ("SPS indexed by admissions", "theta[i] = tau[i] * sps[R + i];", "theta[i] = tau[i] * sps[1 + i];",
     [pp.test_brute_force_planner_optimality]),
    ("bonus uses the accept uniform", "uniforms[(b * (gamma + 1) + ell) * 3 + 2]",
     "uniforms[(b * (gamma + 1) + ell) * 3 + 1]", [vp.test_bonus_only_when_all_accepted_and_flags]),
    ("accept test inverted ratio", "if (u * qk < pt) {", "if (u * pt < qk) {",
     [functools.partial(vp.test_chi2_output_marginal_equals_target, 1)]),
    ("residual recomputed at the next position",
     "draft_logits(U + (b * gamma + k - 1) * static_cast<int64_t>(V), W1, W2t, V, r, prev, L);",
     "draft_logits(U + (b * gamma + (k < gamma ? k : k - 1)) * static_cast<int64_t>(V), W1, W2t, V, r, prev, L);",
     [vp.test_sum_min_identity_on_every_emission_row]),
    ("temperature multiplies", "std::exp(-z / static_cast<double>(T[k]))",
     "std::exp(-z * static_cast<double>(T[k]))", [dp.test_confidence_closed_forms]),
    ("draft inverse CDF from the top", "if (cdf > u) {", "if (cdf > 1.0 - u) {",
     [dp.test_w2_zero_reduces_to_inverse_cdf_categorical]),
    ("draft temperature multiplies", "return static_cast<float>(1.0 / static_cast<double>(tau));",
     "return tau;", [op.test_temperature_limits_uniform_and_argmax]),
    ("greedy takes the last maximum", "if (L[v] > L[best]) best", "if (L[v] >= L[best]) best",
     [op.test_greedy_draft_closed_form_and_ties]),
    ("greedy residual keeps the drafted token", "pd[tokens[b * gamma + k - 1]] = 1.0;",
     "pd[0] = 1.0;", [op.test_greedy_verify_is_lossless_exact_grid]),
    ("tempered residual left unscaled", "    scale_logits(L, beta);\n    softmax_fp64(L.data(), V, pd);",
     "    softmax_fp64(L.data(), V, pd);",
     [functools.partial(op.test_tempered_verify_is_lossless_exact_grid, 0.5)]),
    ("rnn gate roles swapped", "s_next[j] = gate * s_prev[j] + (1.0 - gate) * cand;",
     "s_next[j] = (1.0 - gate) * s_prev[j] + gate * cand;",
     [functools.partial(rp.test_saturated_gates, 1.0)]),
    ("rnn bias read from the candidate rows", "e[j] = std::tanh(row_dot(2 * r + j));",
     "e[j] = std::tanh(row_dot(r + j));", [rp.test_output_path_is_a_tanh_embedding_chain]),
    ("rnn draft conditions every step on the anchor", "x_prev = x_cond;", "x_prev = anchor[b];",
     [rp.test_output_path_is_a_tanh_embedding_chain]),
    ("rnn state not carried between draft steps",
     "rnn_update(Wgco, W1, h + bk * static_cast<int64_t>(d), r, d, x_prev, state, next_state, e);\n      state.swap(next_state);",
     "rnn_update(Wgco, W1, h + bk * static_cast<int64_t>(d), r, d, x_prev, state, next_state, e);",
     [rp.test_state_path_half_gate_closed_form]),
    ("rnn verify reruns the state along the anchor", "x_prev = tokens[bi];", "x_prev = anchor[b];",
     [functools.partial(rp.test_verify_recomputes_the_draft_distribution_along_the_drafted_tokens,
                        "embedding")]),
    ("rnn hidden block read at the embedding offset",
     "for (int i = 0; i < d; ++i) z[2 * r + i] = bf16_to_double(h_row[i]);",
     "for (int i = 0; i < d && i < r; ++i) z[r + i] = bf16_to_double(h_row[i]);",
     [rp.test_state_path_half_gate_closed_form]),
    ("lagged capacity by early stop", "const int64_t k_lag = full_path_count(theta_lag, &mg);",
     "const int64_t k_lag = early_stop_count(theta_lag, &mg);",
     [pp.test_lagged_capacity_is_a_full_path_search_on_a_two_peak_table]),
    ("full path keeps the last maximiser", "if (theta[i] > theta[best]) best = i;",
     "if (theta[i] >= theta[best]) best = i;",
     [pp.test_full_path_takes_the_first_maximiser_on_a_plateau]),
    ("bonus drawn from the last drafted row",
     "const float* row = target + (off + ell) * static_cast<int64_t>(V);",
     "const float* row = target + (off + ell - 1) * static_cast<int64_t>(V);",
     [vp.test_bonus_is_drawn_from_the_row_after_the_last_verified_draft,
      vp.test_two_token_output_exact_grid_with_position_dependent_rows]),
    ("tree children by the smallest logits", "if (L[a] != L[b]) return L[a] > L[b];",
     "if (L[a] != L[b]) return L[a] < L[b];",
     [tp.test_w2_zero_children_are_the_top_c_of_the_base_logits]),
    ("tree path probability as a sum", "t.P = Ppar * t.q;", "t.P = Ppar + t.q;",
     [functools.partial(tp.test_kept_nodes_are_the_most_likely_paths_brute_force, 1)]),
    ("tree expands the least likely nodes", "if (all[a].P != all[bb].P) return all[a].P > all[bb].P;\n        return all[a].idx < all[bb].idx;",
     "if (all[a].P != all[bb].P) return all[a].P < all[bb].P;\n        return all[a].idx < all[bb].idx;",
     [functools.partial(tp.test_tree_structure_beam_and_budget, s) for s in range(10)]),
    ("tree emission re-emits rejected children", "for (int32_t x : kids) excluded[x] = 1;",
     "for (int32_t x : kids) excluded[x] = 0;",
     [tp.test_tree_verify_exact_grid_follows_the_target_chain]),
    ("tree walk reads the root row at every node",
     "const float* row = target + (b * static_cast<int64_t>(N + 1) + (cur + 1)) * V;",
     "const float* row = target + (b * static_cast<int64_t>(N + 1)) * V;",
     [tp.test_tree_verify_exact_grid_follows_the_target_chain]),
    ("tree walk draws every depth with the first uniform",
     "uniforms[(b * (gamma + 1) + depth) * 3 + 2]", "uniforms[(b * (gamma + 1)) * 3 + 2]",
     [tp.test_tree_verify_exact_grid_follows_the_target_chain]),
]


@pytest.mark.parametrize("name,old,new,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, pins, monkeypatch):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old}"
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "m.cpp")
        lib = os.path.join(td, "libm.so")
        open(path, "w").write(src.replace(old, new))
        subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-pthread", path, "-o", lib],
                       check=True)
        mutated = ctypes.CDLL(lib)
        for fn in ("oracle_markov_draft", "oracle_confidence", "oracle_plan", "oracle_verify",
                   "oracle_tree_draft", "oracle_tree_verify"):
            getattr(mutated, fn).restype = ctypes.c_int
        monkeypatch.setattr(oracle, "_lib", mutated)
        caught = False
        for pin in pins:
            try:
                if pin is pp.test_brute_force_planner_optimality:
                    for seed in range(40):
                        pin(seed)
                else:
                    pin()
            except AssertionError:
                caught = True
        assert caught, f"planted mistake '{name}' was not caught"
