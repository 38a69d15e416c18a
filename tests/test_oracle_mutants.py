"""The pins catch plausible mistakes: each mutant below is a copy of the oracle
with one planted error (on the CPU only); at least one pin must fail on it.

The mutants are built from ``oracle/oracle.c`` by a one-line text
substitution into a temporary directory; the real oracle is untouched and is
restored after each case.
"""
import ctypes
import os
import subprocess
import tempfile

import pytest

import oracle
import test_golden
import test_oracle_assign_sort as tas
import test_oracle_attn as tat
import test_oracle_multi as tmu
import test_oracle_sinkhorn as tsk
import test_oracle_soft_gate as tsg

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "window bound exclusive": ("if (i - j <= w) return 1;", "if (i - j < w) return 1;"),
    "causal bound drops the diagonal": ("if (j > i) return 0;", "if (j >= i) return 0;"),
    "group test inverted": ("return gi == gj;", "return gi != gj;"),
    "gqa head map interleaved": ("int64_t kvh = h / group;\n            const int32_t* g = ids + b * n;\n            int64_t cnt = 0;",
                                 "int64_t kvh = h % Hkv;\n            const int32_t* g = ids + b * n;\n            int64_t cnt = 0;"),
    "softmax scale dropped": ("s[a] = scale * dot;", "s[a] = dot;"),
    "score uses v instead of k": ("const uint16_t* krow = kbase + keys[a] * d;",
                                  "const uint16_t* krow = vbase + keys[a] * d;"),
    "lse misses the max": ("*lse = m + log(l);", "*lse = log(l);"),
    "merge takes the wrong part": ("(a * ow[x] + c * ol[x])", "(a * ow[x] + c * ow[x])"),
    "sort reverses each group": ("perm[b * n + off[k] + seen[k]] = (int32_t)t;",
                                 "perm[b * n + off[k + 1] - 1 - seen[k]] = (int32_t)t;"),
    "argmax ties go high": ("if (s[k] > s[best]) best = k;", "if (s[k] >= s[best]) best = k;"),
    "bias subtracted": ("s[k] = bias ? acc + bias[k] : acc;", "s[k] = bias ? acc - bias[k] : acc;"),
    "projection transposed": ("z[j] = z[j] + hm * Prow[j];", "z[j] = z[j] + hm * P[j * d_model + m];"),
    "off-by-one long-range start": ("for (int64_t j = 0; j < i - w; ++j)", "for (int64_t j = 0; j <= i - w; ++j)"),
    "shared group compares one slot": ("if (gi[a] == gj[c]) return 1;", "if (gi[a] == gj[a]) return 1;"),
    "top-m ties go high": ("(best < 0 || s[k] > s[best])", "(best < 0 || s[k] >= s[best])"),
    "top-m margin from the first rank": ("INFINITY : last - next;", "INFINITY : s[ids[r * m]] - next;"),
    "multi window bound exclusive": ("if (i - j <= w || share_group(g + i * m, g + j * m, m)) keys",
                                     "if (i - j < w || share_group(g + i * m, g + j * m, m)) keys"),
    "multi pair count adds both tests": ("cnt += (i - j <= w) || share_group(",
                                         "cnt += (i - j <= w) + share_group("),
    # (a uniform column target of any size is equivalent: the last row step
    # cancels it; unequal targets are the mistake to catch)
    "sinkhorn unequal column targets": ("v[k] = ((double)n / (double)K) / col[k];",
                                        "v[k] = ((double)(n + k) / (double)K) / col[k];"),
    "sinkhorn temperature dropped": ("A[x] = exp((double)S[x] / tau);", "A[x] = exp((double)S[x]);"),
    "sinkhorn last column scale dropped": ("Gb[t * K + k] = A[t * K + k] * u[t] * v[k];",
                                           "Gb[t * K + k] = A[t * K + k] * u[t];"),
    "sinkhorn rows-first step skipped": ("u[t] = 1.0 / r;\n        }\n        for (int64_t it",
                                         "u[t] = 1.0;\n        }\n        for (int64_t it"),
    "sinkhorn column sum misses u": ("col[k] += A[t * K + k] * u[t];", "col[k] += A[t * K + k];"),
    "soft gate reaches into the window": ("if (i - j > w) {\n                    const float* gj",
                                          "if (i - j >= w) {\n                    const float* gj"),
    "soft gate sign flipped": ("gate = 1.0 / (1.0 + exp(-lambda * a));",
                               "gate = 1.0 / (1.0 + exp(lambda * a));"),
    "soft gate affinity of the row with itself": ("a += (double)gi[x] * (double)gj[x];",
                                                  "a += (double)gi[x] * (double)gi[x];"),
    "soft gate dropped": ("double p = gate * exp(s[j] - m);", "double p = exp(s[j] - m);"),
}

PINS = [
    lambda: tat.test_single_group_is_dense_causal(3),
    tat.test_wide_window_is_dense_causal,
    tat.test_lse_is_log_sum_exp_over_allowed_scores,
    tat.test_window_zero_is_causal_attention_within_each_group,
    lambda: tat.test_brute_force_pair_enumeration(*tat.CASES[4]),
    lambda: tat.test_brute_force_pair_enumeration(*tat.CASES[5]),
    tat.test_weights_sum_to_one_and_vanish_outside_the_pattern,
    tat.test_two_part_split_matches_single_softmax,
    tat.test_gqa_head_map_equals_repeated_kv,
    lambda: tat.test_visited_pairs_closed_form(200, 13, 7),
    tas.test_assign_matches_fp64_argmax_outside_tie_band,
    tas.test_assign_exact_tie_takes_lowest_index,
    lambda: tas.test_sort_matches_stable_argsort(3, 100, 4),
    test_golden.test_hand_worked_pattern_and_uniform_score_outputs,
    tmu.test_topk_matches_fp64_ranking_outside_tie_band,
    tmu.test_topk_exact_ties_take_lowest_index_and_m_equals_K,
    lambda: tmu.test_all_groups_is_dense_causal(5),
    lambda: tmu.test_brute_force_set_enumeration(*tmu.CASES[2]),
    lambda: tmu.test_pair_count_inclusion_exclusion(300, 11, 4),
    tsk.test_zero_iterations_is_row_softmax,
    tsk.test_additive_scores_give_uniform_assignment,
    tsk.test_two_by_two_limit_closed_form,
    tsk.test_cross_ratios_are_those_of_exp_scores,
    tsk.test_marginals_rows_exact_columns_converge,
    tsk.test_row_shift_and_column_permutation,
    tsg.test_wide_window_is_causal_attention,
    tsg.test_zero_lambda_halves_far_pairs,
    lambda: tsg.test_uniform_assignment_gives_a_constant_gate(4, 3.0),
    tsg.test_general_gate_against_sdpa_with_affinity_bias,
    lambda: tsg.test_brute_force(17, 3, -2.0, 3),
]


def _failures(lib):
    saved = oracle._lib
    oracle._lib = lib
    failed = 0
    try:
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                failed += 1
    finally:
        oracle._lib = saved
    return failed


def test_unmutated_copy_passes_every_pin():
    assert _failures(oracle._load()) == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name!r} not unique"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib_path = str(tmp_path / "libmutant.so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC",
                           "-shared", "-o", lib_path, str(path), "-lm"])
    lib = oracle.configure(ctypes.CDLL(lib_path))
    assert _failures(lib) >= 1, f"no pin caught mutant {name!r}"
