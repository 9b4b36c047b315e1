"""Plant plausible mistakes in a copy of the CPU oracle; the pins must catch each.

This shows the pins in tests/oracle_pins.py have teeth: every mutant below is
a slip someone could make while writing the filter. Each one is planted in a
copy of oracle/topktopp_oracle.cpp (one or two source edits), compiled with
the host compiler into a temporary library, and must fail at least one pin.
Everything runs on the CPU.
"""

import os
import warnings

import pytest

from oracle.build_oracle import SOURCE, compile_oracle
from oracle.topktopp_oracle import Oracle
from tests import oracle_pins as pins

# name -> list of (text in the oracle source, replacement)
MUTANTS = {
    "topk_masks_ties_too": [("d.masked_k[j] = s[j] < kth ? 1 : 0;", "d.masked_k[j] = s[j] <= kth ? 1 : 0;")],
    "kth_index_off_by_one": [("const double kth = s[V - prm.k];", "const double kth = s[V - prm.k - 1];")],
    "topp_strict_less": [("d.masked_p[j] = d.cum32[j] <= d.t ? 1 : 0;", "d.masked_p[j] = d.cum32[j] < d.t ? 1 : 0;")],
    "last_position_not_forced": [("for (int64_t j = 0; j < V - 1; ++j) d.masked_p[j]",
                                  "for (int64_t j = 0; j < V; ++j) d.masked_p[j]")],
    "cumsum_from_largest": [("  for (int64_t j = 0; j < V; ++j) {\n    c += d.prob[j];",
                             "  for (int64_t j = V - 1; j >= 0; --j) {\n    c += d.prob[j];")],
    "softmax_ignores_topk": [("e[j] = d.masked_k[j] ? 0.0 : std::exp(s[j] - m);", "e[j] = std::exp(s[j] - m);")],
    "t_is_p_not_one_minus_p": [("const float t = 1.0f - p;", "const float t = p;")],
    "ties_reverse_index_order": [("return x[a] < x[b]; });", "return x[a] < x[b] || (x[a] == x[b] && a > b); });")],
    "gather_instead_of_scatter": [("store_bits(out, dtype, b * V + v, d.survives(rank[v]) ? bits : neg_inf_bits(dtype));",
                                   "store_bits(out, dtype, b * V + v, d.survives(v) ? load_bits(logits, dtype, b * V + order[v]) "
                                   ": neg_inf_bits(dtype));")],
    # k beyond V taken as a threshold (an index that wraps around, as a
    # negative index would in a scripting language)
    "topk_disabled_only_for_k_le_0": [("prm.k >= 1 && prm.k <= V - 1", "prm.k >= 1"),
                                      ("const double kth = s[V - prm.k];",
                                       "const double kth = s[((V - prm.k) % V + V) % V];")],
    # kept values re-encoded from their value: a kept -0.0 comes back as +0.0
    "kept_values_as_float_not_bits": [("const uint32_t bits = load_bits(logits, dtype, b * V + v);",
                                       "const uint32_t bits = widen(load_bits(logits, dtype, b * V + v), dtype) == 0.0 ? 0u "
                                       ": load_bits(logits, dtype, b * V + v);")],
}

CHEAP_FIRST = [
    pins.check_hand_cases,
    pins.check_invariants,
    pins.check_topk_counting_random,
    pins.check_nucleus_random,
    pins.check_permutation_equivariance,
    pins.check_bruteforce_tiny,
]

# Slips in the min-p stage; the min-p pins must catch each.
MINP_MUTANTS = {
    "minp_threshold_without_max": [("const double thr = d.prob[V - 1] * mp;", "const double thr = mp;")],
    "minp_threshold_divides": [("const double thr = d.prob[V - 1] * mp;", "const double thr = d.prob[V - 1] / mp;")],
    "minp_at_least_one_keeps_every_max": [("for (int64_t j = 0; j < V - 1; ++j) d.masked_m[j] = 1;",
                                           "for (int64_t j = 0; j < V - 1; ++j) d.masked_m[j] = s[j] < s[V - 1] ? 1 : 0;")],
    "minp_ratio_from_logits": [("d.masked_m[j] = (d.masked_p[j] || d.prob[j] < thr) ? 1 : 0;",
                                "d.masked_m[j] = (d.masked_p[j] || (s[j] - s[0] + 1e-9) < (s[V - 1] - s[0] + 1e-9) * mp) ? 1 : 0;")],
}

MINP_CHECKS = [
    pins.check_minp_hand_cases,
    pins.check_minp_invariants,
    pins.check_minp_random,
    pins.check_minp_bruteforce_tiny,
]

# Slips in the sampling stage; the sampling pins must catch each.
SAMPLE_MUTANTS = {
    "sample_q_by_vocabulary_index": [("const double denom = q[b * V + dd] + eps;",
                                      "const double denom = q[b * V + order[V - 1 - dd]] + eps;")],
    "sample_last_maximum": [("} else if (best_d < 0 || sc > best) {", "} else if (best_d < 0 || sc >= best) {")],
    "sample_ascending_ranks": [("const int64_t j = V - 1 - dd;\n      const double denom",
                                "const int64_t j = dd;\n      const double denom"),
                               ("selected[b] = order[V - 1 - best_d];", "selected[b] = order[best_d];")],
    "sample_eps_ignored": [("const double denom = q[b * V + dd] + eps;", "const double denom = q[b * V + dd];")],
    "sample_none_lowest_index": [("selected[b] = order[V - 1];  // the first maximum of probs: the top rank",
                                  "{ int64_t j0 = V - 1; while (j0 > 0 && x[order[j0 - 1]] == x[order[V - 1]]) --j0; "
                                  "selected[b] = order[j0]; }")],
}

SAMPLE_CHECKS = [
    pins.check_sample_hand_cases,
    pins.check_sample_none_is_top,
    pins.check_sample_bruteforce_tiny,
    pins.check_sample_race_distribution,
]

# Slips in the sorted-survivors output; its pins must catch each.
SURVIVOR_MUTANTS = {
    "survivors_ascending": [("const int64_t j = V - 1 - dd;\n      if (!d.survives(j)) continue;",
                             "const int64_t j = dd;\n      if (!d.survives(j)) continue;")],
    "survivors_renormalised_after_top_p": [
        ("probs[b * cap + n] = d.prob[j];",
         "probs[b * cap + n] = d.prob[j] / [&] { double z = 0.0; for (int64_t i = 0; i < V; ++i) "
         "if (d.survives(i)) z += d.prob[i]; return z; }();")],
    "survivors_ties_lower_index_first": [
        ("indices[b * cap + n] = order[j];",
         "{ int64_t a = j, c = j; while (a > 0 && x[order[a - 1]] == x[order[j]]) --a; "
         "while (c < V - 1 && x[order[c + 1]] == x[order[j]]) ++c; indices[b * cap + n] = order[a + c - j]; }")],
}

SURVIVOR_CHECKS = [
    pins.check_survivor_hand_cases,
    pins.check_survivor_softmax_closed_form,
    pins.check_survivor_bruteforce_tiny,
]


def make_mutant(tmp_path, name, edits) -> Oracle:
    src = open(SOURCE).read()
    for old, new in edits:
        assert src.count(old) == 1, (name, old)
        src = src.replace(old, new)
    path = os.path.join(str(tmp_path), f"{name}.cpp")
    with open(path, "w") as f:
        f.write(src)
    return Oracle(compile_oracle(path, os.path.join(str(tmp_path), f"lib{name}.so"), opt="-O1"))


def caught(checks, fn):
    for check in checks:
        try:
            with warnings.catch_warnings():
                warnings.simplefilter("ignore")
                check(fn)
        except (AssertionError, IndexError, ValueError):
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    mod = make_mutant(tmp_path, name, MUTANTS[name])

    def apply_fn(x, dtype, p, k):
        return mod.apply_top_k_top_p(x, dtype, p, k, keep_traces=False).out

    assert caught(CHEAP_FIRST, apply_fn), f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(MINP_MUTANTS))
def test_min_p_mutant_is_caught(name, tmp_path):
    mod = make_mutant(tmp_path, name, MINP_MUTANTS[name])

    def apply_mp_fn(x, dtype, p, k, min_p):
        return mod.apply_top_k_top_p(x, dtype, p, k, keep_traces=False, min_p_bits=min_p).out

    assert caught(MINP_CHECKS, apply_mp_fn), f"mutant {name} passed every min-p pin"


@pytest.mark.parametrize("name", sorted(SAMPLE_MUTANTS))
def test_sample_mutant_is_caught(name, tmp_path):
    mod = make_mutant(tmp_path, name, SAMPLE_MUTANTS[name])

    def sample_fn(x, dtype, p, k, min_p, q, eps):
        return mod.sample_top_k_top_p(x, dtype, p, k, min_p, q, eps).selected

    assert caught(SAMPLE_CHECKS, sample_fn), f"mutant {name} passed every sampling pin"


@pytest.mark.parametrize("name", sorted(SURVIVOR_MUTANTS))
def test_survivor_mutant_is_caught(name, tmp_path):
    mod = make_mutant(tmp_path, name, SURVIVOR_MUTANTS[name])

    def surv_fn(x, dtype, p, k, min_p, cap):
        r = mod.sorted_survivors(x, dtype, p, k, min_p, cap)
        return r.probs, r.indices, r.counts

    assert caught(SURVIVOR_CHECKS, surv_fn), f"mutant {name} passed every survivor pin"


def test_unmutated_copy_passes_every_pin(tmp_path):
    """The same compile path without edits passes every pin, so a caught
    mutant is caught for its edit and not for the way it was built."""
    mod = make_mutant(tmp_path, "unmutated", [])

    def apply_fn(x, dtype, p, k):
        return mod.apply_top_k_top_p(x, dtype, p, k, keep_traces=False).out

    for check in CHEAP_FIRST:
        check(apply_fn)
