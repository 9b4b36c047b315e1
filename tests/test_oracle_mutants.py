"""Plant plausible mistakes in a copy of the CPU oracle; the pins must catch each.

This shows the pins in tests/oracle_pins.py have teeth: every mutant below is
a one-line slip someone could make while writing the filter, and each one must
fail at least one pin. The mutants live only in memory, on the CPU.
"""

import sys
import types

import pytest

import oracle.topktopp_oracle as O
from tests import oracle_pins as pins

MUTANTS = {
    "topk_masks_ties_too": ("top_k_mask = s < top_k_value", "top_k_mask = s <= top_k_value"),
    "kth_index_off_by_one": ("top_k_value = s[V - int(k_b)]", "top_k_value = s[V - int(k_b) - 1]"),
    "topp_strict_less": ("top_p_mask = probs_sum32 <= t", "top_p_mask = probs_sum32 < t"),
    "last_position_not_forced": ("top_p_mask[V - 1] = False", "pass"),
    "cumsum_from_largest": ("probs_sum = np.cumsum(probs_value)",
                            "probs_sum = np.cumsum(probs_value[::-1])[::-1]"),
    "softmax_ignores_topk": ("s[top_k_mask] = -np.inf", "pass"),
    "t_is_p_not_one_minus_p": ("t = np.float32(np.float32(1.0) - p32)", "t = p32"),
    "ties_reverse_index_order": ('np.argsort(x, kind="stable")', 'np.argsort(-x, kind="stable")[::-1]'),
    "gather_instead_of_scatter": ("out[b, sorted_indices] = sorted_bits",
                                  "out[b] = sorted_bits[sorted_indices]"),
    "topk_disabled_only_for_k_le_0": ("1 <= int(k_b) <= V - 1", "1 <= int(k_b) <= V + 100"),
    "kept_values_as_float_not_bits": ("np.where(masked, NEG_INF_BITS[dtype], row_bits[sorted_indices])",
                                      "np.where(masked, NEG_INF_BITS[dtype], "
                                      "np.where(row_bits[sorted_indices] == NEG_INF_BITS['f32'] >> 16, 0, "
                                      "row_bits[sorted_indices] & ~np.asarray(0x8000, row_bits.dtype)))"),
}

CHEAP_FIRST = [
    pins.check_hand_cases,
    pins.check_invariants,
    pins.check_topk_counting_random,
    pins.check_nucleus_random,
    pins.check_permutation_equivariance,
    pins.check_bruteforce_tiny,
]


def make_mutant(old, new):
    src = open(O.__file__).read()
    assert src.count(old) == 1, old
    name = "oracle_mutant_%x" % (abs(hash((old, new))))
    mod = types.ModuleType(name)
    mod.__file__ = O.__file__
    sys.modules[name] = mod  # dataclasses look their module up here
    exec(compile(src.replace(old, new), name, "exec"), mod.__dict__)
    return mod


# Slips in the min-p stage; the min-p pins must catch each.
MINP_MUTANTS = {
    "minp_threshold_without_max": ("threshold = sort_masked.max() * mp", "threshold = mp"),
    "minp_threshold_divides": ("threshold = sort_masked.max() * mp", "threshold = sort_masked.max() / mp"),
    "minp_at_least_one_keeps_every_max": ("min_p_mask[: V - 1] = True", "min_p_mask = s < s[V - 1]"),
    "minp_ratio_from_logits": ("e = np.exp(s - m)\n            probs = e / np.cumsum(e)[-1]",
                               "probs = np.where(np.isfinite(s), s - s.min() + 1e-9, 0.0)"),
}

MINP_CHECKS = [
    pins.check_minp_hand_cases,
    pins.check_minp_invariants,
    pins.check_minp_random,
    pins.check_minp_bruteforce_tiny,
]


@pytest.mark.parametrize("name", sorted(MINP_MUTANTS))
def test_min_p_mutant_is_caught(name):
    mod = make_mutant(*MINP_MUTANTS[name])

    def apply_mp_fn(x, dtype, p, k, min_p):
        return mod.apply_top_k_top_p(x, dtype, p, k, keep_traces=False, min_p_bits=min_p).out

    for check in MINP_CHECKS:
        try:
            check(apply_mp_fn)
        except (AssertionError, IndexError, ValueError):
            return
    pytest.fail(f"mutant {name} passed every min-p pin")


# Slips in the sampling stage; the sampling pins must catch each.
SAMPLE_MUTANTS = {
    "sample_q_by_vocabulary_index": ("qb = np.asarray(q[b], dtype=np.float64)",
                                     "qb = np.asarray(q[b], dtype=np.float64)[desc]"),
    "sample_last_maximum": ("r = int(np.argmax(score))  # first maximum",
                            "r = len(score) - 1 - int(np.argmax(score[::-1]))"),
    "sample_ascending_ranks": ("desc = perm[::-1]  # descending rank r -> original index",
                               "desc = perm"),
    "sample_eps_ignored": ("score = probs / (qb + float(eps))", "score = probs / qb"),
    "sample_none_lowest_index": ("selected[b] = int(desc[0])",
                                 "selected[b] = int(np.nonzero(x0 == x0.max())[0].min()) "
                                 "if (x0 := widen_to_f64(np.asarray(logits_bits)[b], dtype)) is not None else 0"),
}

SAMPLE_CHECKS = [
    pins.check_sample_hand_cases,
    pins.check_sample_none_is_top,
    pins.check_sample_bruteforce_tiny,
    pins.check_sample_race_distribution,
]


@pytest.mark.parametrize("name", sorted(SAMPLE_MUTANTS))
def test_sample_mutant_is_caught(name):
    mod = make_mutant(*SAMPLE_MUTANTS[name])

    def sample_fn(x, dtype, p, k, min_p, q, eps):
        import warnings

        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            return mod.sample_top_k_top_p(x, dtype, p, k, min_p, q, eps).selected

    for check in SAMPLE_CHECKS:
        try:
            check(sample_fn)
        except (AssertionError, IndexError, ValueError):
            return
    pytest.fail(f"mutant {name} passed every sampling pin")


# Slips in the sorted-survivors output; its pins must catch each.
SURVIVOR_MUTANTS = {
    "survivors_ascending": ("        desc = tr.sorted_indices[::-1]\n        kept_desc = ~masked[::-1]\n        n = int",
                            "        desc = tr.sorted_indices\n        kept_desc = ~masked\n        n = int"),
    "survivors_renormalised_after_top_p": (
        "        xk = np.where(tr.top_k_mask[::-1], -np.inf, x)\n        e = np.exp(xk - xk[0])\n"
        "        step4 = e / e.sum()\n        m = min(n, cap)",
        "        xk = np.where(masked[::-1], -np.inf, x)\n        e = np.exp(xk - xk[0])\n"
        "        step4 = e / e.sum()\n        m = min(n, cap)"),
    "survivors_ties_lower_index_first": ("        desc = tr.sorted_indices[::-1]\n        kept_desc = ~masked[::-1]\n        n = int",
                                         "        desc = np.lexsort((tr.sorted_indices, -widen_to_f64(np.asarray(logits_bits)[b], dtype)[tr.sorted_indices]))\n        desc = tr.sorted_indices[desc]\n        kept_desc = ~masked[::-1]\n        n = int"),
}

SURVIVOR_CHECKS = [
    pins.check_survivor_hand_cases,
    pins.check_survivor_softmax_closed_form,
    pins.check_survivor_bruteforce_tiny,
]


@pytest.mark.parametrize("name", sorted(SURVIVOR_MUTANTS))
def test_survivor_mutant_is_caught(name):
    mod = make_mutant(*SURVIVOR_MUTANTS[name])

    def surv_fn(x, dtype, p, k, min_p, cap):
        r = mod.sorted_survivors(x, dtype, p, k, min_p, cap)
        return r.probs, r.indices, r.counts

    for check in SURVIVOR_CHECKS:
        try:
            check(surv_fn)
        except (AssertionError, IndexError, ValueError):
            return
    pytest.fail(f"mutant {name} passed every survivor pin")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = make_mutant(*MUTANTS[name])

    def apply_fn(x, dtype, p, k):
        return mod.apply_top_k_top_p(x, dtype, p, k, keep_traces=False).out

    for check in CHEAP_FIRST:
        try:
            check(apply_fn)
        except (AssertionError, IndexError, ValueError):
            return
    pytest.fail(f"mutant {name} passed every pin")
