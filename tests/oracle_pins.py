"""Checks that pin the CPU oracle to facts other than its own code.

Each check takes ``apply_fn(logits_bits, dtype, p_bits, k) -> out_bits`` and
raises AssertionError on a mismatch, so the same checks run against the real
oracle (they must pass) and against deliberately broken copies of it (each
copy must fail at least one check).

The facts used:
  * hand-derived cases (tests/golden/hand_cases.txt), including the calling
    example of the ApplyTopKTopPWithSorted page, §7;
  * top-k by counting: the threshold T is the value with
    #(x > T) < k <= #(x >= T), found without sorting;
  * top-p by the textbook nucleus rule (Holtzman et al., "The Curious Case of
    Neural Text Degeneration"): walking from the most probable token down, a
    token is kept while the probability mass strictly above it is below p,
    here p' = 1 - t with t the fp32 value the filter compares against; the
    walk visits equal values from the highest index down, which is the
    reverse of a stable ascending sort;
  * invariants: at least one survivor, survivors form a suffix of the stable
    order, kept bits equal the inputs, p = 0 keeps exactly the last sorted
    position, disabled k values agree, permutation equivariance.
"""

from __future__ import annotations

import math

import numpy as np

from tests.golden_io import NEG_INF_WORD, load_hand_cases
from workloads.synth import bits_to_f32, random_rows


def _vals(bits, dtype):
    return bits_to_f32(np.asarray(bits), dtype).astype(np.float64)


def _t32(p_bits_b, dtype):
    p32 = np.float32(bits_to_f32(np.asarray([p_bits_b]), dtype)[0])
    return np.float32(np.float32(1.0) - p32)


def check_hand_cases(apply_fn):
    for case in load_hand_cases():
        got = apply_fn(case.x, case.dtype, case.p, case.k)
        assert np.array_equal(got, case.expect), (case.name, got, case.expect)


def topk_threshold_by_counting(x, k):
    """Value T with #(x > T) < k <= #(x >= T), by counting (no sort)."""
    for T in set(float(v) for v in x):
        gt = sum(1 for v in x if v > T)
        ge = sum(1 for v in x if v >= T)
        if gt < k <= ge:
            return T
    raise AssertionError("no threshold found")


def expected_keep_bruteforce(x, k, t):
    """Survivor set from counting (top-k) and the nucleus walk (top-p).

    Returns (keep bool array, ambiguous flag). ``ambiguous`` is set when the
    mass above some token is within 1e-9 of p', where double rounding could
    legitimately decide either way.
    """
    V = len(x)
    keep_k = np.ones(V, dtype=bool)
    if k is not None and 1 <= k <= V - 1:
        T = topk_threshold_by_counting(x, k)
        keep_k = np.array([v >= T for v in x])
    if t is None:
        return keep_k, False
    order = sorted(range(V), key=lambda i: (x[i], i), reverse=True)
    alive = [i for i in order if keep_k[i]]
    m = x[alive[0]]
    w = [math.exp(x[i] - m) for i in alive]
    Z = math.fsum(w)
    p_prime = 1.0 - float(t)
    keep = np.zeros(V, dtype=bool)
    ambiguous = False
    for pos, i in enumerate(alive):
        above = math.fsum(w[:pos]) / Z
        if abs(above - p_prime) < 1e-9:
            ambiguous = True
        if pos == 0 or above < p_prime:
            keep[i] = True
    return keep, ambiguous


def check_bruteforce_tiny(apply_fn, dtypes=("f32", "bf16", "f16"), n_rows=6, max_v=8):
    """Every k in [-1, V+1] and a p grid on tiny rows with ties and both zeros."""
    p_grid = [0.0, 0.05, 0.2, 0.35, 0.5, 0.65, 0.8, 0.95, 1.0]
    seed = 0
    for dtype in dtypes:
        for V in range(1, max_v + 1):
            for kind in ("normal", "ties", "zeros", "gumbel"):
                seed += 1
                xb = random_rows(seed, n_rows, V, dtype, kind=kind, scale=1.5)
                for b in range(n_rows):
                    row = xb[b : b + 1]
                    x = list(_vals(row[0], dtype))
                    for kk in [None] + list(range(-1, V + 2)):
                        for pv in [None] + p_grid:
                            if kk is None and pv is None:
                                continue
                            p_bits = None
                            t = None
                            if pv is not None:
                                from workloads.synth import f32_to_bits

                                p_bits = f32_to_bits(np.array([pv], np.float32), dtype)
                                t = _t32(p_bits[0], dtype)
                            k_arr = None if kk is None else np.array([kk], np.int32)
                            got = apply_fn(row, dtype, p_bits, k_arr)[0]
                            keep, amb = expected_keep_bruteforce(x, kk, t)
                            if amb:
                                continue
                            exp = np.where(keep, row[0], NEG_INF_WORD[dtype]).astype(row.dtype)
                            assert np.array_equal(got, exp), (dtype, V, kind, b, kk, pv, x, got, exp)


def check_topk_counting_random(apply_fn, dtype="f32", V=257, B=24):
    """Larger rows, k only: survivors are exactly {x >= T} with T by counting."""
    for kind in ("normal", "ties", "zeros"):
        xb = random_rows(1000 + V, B, V, dtype, kind=kind)
        rng = np.random.default_rng(7)
        k = rng.integers(1, V - 1, size=B, endpoint=True).astype(np.int32)
        got = apply_fn(xb, dtype, None, k)
        for b in range(B):
            x = _vals(xb[b], dtype)
            T = topk_threshold_by_counting(list(x), int(k[b]))
            exp = np.where(x >= T, xb[b], NEG_INF_WORD[dtype]).astype(xb.dtype)
            assert np.array_equal(got[b], exp), (kind, b)


def check_nucleus_random(apply_fn, dtype="f32", V=96, B=32):
    """Moderate rows, joint and p-only, against the nucleus walk."""
    for kind in ("normal", "ties", "gumbel"):
        xb = random_rows(2000 + V, B, V, dtype, kind=kind)
        rng = np.random.default_rng(11)
        k = rng.integers(-1, V + 1, size=B, endpoint=True).astype(np.int32)
        pf = rng.uniform(0.0, 1.0, size=B).astype(np.float32)
        from workloads.synth import f32_to_bits

        p = f32_to_bits(pf, dtype)
        for use_k in (True, False):
            got = apply_fn(xb, dtype, p, k if use_k else None)
            for b in range(B):
                x = list(_vals(xb[b], dtype))
                keep, amb = expected_keep_bruteforce(x, int(k[b]) if use_k else None, _t32(p[b], dtype))
                if amb:
                    continue
                exp = np.where(keep, xb[b], NEG_INF_WORD[dtype]).astype(xb.dtype)
                assert np.array_equal(got[b], exp), (kind, b, use_k)


def check_invariants(apply_fn, dtype="bf16", V=300, B=16):
    from workloads.synth import f32_to_bits

    rng = np.random.default_rng(5)
    for kind in ("normal", "ties", "zeros", "spikes", "const"):
        xb = random_rows(3000 + V, B, V, dtype, kind=kind)
        vals = _vals(xb, dtype).reshape(B, V)
        k = rng.integers(1, V - 1, size=B, endpoint=True).astype(np.int32)
        p = f32_to_bits(rng.uniform(0.0, 1.0, size=B).astype(np.float32), dtype)
        neg = NEG_INF_WORD[dtype]
        out = apply_fn(xb, dtype, p, k)
        for b in range(B):
            kept = out[b] != neg
            # at least one survivor; kept bits are the input bits
            assert kept.any()
            assert np.array_equal(out[b][kept], xb[b][kept])
            # survivors form a suffix of the stable ascending order
            order = sorted(range(V), key=lambda i: (vals[b, i], i))
            flags = kept[order]
            first = int(np.argmax(flags))
            assert flags[first:].all(), (kind, b)
        # p = 0 keeps exactly the last sorted position (max, highest index)
        p0 = f32_to_bits(np.zeros(B, np.float32), dtype)
        out0 = apply_fn(xb, dtype, p0, None)
        for b in range(B):
            kept = np.nonzero(out0[b] != neg)[0]
            mx = vals[b].max()
            assert list(kept) == [int(np.nonzero(vals[b] == mx)[0].max())], (kind, b)
        # k = 1 without p keeps the max and all its ties
        out1 = apply_fn(xb, dtype, None, np.ones(B, np.int32))
        for b in range(B):
            assert np.array_equal(out1[b] != neg, vals[b] == vals[b].max()), (kind, b)
        # disabled k values agree with each other and with k absent
        outs = [apply_fn(xb, dtype, p, np.full(B, kk, np.int32)) for kk in (0, -3, V, V + 5)]
        ref = apply_fn(xb, dtype, p, None)
        for o in outs:
            assert np.array_equal(o, ref), kind
        # p = 1 (t = 0) with k equals k alone when no probability underflows
        p1 = f32_to_bits(np.ones(B, np.float32), dtype)
        assert np.array_equal(apply_fn(xb, dtype, p1, k), apply_fn(xb, dtype, None, k)), kind


def check_permutation_equivariance(apply_fn, dtype="f32", V=200, B=8):
    from workloads.synth import f32_to_bits

    xb = random_rows(4000, B, V, dtype, kind="normal")
    rng = np.random.default_rng(9)
    k = rng.integers(1, V, size=B).astype(np.int32)
    p = f32_to_bits(rng.uniform(0.2, 0.99, size=B).astype(np.float32), dtype)
    out = apply_fn(xb, dtype, p, k)
    for trial in range(3):
        perm = rng.permutation(V)
        outp = apply_fn(xb[:, perm], dtype, p, k)
        for b in range(B):
            if len(set(xb[b].tolist())) != V:
                continue  # equivariance holds for distinct values only
            assert np.array_equal(outp[b], out[b][perm])


ALL_CHECKS = [
    check_hand_cases,
    check_topk_counting_random,
    check_nucleus_random,
    check_invariants,
    check_permutation_equivariance,
    check_bruteforce_tiny,
]


# ---------------------------------------------------------------- min-p ---
# The min-p stage of Ascend's "aclnnTopKTopPSampleV2" page masks positions
# whose probability is below the largest probability times min_p. The checks
# below use the equivalent logit-space form, x - max(x) >= ln(min_p) (the
# softmax normalisation cancels in the ratio), evaluated element by element
# with Python floats, and the page's special cases: min_p <= 0 skips the
# stage, min_p >= 1 keeps a single token with the maximum value. Each check
# takes ``apply_mp_fn(logits_bits, dtype, p_bits, k, min_p_bits) -> out_bits``.


def minp_keep_logit_space(x, mp):
    """Min-p survivors of a row by the logit-space rule; (keep, ambiguous)."""
    V = len(x)
    if mp is None or not (mp > 0.0):
        return np.ones(V, dtype=bool), False
    m = max(x)
    if mp >= 1.0:
        keep = np.zeros(V, dtype=bool)
        keep[max(i for i in range(V) if x[i] == m)] = True
        return keep, False
    ln_mp = math.log(mp)
    keep = np.array([(v - m) >= ln_mp for v in x])
    ambiguous = any(abs((v - m) - ln_mp) < 1e-9 for v in x)
    return keep, ambiguous


def check_minp_hand_cases(apply_mp_fn):
    for case in load_hand_cases("min_p_cases.txt"):
        got = apply_mp_fn(case.x, case.dtype, case.p, case.k, case.min_p)
        assert np.array_equal(got, case.expect), (case.name, got, case.expect)


def check_minp_bruteforce_tiny(apply_mp_fn, dtypes=("f32", "bf16"), n_rows=4, max_v=7):
    """Tiny rows: every k, a p grid and a min_p grid against counting, the
    nucleus walk and the logit-space rule, intersected."""
    from workloads.synth import f32_to_bits

    mp_grid = [-0.5, 0.0, 1e-3, 0.05, 0.2, 0.5, 0.9, 1.0, 1.5]
    p_grid = [None, 0.0, 0.35, 0.8, 1.0]
    seed = 500
    for dtype in dtypes:
        for V in range(1, max_v + 1):
            for kind in ("normal", "ties", "zeros"):
                seed += 1
                xb = random_rows(seed, n_rows, V, dtype, kind=kind, scale=1.5)
                for b in range(n_rows):
                    row = xb[b : b + 1]
                    x = list(_vals(row[0], dtype))
                    for kk in [None, -1, 1, 2, V - 1, V]:
                        for pv in p_grid:
                            for mpv in mp_grid:
                                mp_bits = f32_to_bits(np.array([mpv], np.float32), dtype)
                                mp = float(_vals(mp_bits, dtype)[0])
                                p_bits = None
                                t = None
                                if pv is not None:
                                    p_bits = f32_to_bits(np.array([pv], np.float32), dtype)
                                    t = _t32(p_bits[0], dtype)
                                k_arr = None if kk is None else np.array([kk], np.int32)
                                got = apply_mp_fn(row, dtype, p_bits, k_arr, mp_bits)[0]
                                keep_kp, amb1 = expected_keep_bruteforce(x, kk, t)
                                keep_m, amb2 = minp_keep_logit_space(x, mp)
                                if amb1 or amb2:
                                    continue
                                exp = np.where(keep_kp & keep_m, row[0], NEG_INF_WORD[dtype]).astype(row.dtype)
                                assert np.array_equal(got, exp), (dtype, V, kind, b, kk, pv, mpv, x, got, exp)


def check_minp_random(apply_mp_fn, dtype="f32", V=300, B=24):
    """Moderate rows with ties: min-p alone and with top-k / top-p."""
    from workloads.synth import f32_to_bits

    rng = np.random.default_rng(21)
    for kind in ("normal", "ties", "gumbel"):
        xb = random_rows(6000 + V, B, V, dtype, kind=kind)
        mp = f32_to_bits(np.exp(rng.uniform(-8.0, 0.0, size=B)).astype(np.float32), dtype)
        k = rng.integers(1, V - 1, size=B, endpoint=True).astype(np.int32)
        p = f32_to_bits(rng.uniform(0.0, 1.0, size=B).astype(np.float32), dtype)
        for pp, kk in ((None, None), (None, k), (p, None), (p, k)):
            got = apply_mp_fn(xb, dtype, pp, kk, mp)
            for b in range(B):
                x = list(_vals(xb[b], dtype))
                t = None if pp is None else _t32(pp[b], dtype)
                keep_kp, amb1 = expected_keep_bruteforce(x, None if kk is None else int(kk[b]), t)
                keep_m, amb2 = minp_keep_logit_space(x, float(_vals(mp[b : b + 1], dtype)[0]))
                if amb1 or amb2:
                    continue
                exp = np.where(keep_kp & keep_m, xb[b], NEG_INF_WORD[dtype]).astype(xb.dtype)
                assert np.array_equal(got[b], exp), (kind, b, pp is None, kk is None)


def check_minp_invariants(apply_mp_fn, dtype="bf16", V=257, B=16):
    """At least one survivor; min_p >= 1 keeps exactly one position; min_p <= 0
    changes nothing; larger min_p keeps a subset."""
    from workloads.synth import f32_to_bits

    rng = np.random.default_rng(23)
    neg = NEG_INF_WORD[dtype]
    for kind in ("ties", "spikes", "const", "zeros"):
        xb = random_rows(7000 + V, B, V, dtype, kind=kind)
        vals = _vals(xb, dtype).reshape(B, V)
        k = rng.integers(1, V - 1, size=B, endpoint=True).astype(np.int32)
        p = f32_to_bits(rng.uniform(0.0, 1.0, size=B).astype(np.float32), dtype)
        ones = f32_to_bits(np.ones(B, np.float32), dtype)
        out1 = apply_mp_fn(xb, dtype, None, None, ones)
        for b in range(B):
            kept = np.nonzero(out1[b] != neg)[0]
            mx = vals[b].max()
            assert list(kept) == [int(np.nonzero(vals[b] == mx)[0].max())], (kind, b)
        for pp, kk in ((p, k), (p, None), (None, k)):
            base = apply_mp_fn(xb, dtype, pp, kk, None)
            for z in (0.0, -2.0):
                zb = f32_to_bits(np.full(B, z, np.float32), dtype)
                assert np.array_equal(apply_mp_fn(xb, dtype, pp, kk, zb), base), kind
            prev = base != neg
            for mpv in (1e-4, 0.01, 0.1, 0.5, 0.99):
                mb = f32_to_bits(np.full(B, mpv, np.float32), dtype)
                cur = apply_mp_fn(xb, dtype, pp, kk, mb) != neg
                assert cur.any(axis=1).all()
                assert not (cur & ~prev).any(), (kind, mpv)
                prev = cur


MINP_CHECKS = [
    check_minp_hand_cases,
    check_minp_invariants,
    check_minp_random,
    check_minp_bruteforce_tiny,
]


# ------------------------------------------------------------- sampling ---
# Sampling after the filter ("Subsequent processing" of the TKS page). Each
# check takes ``sample_fn(logits_bits, dtype, p_bits, k, min_p_bits, q, eps)
# -> selected int array``. The facts used: hand-derived cases
# (tests/golden/sample_cases.txt); brute force with the survivors from
# counting, the nucleus walk and the logit-space min-p rule, and the ranks
# from sorting (value, index) pairs in descending order; and the exponential
# race theorem: with q drawn i.i.d. from Exp(1), argmax_r prob_r / q_r picks
# each survivor with probability equal to its probability renormalised over
# the survivors.


def check_sample_hand_cases(sample_fn):
    for case in load_hand_cases("sample_cases.txt"):
        got = sample_fn(case.x, case.dtype, case.p, case.k, case.min_p, case.q, case.eps)
        assert np.array_equal(np.asarray(got), case.expect_idx), (case.name, got, case.expect_idx)


def _expected_sample(x, kk, t, mp, q_row, eps):
    """Brute-force pick; (index or None when ambiguous)."""
    keep_kp, amb1 = expected_keep_bruteforce(x, kk, t)
    keep_m, amb2 = minp_keep_logit_space(x, mp)
    if amb1 or amb2:
        return None
    keep = keep_kp & keep_m
    order = sorted(range(len(x)), key=lambda i: (x[i], i), reverse=True)  # descending rank -> index
    m = x[order[0]]
    if q_row is None:
        return order[0]
    scores = []
    for r, i in enumerate(order):
        scores.append(math.exp(x[i] - m) / (q_row[r] + eps) if keep[i] else -1.0)
    best = max(scores)
    near = [s for s in scores if s >= 0 and abs(s - best) <= 1e-9 * max(best, 1e-300) and s != best]
    if near:
        return None
    return order[scores.index(best)]


def check_sample_bruteforce_tiny(sample_fn, dtypes=("f32", "bf16"), n_rows=4, max_v=7):
    from workloads.synth import f32_to_bits

    rng = np.random.default_rng(41)
    seed = 900
    for dtype in dtypes:
        for V in range(2, max_v + 1):
            for kind in ("normal", "ties"):
                seed += 1
                xb = random_rows(seed, n_rows, V, dtype, kind=kind, scale=1.5)
                for b in range(n_rows):
                    row = xb[b : b + 1]
                    x = list(_vals(row[0], dtype))
                    for kk in (None, 1, 2, V - 1):
                        for pv in (None, 0.5, 0.9):
                            for mpv in (None, 0.1):
                                for use_q in (False, True):
                                    if kk is None and pv is None and mpv is None:
                                        continue
                                    q = rng.exponential(1.0, size=(1, V)) if use_q else None
                                    eps = 1e-6
                                    p_bits = None if pv is None else f32_to_bits(np.array([pv], np.float32), dtype)
                                    t = None if pv is None else _t32(p_bits[0], dtype)
                                    mp_bits = None if mpv is None else f32_to_bits(np.array([mpv], np.float32), dtype)
                                    mp = None if mpv is None else float(_vals(mp_bits, dtype)[0])
                                    k_arr = None if kk is None else np.array([kk], np.int32)
                                    exp = _expected_sample(x, kk, t, mp, None if q is None else q[0], eps)
                                    if exp is None:
                                        continue
                                    got = sample_fn(row, dtype, p_bits, k_arr, mp_bits, q, eps)
                                    assert int(got[0]) == exp, (dtype, V, kind, b, kk, pv, mpv, use_q, x, got, exp)


def check_sample_race_distribution(sample_fn, draws=20000):
    """With q ~ Exp(1), the pick frequencies match the survivors' renormalised
    probabilities (each within 4.5 standard errors)."""
    from workloads.synth import f32_to_bits

    x = np.array([0.0, 1.0, 1.5, -2.0, 2.0, 0.5], np.float32)
    V = len(x)
    k = 4  # keeps 2.0, 1.5, 1.0, 0.5
    xb = np.repeat(f32_to_bits(x, "f32")[None, :], draws, axis=0)
    rng = np.random.default_rng(12345)
    q = rng.exponential(1.0, size=(draws, V))
    got = np.asarray(sample_fn(xb, "f32", None, np.full(draws, k, np.int32), None, q, 0.0))
    kept = [4, 2, 1, 5]
    w = np.exp(x[kept].astype(np.float64) - 2.0)
    w /= w.sum()
    for i, pi in zip(kept, w):
        f = np.mean(got == i)
        se = math.sqrt(pi * (1 - pi) / draws)
        assert abs(f - pi) <= 4.5 * se, (i, f, pi)
    assert np.isin(got, kept).all()


def check_sample_none_is_top(sample_fn, dtype="bf16", V=300, B=12):
    """Without q the pick is the maximum value with the highest index."""
    from workloads.synth import f32_to_bits

    rng = np.random.default_rng(43)
    for kind in ("ties", "normal", "const"):
        xb = random_rows(8000 + V, B, V, dtype, kind=kind)
        k = rng.integers(1, V - 1, size=B, endpoint=True).astype(np.int32)
        p = f32_to_bits(rng.uniform(0.0, 1.0, size=B).astype(np.float32), dtype)
        got = np.asarray(sample_fn(xb, dtype, p, k, None, None, 0.0))
        vals = _vals(xb, dtype).reshape(B, V)
        for b in range(B):
            mx = vals[b].max()
            assert int(got[b]) == int(np.nonzero(vals[b] == mx)[0].max()), (kind, b)


SAMPLE_CHECKS = [
    check_sample_hand_cases,
    check_sample_none_is_top,
    check_sample_bruteforce_tiny,
    check_sample_race_distribution,
]


# ----------------------------------------------------- sorted survivors ---
# Each check takes ``surv_fn(logits_bits, dtype, p_bits, k, min_p_bits, cap)
# -> (probs [B, cap], indices [B, cap], counts [B])``. The facts used:
# hand-derived cases (tests/golden/survivor_cases.txt); the brute-force
# survivor sets (counting, the nucleus walk, the logit-space min-p rule)
# ordered by sorting (value, index) pairs in descending order; and the
# closed form that, without top-p and min-p, the listed probabilities are a
# softmax over exactly the listed values (they sum to 1 and their ratios are
# exp of the value differences).


def check_survivor_hand_cases(surv_fn):
    for case in load_hand_cases("survivor_cases.txt"):
        probs, idx, cnt = surv_fn(case.x, case.dtype, case.p, case.k, case.min_p, case.cap)
        assert np.array_equal(np.asarray(idx), case.expect_idx), (case.name, idx)
        assert np.allclose(np.asarray(probs), case.expect_probs, atol=6e-5), (case.name, probs)
        assert np.array_equal(np.asarray(cnt), case.expect_count), (case.name, cnt)


def check_survivor_bruteforce_tiny(surv_fn, dtypes=("f32", "bf16"), n_rows=4, max_v=7):
    from workloads.synth import f32_to_bits

    seed = 1400
    for dtype in dtypes:
        for V in range(2, max_v + 1):
            for kind in ("normal", "ties", "zeros"):
                seed += 1
                xb = random_rows(seed, n_rows, V, dtype, kind=kind, scale=1.5)
                for b in range(n_rows):
                    row = xb[b : b + 1]
                    x = list(_vals(row[0], dtype))
                    for kk in (None, 1, 2, V - 1):
                        for pv in (None, 0.5, 0.9):
                            for mpv in (None, 0.2):
                                if kk is None and pv is None and mpv is None:
                                    continue
                                p_bits = None if pv is None else f32_to_bits(np.array([pv], np.float32), dtype)
                                t = None if pv is None else _t32(p_bits[0], dtype)
                                mp_bits = None if mpv is None else f32_to_bits(np.array([mpv], np.float32), dtype)
                                mp = None if mpv is None else float(_vals(mp_bits, dtype)[0])
                                keep_kp, amb1 = expected_keep_bruteforce(x, kk, t)
                                keep_m, amb2 = minp_keep_logit_space(x, mp)
                                if amb1 or amb2:
                                    continue
                                keep = keep_kp & keep_m
                                order = [i for i in sorted(range(V), key=lambda i: (x[i], i), reverse=True) if keep[i]]
                                cap = V + 1
                                _, idx, cnt = surv_fn(row, dtype, p_bits, None if kk is None else np.array([kk], np.int32),
                                                      mp_bits, cap)
                                exp = order + [-1] * (cap - len(order))
                                assert list(np.asarray(idx)[0]) == exp, (dtype, V, kind, b, kk, pv, mpv, x, idx)
                                assert int(np.asarray(cnt)[0]) == len(order)


def check_survivor_softmax_closed_form(surv_fn, dtype="f32", V=200, B=10):
    rng = np.random.default_rng(47)
    xb = random_rows(9100, B, V, dtype, kind="normal")
    k = rng.integers(1, V - 1, size=B, endpoint=True).astype(np.int32)
    probs, idx, cnt = (np.asarray(a) for a in surv_fn(xb, dtype, None, k, None, V))
    vals = _vals(xb, dtype).reshape(B, V)
    for b in range(B):
        n = int(cnt[b])
        assert abs(probs[b, :n].sum() - 1.0) <= 1e-9, b
        v = vals[b, idx[b, :n]]
        ratio = probs[b, :n] / probs[b, 0]
        assert np.allclose(ratio, np.exp(v - v[0]), rtol=1e-9), b
        assert np.all(np.diff(v) <= 0), b


SURVIVOR_CHECKS = [
    check_survivor_hand_cases,
    check_survivor_softmax_closed_form,
    check_survivor_bruteforce_tiny,
]
