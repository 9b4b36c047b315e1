"""The CPU oracle against its pins (no GPU needed)."""

import numpy as np
import pytest

from oracle import apply_top_k_top_p, apply_top_k_top_p_with_sorted
from tests import oracle_pins as pins
from workloads.synth import bits_to_f32, make_workload, random_rows, split_modes, stable_ascending_sort


def oracle_apply(x, dtype, p, k):
    return apply_top_k_top_p(x, dtype, p, k, keep_traces=False).out


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pins(check):
    check(oracle_apply)


def oracle_apply_mp(x, dtype, p, k, min_p):
    return apply_top_k_top_p(x, dtype, p, k, keep_traces=False, min_p_bits=min_p).out


@pytest.mark.parametrize("check", pins.MINP_CHECKS, ids=lambda c: c.__name__)
def test_oracle_min_p_pins(check):
    check(oracle_apply_mp)


def oracle_sample(x, dtype, p, k, min_p, q, eps):
    from oracle import sample_top_k_top_p

    return sample_top_k_top_p(x, dtype, p, k, min_p, q, eps).selected


@pytest.mark.parametrize("check", pins.SAMPLE_CHECKS, ids=lambda c: c.__name__)
def test_oracle_sample_pins(check):
    check(oracle_sample)


def oracle_survivors(x, dtype, p, k, min_p, cap):
    from oracle import sorted_survivors

    r = sorted_survivors(x, dtype, p, k, min_p, cap)
    return r.probs, r.indices, r.counts


@pytest.mark.parametrize("check", pins.SURVIVOR_CHECKS, ids=lambda c: c.__name__)
def test_oracle_survivor_pins(check):
    check(oracle_survivors)


def test_min_p_absent_equals_before():
    """Without min-p the oracle's output is unchanged by the min-p code path."""
    xb = random_rows(88, 6, 200, "bf16", kind="ties")
    k, p = pins_params(6, 200, "bf16")
    a = apply_top_k_top_p(xb, "bf16", p, k, keep_traces=False).out
    b = apply_top_k_top_p(xb, "bf16", p, k, keep_traces=False, min_p_bits=None).out
    assert np.array_equal(a, b)


def test_with_sorted_min_p_matches_apply():
    """The pre-sorted entry with min-p equals the sorting entry with min-p."""
    from workloads.synth import f32_to_bits

    for dtype, kind in (("bf16", "normal"), ("f32", "ties")):
        xb = random_rows(79, 10, 301, dtype, kind=kind)
        k, p = pins_params(10, 301, dtype)
        mp = f32_to_bits(np.linspace(-0.1, 1.1, 10).astype(np.float32), dtype)
        ref = apply_top_k_top_p(xb, dtype, p, k, keep_traces=False, min_p_bits=mp).out
        idx, sv = stable_ascending_sort(xb, dtype)
        for logits in (xb, None):
            got = apply_top_k_top_p_with_sorted(sv, idx, dtype, p, k, logits_bits=logits, min_p_bits=mp).out
            assert np.array_equal(got, ref)


def test_with_sorted_matches_apply():
    """Pre-sorted entry on a stable sort equals the sorting entry (both forms)."""
    for dtype, kind in (("bf16", "normal"), ("f32", "ties"), ("f16", "zeros")):
        xb = random_rows(77, 12, 333, dtype, kind=kind)
        k, p = pins_params(12, 333, dtype)
        ref = oracle_apply(xb, dtype, p, k)
        idx, sv = stable_ascending_sort(xb, dtype)
        a = apply_top_k_top_p_with_sorted(sv, idx, dtype, p, k, logits_bits=xb).out
        b = apply_top_k_top_p_with_sorted(sv, idx, dtype, p, k, logits_bits=None).out
        assert np.array_equal(a, ref)
        assert np.array_equal(b, ref)


def pins_params(B, V, dtype):
    from workloads.synth import random_params

    return random_params(B * 1000 + V, B, V, dtype)


def test_cumsum_numerics():
    """The float64 cumsum ends at 1 and never decreases."""
    for c in (1, 2, 3):
        wl = make_workload(c, rows=range(3))
        res = apply_top_k_top_p(wl.logits, wl.dtype, wl.p, wl.k)
        for tr in res.traces:
            if tr.probs_sum32 is None:
                continue
            assert np.all(np.diff(tr.probs_sum32.astype(np.float64)) >= 0)
            assert abs(float(tr.probs_sum32[-1]) - 1.0) <= 1e-6


def test_errors():
    x = np.zeros((1, 4), np.uint32)
    with pytest.raises(ValueError):
        apply_top_k_top_p(x, "f32", None, None)
    with pytest.raises(ValueError):
        apply_top_k_top_p(x, "f64", None, np.ones(1, np.int32))


def test_empty_and_single_column():
    x = np.zeros((0, 5), np.uint16)
    assert apply_top_k_top_p(x, "bf16", None, np.ones(0, np.int32)).out.shape == (0, 5)
    x1 = random_rows(3, 4, 1, "bf16")
    out = oracle_apply(x1, "bf16", np.zeros(4, np.uint16), np.ones(4, np.int32))
    assert np.array_equal(out, x1)


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
def test_workload_invariants(c):
    """Invariants on a few real rows of every workload."""
    wl = make_workload(c, rows=[0, 1, 2, 3])
    neg = {"f32": 0xFF800000, "f16": 0xFC00, "bf16": 0xFF80}[wl.dtype]
    if wl.entry == "apply":
        res = apply_top_k_top_p(wl.logits, wl.dtype, wl.p, wl.k)
    else:
        res = apply_top_k_top_p_with_sorted(wl.sorted_value, wl.sorted_indices, wl.dtype, wl.p, wl.k,
                                            logits_bits=wl.logits)
        ref = apply_top_k_top_p(wl.logits, wl.dtype, wl.p, wl.k, keep_traces=False).out
        assert np.array_equal(res.out, ref)
    vals = bits_to_f32(wl.logits, wl.dtype).reshape(wl.B, wl.V)
    for b in range(wl.B):
        kept = res.out[b] != neg
        assert kept.any()
        assert np.array_equal(res.out[b][kept], wl.logits[b][kept])
        assert kept[int(np.argmax(vals[b]))] or vals[b][kept].max() == vals[b].max()
        if wl.k is not None and 1 <= wl.k[b] <= wl.V - 1:
            # top-k survivors are at least k and include every value above the threshold
            assert kept.sum() <= np.count_nonzero(vals[b] >= np.sort(vals[b])[wl.V - wl.k[b]])


def test_workload3_modes_match_null_calls():
    """Workload 3's single call (k=0 / p=1 stand-ins) equals calls with absent p / k."""
    wl = make_workload(3, rows=range(6))
    full = oracle_apply(wl.logits, wl.dtype, wl.p, wl.k)
    for pos, p, k in split_modes(wl):
        sub = apply_top_k_top_p(wl.logits[pos], wl.dtype, p, k, keep_traces=False).out
        assert np.array_equal(sub, full[pos])


def test_t_readings_report():
    """The two readings of 1 - p agree for fp32 p >= 0.5 and differ only below (reported)."""
    from oracle import one_minus_p
    from workloads.synth import f32_to_bits

    for pv in (0.5, 0.6, 0.75, 0.9, 0.99):
        for dtype in ("bf16", "f16"):
            pb = f32_to_bits(np.array([pv], np.float32), dtype)[0]
            assert one_minus_p(pb, dtype, "fp32") == one_minus_p(pb, dtype, "dtype")


def test_t_reading_dtype_hand_rounded():
    """The other reading of step 6 (1 - p rounded to p's dtype, AKP §2 step 6
    with p in the logits dtype, §3) against values rounded by hand. Both
    readings agree for p >= 0.5 (above); below 0.5, 1 - p needs one bit more
    than the dtype holds:
      bf16 0x3E9B = 0.302734375: 1 - p = 0.697265625 = 178.5 * 2^-8, a tie,
        rounds to even 178 * 2^-8 = 0.6953125;
      bf16 0x3DCD = 0.10009765625: 1 - p = 0.89990234375 = 230.375 * 2^-8
        rounds to 230 * 2^-8 = 0.8984375;
      fp16 0x34CD = 1229 * 2^-12: 1 - p = 2867 * 2^-12 = 1433.5 * 2^-11, a tie,
        rounds to even 1434 * 2^-11 = 0.7001953125;
      fp16 0x2E66 = 1638 * 2^-14: 1 - p = 14746 * 2^-14 = 1843.25 * 2^-11
        rounds to 1843 * 2^-11 = 0.89990234375."""
    from oracle import one_minus_p

    cases = [("bf16", 0x3E9B, 0.697265625, 0.6953125), ("bf16", 0x3DCD, 0.89990234375, 0.8984375),
             ("f16", 0x34CD, 0.699951171875, 0.7001953125), ("f16", 0x2E66, 0.9000244140625, 0.89990234375)]
    for dtype, bits, t32, tdt in cases:
        assert one_minus_p(bits, dtype, "fp32") == np.float32(t32), (dtype, hex(bits))
        assert one_minus_p(bits, dtype, "dtype") == np.float32(tdt), (dtype, hex(bits))


def test_t_reading_changes_mask_on_flat_row():
    """A row of 1000 equal values has cumulative probabilities (j + 1) / 1000,
    and ties survive from the highest index down. bf16 p = 0x3E9B: the fp32
    reading t = 0.697265625 masks ranks with j + 1 <= 697 and keeps the 303
    highest indices; the dtype reading t = 0.6953125 keeps 305. fp16 p =
    0x34CD: t = 0.699951171875 keeps 301, the dtype reading 0.7001953125
    keeps 300."""
    for dtype, pbits, keep32, keepdt in (("bf16", 0x3E9B, 303, 305), ("f16", 0x34CD, 301, 300)):
        x = np.zeros((1, 1000), np.uint16)  # +0.0 in both dtypes
        p = np.array([pbits], np.uint16)
        for reading, keep in (("fp32", keep32), ("dtype", keepdt)):
            out = apply_top_k_top_p(x, dtype, p, None, keep_traces=False, t_reading=reading).out[0]
            kept = np.nonzero(out == 0)[0]
            assert np.array_equal(kept, np.arange(1000 - keep, 1000)), (dtype, reading, len(kept))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_neg_inf_entries_are_zero_probability(dtype):
    """-inf entries have probability zero and sit below every finite value in
    the stable order, so removing them from a row leaves the decisions on the
    finite entries unchanged (with k at most the number of finite entries),
    and the -inf positions come out as -inf."""
    neg = {"f32": 0xFF800000, "f16": 0xFC00, "bf16": 0xFF80}[dtype]
    rng = np.random.default_rng(5)
    for trial in range(12):
        V = int(rng.integers(3, 400))
        xb = random_rows(900 + trial, 1, V, dtype, kind=("normal", "ties", "gumbel")[trial % 3])
        n_fin = int(rng.integers(1, V))
        fin = np.sort(rng.permutation(V)[:n_fin])
        full = np.full_like(xb, neg)
        full[0, fin] = xb[0, fin]
        comp = np.ascontiguousarray(xb[:, fin])
        p = xb[:, :1].copy()
        p[0, 0] = {"f32": np.float32(0.7).view(np.uint32), "f16": np.float16(0.7).view(np.uint16),
                   "bf16": np.uint16(np.float32(0.7).view(np.uint32) >> 16)}[dtype]
        p = p[:, 0]
        for k in (None, np.array([int(rng.integers(1, n_fin + 1))], np.int32)):
            a = apply_top_k_top_p(full, dtype, p, k).out
            c = apply_top_k_top_p(comp, dtype, p, k).out
            assert np.array_equal(a[0, fin], c[0]), (dtype, trial, k)
            rest = np.setdiff1d(np.arange(V), fin)
            assert (a[0, rest] == neg).all()
