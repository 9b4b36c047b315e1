"""The min-p stage on the HIP path vs the CPU oracle, through the C ABI
(needs an MI355X). Min-p follows the "minP sampling" stage of Ascend's
aclnnTopKTopPSampleV2 page; the oracle and its pins define it."""

import numpy as np
import pytest

from oracle import apply_top_k_top_p as oracle_apply
from oracle import apply_top_k_top_p_with_sorted as oracle_sorted
from tests.golden_io import load_hand_cases
from tests.gpu_util import gpu_apply, gpu_with_sorted, need_gpu, say
from tests.parity import NEG_INF_WORD, ParityReport, compare
from workloads.synth import (
    f32_to_bits,
    make_workload,
    min_p_for_workload,
    random_min_p,
    random_params,
    random_rows,
    stable_ascending_sort,
)

pytestmark = pytest.mark.gpu

POLICIES = {"auto": 0, "multipass": 1, "stream": 2}


@pytest.fixture(params=sorted(POLICIES), scope="module")
def policy(request):
    need_gpu()
    import top_logits_filtering_amd as tk

    prev = tk.set_plan_policy(POLICIES[request.param])
    yield request.param
    tk.set_plan_policy(prev)


def test_min_p_hand_cases(policy):
    for case in load_hand_cases("min_p_cases.txt"):
        got = gpu_apply(case.x, case.dtype, case.p, case.k, case.min_p)
        assert np.array_equal(got, case.expect), (policy, case.name, got, case.expect)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_min_p_random_rows(dtype, policy):
    """Several tiles and ragged tails; min-p alone and with top-k / top-p."""
    total = ParityReport()
    seed = {"f32": 1, "f16": 2, "bf16": 3}[dtype] * 1000
    for V in (2, 7, 1000, 4099, 20011, 170001):
        for kind in ("normal", "ties", "gumbel", "spikes", "const"):
            seed += 1
            B = 6 if V < 20000 else 3
            xb = random_rows(seed, B, V, dtype, kind=kind)
            k, p = random_params(seed, B, V, dtype)
            mp = random_min_p(seed, B, dtype)
            for pp, kk in ((None, None), (None, k), (p, None), (p, k)):
                got = gpu_apply(xb, dtype, pp, kk, mp)
                ref = oracle_apply(xb, dtype, pp, kk, min_p_bits=mp)
                rep = compare(got, xb, ref, dtype)
                assert rep.hard_mismatches == 0, (V, kind, pp is None, kk is None, rep.details[:2])
                total.merge(rep)
    say(f"min-p {dtype}/{policy}: {total}")


def test_min_p_extremes(policy):
    """min_p <= 0, tiny, near 1, exactly 1, above 1; with and without k / p."""
    dtype = "bf16"
    V = 3001
    xb = random_rows(57, 8, V, dtype, kind="ties")
    for mpv in (-1.0, 0.0, 1e-30, 1e-6, 0.01, 0.5, 0.999, 1.0, 1.5):
        mp = f32_to_bits(np.full(8, mpv, np.float32), dtype)
        for pv, kv in ((None, None), (0.9, None), (None, 50), (0.5, 200), (0.0, None), (None, 1)):
            p = None if pv is None else f32_to_bits(np.full(8, pv, np.float32), dtype)
            k = None if kv is None else np.full(8, kv, np.int32)
            got = gpu_apply(xb, dtype, p, k, mp)
            ref = oracle_apply(xb, dtype, p, k, min_p_bits=mp)
            rep = compare(got, xb, ref, dtype)
            assert rep.hard_mismatches == 0, (mpv, pv, kv, rep.details[:2])


def test_min_p_absent_matches_plain_entry():
    """A NULL min_p gives the plain entry point's output."""
    need_gpu()
    wl = make_workload(3, rows=range(24))
    a = gpu_apply(wl.logits, wl.dtype, wl.p, wl.k)
    zeros = f32_to_bits(np.zeros(wl.B, np.float32), wl.dtype)
    b = gpu_apply(wl.logits, wl.dtype, wl.p, wl.k, zeros)  # min_p = 0: the stage is skipped
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_min_p_with_sorted(dtype):
    """Pre-sorted rows: the shared-memory copy of the top values (small k),
    the global search (p only, min-p only), with and without logits."""
    need_gpu()
    total = ParityReport()
    seed = 1700
    for V, kind in ((5, "normal"), (1000, "ties"), (70001, "normal"), (70001, "ties"), (262144, "normal")):
        seed += 1
        B = 4
        xb = random_rows(seed, B, V, dtype, kind=kind, scale=3.0)
        idx, sv = stable_ascending_sort(xb, dtype)
        k, p = random_params(seed, B, V, dtype, k_lo=1, k_hi=min(V, 4096))
        mp = random_min_p(seed, B, dtype)
        for pp, kk in ((None, None), (None, k), (p, None), (p, k)):
            ref = oracle_sorted(sv, idx, dtype, pp, kk, logits_bits=xb, min_p_bits=mp)
            for use_logits in (True, False):
                got = gpu_with_sorted(sv, idx, dtype, pp, kk, xb if use_logits else None, mp)
                rep = compare(got, xb, ref, dtype)
                assert rep.hard_mismatches == 0, (V, kind, use_logits, pp is None, kk is None, rep.details[:2])
                total.merge(rep)
    say(f"with_sorted min-p {dtype}: {total}")


def test_min_p_workload3_sampled(policy):
    """The timed shape (B=256, V=151936, bf16, mixed modes) with a min_p per
    row: the oracle on sampled rows, properties on every row."""
    wl = make_workload(3)
    mp = min_p_for_workload(3, wl.B, wl.dtype)
    got = gpu_apply(wl.logits, wl.dtype, wl.p, wl.k, mp)
    rows = np.array([0, 1, 2, 3, 4, 5, 100, 101, 102, wl.B - 1])
    ref = oracle_apply(wl.logits[rows], wl.dtype, wl.p[rows], wl.k[rows], min_p_bits=mp[rows])
    rep = compare(got[rows], wl.logits[rows], ref, wl.dtype, row_ids=rows)
    say(f"workload 3 + min-p sampled ({policy}): {rep}")
    assert rep.hard_mismatches == 0, rep.details[:3]
    # every row: kept bits are inputs, at least one survivor, and min-p alone
    # never keeps less than the min-p rule in logit space
    neg = NEG_INF_WORD[wl.dtype]
    assert np.all((got == wl.logits) | (got == neg))
    assert (got != neg).any(axis=1).all()
    plain = gpu_apply(wl.logits, wl.dtype, wl.p, wl.k)
    assert not ((got != neg) & (plain == neg)).any(), "min-p revived a position"
