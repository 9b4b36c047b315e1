"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X). Every row
of the five workloads is compared in tests/test_gpu_workloads_full.py; the
tests here cover the branch points of each plan on smaller inputs."""

import numpy as np
import pytest

from oracle import apply_top_k_top_p as oracle_apply
from oracle import apply_top_k_top_p_with_sorted as oracle_sorted
from tests.golden_io import load_hand_cases
from tests.gpu_util import gpu_apply, gpu_with_sorted, need_gpu, say
from tests.parity import ParityReport, compare
from workloads.synth import f32_to_bits, make_workload, random_params, random_rows, split_modes, stable_ascending_sort

pytestmark = pytest.mark.gpu

POLICIES = {"auto": 0, "multipass": 1, "stream": 2}


@pytest.fixture(params=sorted(POLICIES), scope="module")
def policy(request):
    need_gpu()
    import top_logits_filtering_amd as tk

    prev = tk.set_plan_policy(POLICIES[request.param])
    yield request.param
    tk.set_plan_policy(prev)


def _check(rep: ParityReport, what):
    say(f"{what}: {rep}")
    assert rep.hard_mismatches == 0, rep.details[:3]


def test_hand_cases(policy):
    for case in load_hand_cases():
        got = gpu_apply(case.x, case.dtype, case.p, case.k)
        assert np.array_equal(got, case.expect), (policy, case.name, got, case.expect)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_random_rows(dtype, policy):
    """Several tiles plus ragged tails, every mode, odd k and p values."""
    total = ParityReport()
    seed = {"f32": 1, "f16": 2, "bf16": 3}[dtype] * 100
    for V in (2, 3, 7, 64, 1000, 1031, 4099, 20011, 70001, 170001):
        for kind in ("normal", "ties", "zeros", "gumbel", "spikes", "const", "wide"):
            seed += 1
            B = 6 if V < 20000 else (3 if V < 100000 else 2)
            xb = random_rows(seed, B, V, dtype, kind=kind)
            k, p = random_params(seed, B, V, dtype)
            k_small = np.minimum(np.abs(k), max(1, V // 3)).astype(np.int32)
            for pp, kk in ((None, k), (p, None), (p, k), (p, k_small)):
                got = gpu_apply(xb, dtype, pp, kk)
                ref = oracle_apply(xb, dtype, pp, kk)
                rep = compare(got, xb, ref, dtype)
                assert rep.hard_mismatches == 0, (V, kind, pp is None, kk is None, rep.details[:2])
                total.merge(rep)
    say(f"{dtype}/{policy}: {total}")


def test_extreme_p_and_k(policy):
    """p <= 0, p >= 1, p > 1, k = 1, k = V-1, k out of range."""
    dtype = "bf16"
    V = 3001
    xb = random_rows(55, 8, V, dtype, kind="ties")
    for pv in (-0.5, 0.0, 1e-7, 0.999999, 1.0, 1.5):
        for kv in (None, 1, 2, V - 1, V, 0, -4):
            p = None if pv is None else f32_to_bits(np.full(8, pv, np.float32), dtype)
            k = None if kv is None else np.full(8, kv, np.int32)
            got = gpu_apply(xb, dtype, p, k)
            ref = oracle_apply(xb, dtype, p, k)
            _check(compare(got, xb, ref, dtype), f"p={pv} k={kv}")


def test_single_column_and_empty():
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    xb = random_rows(9, 5, 1, "f32")
    got = gpu_apply(xb, "f32", np.zeros(5, np.uint32), np.ones(5, np.int32))
    assert np.array_equal(got, xb)
    empty = torch.empty((0, 7), device="cuda", dtype=torch.bfloat16)
    assert tk.apply_top_k_top_p(empty, None, torch.ones(0, dtype=torch.int32, device="cuda")).shape == (0, 7)


def test_workload3_absent_p_and_k():
    """The three modes called with truly absent p / k match the single timed call."""
    need_gpu()
    wl = make_workload(3, rows=range(30))
    full = gpu_apply(wl.logits, wl.dtype, wl.p, wl.k)
    for pos, p, k in split_modes(wl):
        sub = gpu_apply(wl.logits[pos], wl.dtype, p, k)
        assert np.array_equal(sub, full[pos])


def test_determinism():
    need_gpu()
    wl = make_workload(3, rows=range(64))
    a = gpu_apply(wl.logits, wl.dtype, wl.p, wl.k)
    b = gpu_apply(wl.logits, wl.dtype, wl.p, wl.k)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_with_sorted_random(dtype):
    need_gpu()
    total = ParityReport()
    seed = 900
    for V in (2, 5, 1000, 4099, 70001):
        for kind in ("normal", "ties", "zeros", "gumbel", "const"):
            seed += 1
            B = 5
            xb = random_rows(seed, B, V, dtype, kind=kind)
            k, p = random_params(seed, B, V, dtype)
            idx, sv = stable_ascending_sort(xb, dtype)
            for pp, kk in ((None, k), (p, None), (p, k)):
                ref = oracle_sorted(sv, idx, dtype, pp, kk, logits_bits=xb)
                for use_logits in (True, False):
                    got = gpu_with_sorted(sv, idx, dtype, pp, kk, xb if use_logits else None)
                    rep = compare(got, xb, ref, dtype)
                    assert rep.hard_mismatches == 0, (V, kind, use_logits, rep.details[:2])
                    total.merge(rep)
    say(f"with_sorted {dtype}: {total}")


@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("f32", 65536), ("f16", 32000)])
def test_candidate_plan_branch_points(dtype, V):
    """Rows held in registers, with k and p placed around the plan's branch
    points: candidate counts of about one wave (one-wave ranking up to 64),
    the one-pass joint selection, k beyond the 2048 per-thread maxima, and
    top-p boundaries inside runs of equal values (values on a 0.5 grid)."""
    total = ParityReport()
    seed = 900
    for scale in (1.0, 3.0):
        seed += 1
        xb = random_rows(seed, 2, V, dtype, kind="ties", scale=scale)
        for kv in (0, 1, 5, 40, 63, 64, 65, 100, 500, 1000, 2047, 2048, 2049, 3000):
            for pv in (None, 0.05, 0.5, 0.9, 0.99):
                k = np.full(2, kv, np.int32)
                p = None if pv is None else f32_to_bits(np.full(2, pv, np.float32), dtype)
                if p is None and kv == 0:
                    continue
                got = gpu_apply(xb, dtype, p, k)
                ref = oracle_apply(xb, dtype, p, k)
                rep = compare(got, xb, ref, dtype)
                assert rep.hard_mismatches == 0, (scale, kv, pv, rep.details[:2])
                total.merge(rep)
    say(f"{dtype} V={V}: {total}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_with_sorted_copy_boundary(dtype):
    """Pre-sorted rows around the shared-memory copy of the top values: k near
    the copy's reach (k + the tie margin against its size), long runs of equal
    values at the k-th largest (values on a 0.5 grid), whole rows that fit."""
    need_gpu()
    total = ParityReport()
    seed = 1300
    for V, kind in ((6144, "normal"), (70001, "normal"), (70001, "ties"), (262144, "normal")):
        seed += 1
        xb = random_rows(seed, 2, V, dtype, kind=kind, scale=3.0)
        idx, sv = stable_ascending_sort(xb, dtype)
        for kv in (1, 2, 50, 1000, 4095, 5119, 5120, 5121, 6000):
            for pv in (None, 0.3, 0.9):
                k = np.full(2, kv, np.int32)
                p = None if pv is None else f32_to_bits(np.full(2, pv, np.float32), dtype)
                ref = oracle_sorted(sv, idx, dtype, p, k, logits_bits=xb)
                got = gpu_with_sorted(sv, idx, dtype, p, k, xb)
                rep = compare(got, xb, ref, dtype)
                assert rep.hard_mismatches == 0, (V, kind, kv, pv, rep.details[:2])
                total.merge(rep)
    say(f"with_sorted copy boundary {dtype}: {total}")


@pytest.mark.parametrize("dtype,V", [("bf16", 262144), ("f32", 262144), ("bf16", 262143)])
def test_with_sorted_global_search_full_rows(dtype, V):
    """Pre-sorted rows whose boundary search reads global memory: top-p
    without k (the segmented two-level scan over the whole row), k beyond
    the shared-memory copy of the top values, and a length that is not a
    whole number of 16-byte vectors (one position per group)."""
    need_gpu()
    total = ParityReport()
    seed = 1700 + V % 7
    for kind in ("normal", "ties"):
        seed += 1
        xb = random_rows(seed, 3, V, dtype, kind=kind, scale=3.0)
        idx, sv = stable_ascending_sort(xb, dtype)
        for kv, pv in ((None, 0.5), (None, 0.99), (None, 0.02), (7000, 0.9), (200000, 0.999)):
            k = None if kv is None else np.full(3, kv, np.int32)
            p = f32_to_bits(np.full(3, pv, np.float32), dtype)
            ref = oracle_sorted(sv, idx, dtype, p, k, logits_bits=xb)
            for use_logits in (True, False):
                got = gpu_with_sorted(sv, idx, dtype, p, k, xb if use_logits else None)
                rep = compare(got, xb, ref, dtype)
                assert rep.hard_mismatches == 0, (kind, kv, pv, use_logits, rep.details[:2])
                total.merge(rep)
    say(f"with_sorted global search {dtype} V={V}: {total}")


@pytest.mark.parametrize("dtype,V", [("bf16", 65546), ("bf16", 200000), ("f32", 32771), ("f32", 98304),
                                     ("f16", 131080)])
def test_with_sorted_without_k_segment_table(dtype, V):
    """Pre-sorted rows without k, whose top-p boundary comes from the table of
    segment masses the pre-pass writes into each slice's output region; the
    last slice of 65546 bf16 or 32771 fp32 values is too short to hold the
    table and searches the sorted row itself. p from nearly 0 to nearly 1,
    with and without min-p, ties and distinct values."""
    need_gpu()
    total = ParityReport()
    seed = 1900 + V % 97
    for kind in ("normal", "ties"):
        seed += 1
        B = 6
        xb = random_rows(seed, B, V, dtype, kind=kind, scale=3.0)
        idx, sv = stable_ascending_sort(xb, dtype)
        p = f32_to_bits(np.array([0.02, 0.3, 0.5, 0.9, 0.99, 0.9999], np.float32), dtype)
        mp = f32_to_bits(np.array([0.0, 0.01, 0.2, 1e-4, 0.5, 1.0], np.float32), dtype)
        for mm in (None, mp):
            ref = oracle_sorted(sv, idx, dtype, p, None, logits_bits=xb, min_p_bits=mm)
            got = gpu_with_sorted(sv, idx, dtype, p, None, xb, min_p=mm)
            rep = compare(got, xb, ref, dtype)
            assert rep.hard_mismatches == 0, (kind, mm is None, rep.details[:2])
            total.merge(rep)
    say(f"with_sorted without k, segment table {dtype} V={V}: {total}")


@pytest.mark.parametrize("dtype,V", [("bf16", 65546), ("bf16", 262144), ("f32", 32771), ("f16", 131080)])
def test_with_sorted_disabled_k(dtype, V):
    """Pre-sorted rows with k given: rows whose k is 0, V or more, or negative
    have no top-k, and their top-p boundary is searched over the whole sorted
    row, while the other rows of the batch search the copy of the top values.
    Mixed batches, with and without min-p and with and without logits; all
    rows' k disabled too."""
    need_gpu()
    total = ParityReport()
    seed = 2600 + V % 89
    for kind in ("normal", "ties"):
        seed += 1
        B = 8
        xb = random_rows(seed, B, V, dtype, kind=kind, scale=3.0)
        idx, sv = stable_ascending_sort(xb, dtype)
        p = f32_to_bits(np.array([0.02, 0.3, 0.5, 0.9, 0.99, 0.9999, 0.7, 0.95], np.float32), dtype)
        mp = f32_to_bits(np.array([0.0, 0.01, 0.2, 1e-4, 0.5, 1.0, 0.05, 0.0], np.float32), dtype)
        mixed = np.array([0, 50, V, 3000, -1, 1, V + 7, 0], np.int32)
        none_on = np.array([0, V, -5, 0, V + 1, 0, 0, V], np.int32)
        for k in (mixed, none_on):
            for mm in (None, mp):
                for logits in (xb, None):
                    ref = oracle_sorted(sv, idx, dtype, p, k, logits_bits=xb, min_p_bits=mm)
                    got = gpu_with_sorted(sv, idx, dtype, p, k, logits, min_p=mm)
                    rep = compare(got, xb, ref, dtype)
                    assert rep.hard_mismatches == 0, (kind, k[:3], mm is None, logits is None, rep.details[:2])
                    total.merge(rep)
    say(f"with_sorted with disabled k {dtype} V={V}: {total}")


NEG_INF_BITS = {"f32": 0xFF800000, "f16": 0xFC00, "bf16": 0xFF80}


@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("f32", 70001), ("f16", 32000), ("bf16", 4099)])
def test_rows_mostly_neg_inf(dtype, V, policy):
    """Rows whose entries are largely -inf (a vocabulary masked by an earlier
    stage, e.g. a grammar constraint): half, 99 %, all but 1000, all but one,
    with the finite entries at random positions. -inf entries have zero
    probability; they are masked, and they count in the stable order like any
    other value below the survivors."""
    need_gpu()
    total = ParityReport()
    rng = np.random.default_rng(V)
    for i, keep in enumerate((V // 2, V // 100, 1000, 1)):
        B = 3
        xb = random_rows(7000 + V + i, B, V, dtype, kind=("normal", "gumbel", "ties", "spikes")[i])
        for b in range(B):
            masked = rng.permutation(V)[:V - keep]
            xb[b, masked] = NEG_INF_BITS[dtype]
        k, p = random_params(7000 + V + i, B, V, dtype, k_lo=1, k_hi=min(V, 3000))
        k_big = np.full(B, min(V - 1, keep + 5), np.int32)  # k beyond the finite entries
        for pp, kk in ((None, k), (p, None), (p, k), (p, k_big), (None, k_big)):
            got = gpu_apply(xb, dtype, pp, kk)
            rep = compare(got, xb, oracle_apply(xb, dtype, pp, kk), dtype)
            assert rep.hard_mismatches == 0, (dtype, V, keep, pp is None, kk is None, rep.details[:2])
            total.merge(rep)
    say(f"mostly -inf {dtype} V={V} {policy}: {total}")


@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("f32", 70001), ("f16", 4099)])
def test_mostly_neg_inf_other_entries(dtype, V, policy):
    """The same kind of rows (-inf except 1000 or one entry, or half) through
    the pre-sorted entry (with and without logits), min-p, QSample and the
    sorted survivors."""
    need_gpu()
    import torch
    import top_logits_filtering_amd as tk

    from oracle import sample_top_k_top_p as o_sample
    from oracle import sorted_survivors as o_surv
    from tests.gpu_util import k_dev, to_dev
    from tests.parity import compare_samples, compare_survivors
    from workloads.synth import random_min_p

    rng = np.random.default_rng(V + 1)
    for i, keep in enumerate((V // 2, 1000, 1)):
        B = 3
        seed = 7100 + V + i
        xb = random_rows(seed, B, V, dtype, kind=("gumbel", "normal", "ties")[i])
        for b in range(B):
            xb[b, rng.permutation(V)[:V - keep]] = NEG_INF_BITS[dtype]
        k, p = random_params(seed, B, V, dtype, k_lo=1, k_hi=min(V, 3000))
        mp = random_min_p(seed, B, dtype, specials=False)
        case = (dtype, V, keep, policy)
        idx, sv = stable_ascending_sort(xb, dtype)
        for logits in (xb, None):
            got = gpu_with_sorted(sv, idx, dtype, p, k, logits)
            rep = compare(got, xb, oracle_sorted(sv, idx, dtype, p, k, logits_bits=xb), dtype)
            assert rep.hard_mismatches == 0, (case, "sorted", logits is None, rep.details[:2])
        got = gpu_apply(xb, dtype, p, None, min_p=mp)
        rep = compare(got, xb, oracle_apply(xb, dtype, p, None, min_p_bits=mp), dtype)
        assert rep.hard_mismatches == 0, (case, "min_p", rep.details[:2])
        q = rng.exponential(1.0, size=(B, V)).astype(np.float32)
        sel = tk.sample_top_k_top_p(to_dev(xb, dtype), to_dev(p, dtype), k_dev(k), None, torch.from_numpy(q).cuda(),
                                    1e-6)
        torch.cuda.synchronize()
        h, _, det = compare_samples(sel.cpu().numpy(), o_sample(xb, dtype, p, k, None, q.astype(np.float64), 1e-6))
        assert h == 0, (case, "qsample", det[:2])
        pr, ix, cn = tk.top_k_top_p_sorted_survivors(to_dev(xb, dtype), to_dev(p, dtype), None, None, cap=64)
        torch.cuda.synchronize()
        h, det = compare_survivors(pr.cpu().numpy().astype(np.float64), ix.cpu().numpy(), cn.cpu().numpy(),
                                   o_surv(xb, dtype, p, None, None, 64))
        assert h == 0, (case, "survivors", det[:2])
    say(f"mostly -inf, other entries {dtype} V={V} {policy}: ok")
