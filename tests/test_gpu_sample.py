"""Sampling after the filter on the HIP path vs the CPU oracle, through the C
ABI (needs an MI355X). The oracle and its pins define the stage ("Subsequent
processing" of Ascend's aclnnTopKTopPSampleV2 page)."""

import numpy as np
import pytest

from oracle import sample_top_k_top_p as oracle_sample
from tests.golden_io import load_hand_cases
from tests.gpu_util import from_dev, k_dev, need_gpu, say, to_dev
from tests.parity import compare, compare_samples
from workloads.synth import f32_to_bits, make_workload, random_min_p, random_params, random_rows

pytestmark = pytest.mark.gpu

POLICIES = {"auto": 0, "multipass": 1, "stream": 2}


@pytest.fixture(params=sorted(POLICIES), scope="module")
def policy(request):
    need_gpu()
    import top_logits_filtering_amd as tk

    prev = tk.set_plan_policy(POLICIES[request.param])
    yield request.param
    tk.set_plan_policy(prev)


def gpu_sample(xb, dtype, p=None, k=None, min_p=None, q=None, eps=0.0, with_out=False):
    import torch
    import top_logits_filtering_amd as tk

    x = to_dev(xb, dtype)
    out = torch.empty_like(x) if with_out else None
    qd = None if q is None else torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32)).cuda()
    sel = tk.sample_top_k_top_p(x, to_dev(p, dtype), k_dev(k), to_dev(min_p, dtype), qd, eps, out=out)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), (None if out is None else from_dev(out, dtype))


def test_sample_hand_cases(policy):
    for case in load_hand_cases("sample_cases.txt"):
        got, _ = gpu_sample(case.x, case.dtype, case.p, case.k, case.min_p, case.q, case.eps)
        assert np.array_equal(got, case.expect_idx), (policy, case.name, got, case.expect_idx)


def _q(seed, B, V):
    rng = np.random.default_rng(seed)
    return rng.exponential(1.0, size=(B, V)).astype(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_sample_random_rows(dtype, policy):
    """Several tiles and ragged tails, every filter mode, None and QSample;
    the filtered output, when asked for, equals the filter's."""
    hard = soft = 0
    seed = {"f32": 1, "f16": 2, "bf16": 3}[dtype] * 3000
    for V in (2, 7, 1000, 4099, 20011, 170001):
        for kind in ("normal", "ties", "gumbel", "spikes"):
            seed += 1
            B = 6 if V < 20000 else 3
            xb = random_rows(seed, B, V, dtype, kind=kind)
            k, p = random_params(seed, B, V, dtype, k_lo=1, k_hi=min(V, 1500))
            mp = random_min_p(seed, B, dtype, specials=False)
            q = _q(seed, B, V)
            for pp, kk, mm in ((None, k, None), (p, None, None), (p, k, None), (p, k, mp), (None, None, mp)):
                for qq in (None, q):
                    got, out = gpu_sample(xb, dtype, pp, kk, mm, qq, 1e-6, with_out=(qq is not None))
                    ref = oracle_sample(xb, dtype, pp, kk, mm, None if qq is None else qq.astype(np.float64), 1e-6)
                    h, s_, det = compare_samples(got, ref)
                    assert h == 0, (V, kind, pp is None, kk is None, mm is None, qq is None, det[:3])
                    hard += h
                    soft += s_
                    if out is not None:
                        rep = compare(out, xb, ref.filtered, dtype)
                        assert rep.hard_mismatches == 0, rep.details[:2]
    say(f"sample {dtype}/{policy}: near-tie picks {soft}")


def test_sample_without_out_matches_with_out():
    need_gpu()
    wl = make_workload(3, rows=range(30))
    q = _q(7, wl.B, wl.V)
    a, _ = gpu_sample(wl.logits, wl.dtype, wl.p, wl.k, None, q, 1e-6, with_out=False)
    b, out = gpu_sample(wl.logits, wl.dtype, wl.p, wl.k, None, q, 1e-6, with_out=True)
    assert np.array_equal(a, b)
    import top_logits_filtering_amd as tk
    import torch

    plain = from_dev(tk.apply_top_k_top_p(to_dev(wl.logits, wl.dtype), to_dev(wl.p, wl.dtype), k_dev(wl.k)), wl.dtype)
    torch.cuda.synchronize()
    assert np.array_equal(out, plain)


def test_sample_large_survivor_sets(policy):
    """QSample and the argmax on rows that keep tens of thousands of
    survivors (nearly flat rows, and constant rows where only the index
    order ranks them), every pick against the oracle."""
    cases = [("bf16", 40000, "normal", [0.99, 0.5, 0.02, 0.001]), ("f32", 40000, "const", [0.99, 0.7, 0.3]),
             ("bf16", 151936, "normal", [0.99, 0.9]), ("f16", 70001, "const", [0.999])]
    for dtype, V, kind, ps in cases:
        B = len(ps)
        xb = random_rows(77 + V, B, V, dtype, kind=kind, scale=0.05)  # nearly flat rows
        p = f32_to_bits(np.array(ps, np.float32), dtype)
        q = _q(78 + V, B, V)
        got, _ = gpu_sample(xb, dtype, p, None, None, q, 1e-6)
        ref = oracle_sample(xb, dtype, p, None, None, q.astype(np.float64), 1e-6)
        n = [int((~(tr.top_k_mask | tr.top_p_mask)).sum()) for tr in ref.filtered.traces]
        h, s_, det = compare_samples(got, ref)
        assert h == 0, (dtype, V, kind, n, det)
        say(f"large survivor sets {dtype} V={V} {kind} ({policy}): survivors {n}, near-tie picks {s_}")
        none, _ = gpu_sample(xb, dtype, p, None, None, None)
        assert np.array_equal(none, oracle_sample(xb, dtype, p, None, None, None).selected)


