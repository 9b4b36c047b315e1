"""The sorted-survivors output (TKS intermediate output) on the HIP path vs
the CPU oracle, through the C ABI (needs an MI355X)."""

import numpy as np
import pytest

from oracle import sorted_survivors as oracle_survivors
from tests.golden_io import load_hand_cases
from tests.gpu_util import k_dev, need_gpu, say, to_dev
from tests.parity import compare_survivors
from workloads.synth import f32_to_bits, random_min_p, random_params, random_rows

pytestmark = pytest.mark.gpu

POLICIES = {"auto": 0, "multipass": 1, "stream": 2}


@pytest.fixture(params=sorted(POLICIES), scope="module")
def policy(request):
    need_gpu()
    import top_logits_filtering_amd as tk

    prev = tk.set_plan_policy(POLICIES[request.param])
    yield request.param
    tk.set_plan_policy(prev)


def gpu_survivors(xb, dtype, p=None, k=None, min_p=None, cap=64, with_probs=True):
    import torch
    import top_logits_filtering_amd as tk

    pr, idx, cnt = tk.top_k_top_p_sorted_survivors(to_dev(xb, dtype), to_dev(p, dtype), k_dev(k), to_dev(min_p, dtype),
                                                   cap=cap, with_probs=with_probs)
    torch.cuda.synchronize()
    return (None if pr is None else pr.cpu().numpy().astype(np.float64)), idx.cpu().numpy(), cnt.cpu().numpy()


def test_survivor_hand_cases(policy):
    for case in load_hand_cases("survivor_cases.txt"):
        pr, idx, cnt = gpu_survivors(case.x, case.dtype, case.p, case.k, case.min_p, case.cap)
        assert np.array_equal(idx, case.expect_idx), (policy, case.name, idx)
        assert np.allclose(pr, case.expect_probs, atol=6e-5), (policy, case.name, pr)
        assert np.array_equal(cnt, case.expect_count), (policy, case.name, cnt)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_survivors_random_rows(dtype, policy):
    seed = {"f32": 1, "f16": 2, "bf16": 3}[dtype] * 5000
    for V in (1, 2, 7, 1000, 4099, 20011, 170001):
        for kind in ("normal", "ties", "gumbel"):
            seed += 1
            B = 5 if V < 20000 else 3
            xb = random_rows(seed, B, V, dtype, kind=kind)
            k, p = random_params(seed, B, V, dtype, k_lo=1, k_hi=min(V, 1500))
            mp = random_min_p(seed, B, dtype, specials=False)
            for pp, kk, mm in ((None, k, None), (p, None, None), (p, k, mp), (None, None, mp)):
                for cap in (1, 100, 2048):
                    pr, idx, cnt = gpu_survivors(xb, dtype, pp, kk, mm, cap)
                    ref = oracle_survivors(xb, dtype, pp, kk, mm, cap)
                    h, det = compare_survivors(pr, idx, cnt, ref)
                    assert h == 0, (V, kind, pp is None, kk is None, mm is None, cap, det[:3])
    say(f"survivors {dtype}/{policy}: ok")




def test_survivors_large_sets(policy):
    """Rows that keep tens of thousands of survivors (nearly flat and constant
    rows, p near 1, no top-k): every listed index, probability and count
    against the oracle, with a capacity below and above the count."""
    cases = [("bf16", 40000, "normal", [0.99, 0.5]), ("f32", 40000, "const", [0.99, 0.3]),
             ("bf16", 151936, "normal", [0.99])]
    for dtype, V, kind, ps in cases:
        B = len(ps)
        xb = random_rows(91 + V, B, V, dtype, kind=kind, scale=0.05)
        p = f32_to_bits(np.array(ps, np.float32), dtype)
        for cap in (5000, V):
            pr, idx, cnt = gpu_survivors(xb, dtype, p, None, None, cap)
            ref = oracle_survivors(xb, dtype, p, None, None, cap)
            h, det = compare_survivors(pr, idx, cnt, ref)
            assert h == 0, (dtype, V, kind, cap, det[:3])
        say(f"survivors large sets {dtype} V={V} {kind} ({policy}): counts {ref.counts.tolist()}")
