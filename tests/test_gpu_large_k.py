"""Rows with large k (above the 1536 where a thread keeps four vector maxima
for the bound, up to the 3072 the bound serves, and just past it), on the
HIP path vs the CPU oracle, through the C ABI (needs an MI355X). Such rows
list more candidate vectors than the vector list holds, so their candidate
elements are listed straight from the register tile; rows past 3072 take
the multi-pass plan. The filter, top-p and min-p on top, QSample, the argmax
and the sorted survivors are compared."""

import numpy as np
import pytest

from oracle import apply_top_k_top_p as oracle_apply
from oracle import sample_top_k_top_p as oracle_sample
from oracle import sorted_survivors as oracle_survivors
from tests.gpu_util import gpu_apply, need_gpu, say
from tests.parity import ParityReport, compare, compare_samples, compare_survivors
from tests.test_gpu_sample import gpu_sample
from tests.test_gpu_survivors import gpu_survivors
from workloads.synth import f32_to_bits, random_rows

pytestmark = pytest.mark.gpu

KS = [1536, 1537, 2048, 2500, 3072, 3073]


@pytest.mark.parametrize("dtype,V,kind", [("bf16", 151936, "gumbel"), ("bf16", 151936, "normal"),
                                          ("f16", 70001, "ties"), ("f32", 50021, "normal"), ("bf16", 8193, "normal")])
def test_large_k(dtype, V, kind):
    need_gpu()
    B = len(KS)
    xb = random_rows(5300 + V % 89, B, V, dtype, kind=kind, scale=4.0 if kind == "gumbel" else 3.0)
    k = np.array(KS, np.int32)
    p = f32_to_bits(np.array([0.99, 0.95, 0.9, 0.999, 0.5, 0.97], np.float32), dtype)
    mp = f32_to_bits(np.array([1e-4, 1e-3, 1e-6, 0.01, 1e-5, 1e-4], np.float32), dtype)
    total = ParityReport()
    for pp, mm in ((None, None), (p, None), (p, mp)):
        got = gpu_apply(xb, dtype, pp, k, mm)
        ref = oracle_apply(xb, dtype, pp, k, min_p_bits=mm)
        rep = compare(got, xb, ref, dtype)
        assert rep.hard_mismatches == 0, (pp is None, mm is None, rep.details[:3])
        total.merge(rep)
    say(f"large k {dtype} V={V} {kind}: {total}")


@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("f16", 32000)])
def test_large_k_sampling_and_survivors(dtype, V):
    need_gpu()
    B = len(KS)
    xb = random_rows(5400 + V % 89, B, V, dtype, kind="gumbel", scale=4.0)
    k = np.array(KS, np.int32)
    p = f32_to_bits(np.array([1.0, 0.99, 0.95, 1.0, 0.999, 0.9], np.float32), dtype)
    q = np.random.default_rng(5401).exponential(1.0, size=(B, V)).astype(np.float32)
    got, out = gpu_sample(xb, dtype, p, k, None, q, 1e-6, with_out=True)
    ref = oracle_sample(xb, dtype, p, k, None, q.astype(np.float64), 1e-6)
    h, s_, det = compare_samples(got, ref)
    assert h == 0, det[:3]
    rep = compare(out, xb, ref.filtered, dtype)
    assert rep.hard_mismatches == 0, rep.details[:3]
    none, _ = gpu_sample(xb, dtype, p, k, None, None)
    assert np.array_equal(none, oracle_sample(xb, dtype, p, k, None, None).selected)
    for cap in (1024, 4096):
        pr, idx, cnt = gpu_survivors(xb, dtype, p, k, None, cap)
        h, det = compare_survivors(pr, idx, cnt, oracle_survivors(xb, dtype, p, k, None, cap))
        assert h == 0, (cap, det[:3])
    say(f"large k sampling and survivors {dtype} V={V}: near-tie picks {s_}")
