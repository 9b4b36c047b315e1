"""Top-p-only rows whose survivors overflow the candidate list (wide rows
with p between 0.8 and 0.99: thousands of survivors), on the HIP path vs the
CPU oracle, through the C ABI (needs an MI355X). Such rows leave the
candidate plan for the multi-pass plan; the filter, min-p on top, QSample,
the argmax and the sorted survivors are all compared."""

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

PS = [0.8, 0.9, 0.95, 0.99]

# register-resident shapes of each dtype, ragged tails included
SHAPES = [("bf16", 151936, "normal"), ("f16", 32000, "normal"), ("f32", 50021, "normal"), ("bf16", 70001, "ties"),
          ("f16", 20011, "wide"), ("bf16", 4099, "normal")]


@pytest.mark.parametrize("dtype,V,kind", SHAPES)
def test_wide_rows_top_p_only(dtype, V, kind):
    need_gpu()
    B = len(PS)
    xb = random_rows(5100 + V % 97, B, V, dtype, kind=kind, scale=3.0)
    p = f32_to_bits(np.array(PS, np.float32), dtype)
    mp = f32_to_bits(np.array([1e-4, 1e-3, 1e-5, 0.05], np.float32), dtype)
    total = ParityReport()
    for mm in (None, mp):
        got = gpu_apply(xb, dtype, p, None, mm)
        ref = oracle_apply(xb, dtype, p, None, min_p_bits=mm)
        rep = compare(got, xb, ref, dtype)
        assert rep.hard_mismatches == 0, (mm is None, rep.details[:3])
        total.merge(rep)
    n = [int((~(tr.top_k_mask | tr.top_p_mask)).sum()) for tr in ref.traces]
    say(f"top-p-only wide rows {dtype} V={V} {kind}: survivors {n}; {total}")


@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("f16", 32000)])
def test_wide_rows_sampling_and_survivors(dtype, V):
    need_gpu()
    B = len(PS)
    xb = random_rows(5200 + V % 97, B, V, dtype, kind="normal", scale=3.0)
    p = f32_to_bits(np.array(PS, np.float32), dtype)
    q = np.random.default_rng(5201).exponential(1.0, size=(B, V)).astype(np.float32)
    got, out = gpu_sample(xb, dtype, p, None, None, q, 1e-6, with_out=True)
    ref = oracle_sample(xb, dtype, p, None, None, q.astype(np.float64), 1e-6)
    h, s_, det = compare_samples(got, ref)
    assert h == 0, det[:3]
    rep = compare(out, xb, ref.filtered, dtype)
    assert rep.hard_mismatches == 0, rep.details[:3]
    none, _ = gpu_sample(xb, dtype, p, None, None, None)
    assert np.array_equal(none, oracle_sample(xb, dtype, p, None, None, None).selected)
    for cap in (1024, V):
        pr, idx, cnt = gpu_survivors(xb, dtype, p, None, None, cap)
        h, det = compare_survivors(pr, idx, cnt, oracle_survivors(xb, dtype, p, None, None, cap))
        assert h == 0, (cap, det[:3])
    say(f"top-p-only wide rows, sampling and survivors {dtype} V={V}: near-tie picks {s_}")
