"""The longest rows the library accepts (V = 2^20, and 2^20 - 1 for a ragged
tail) on every entry point, against the CPU oracle (needs an MI355X). Rows
this long are streamed from global memory: they exceed a block's register
tile, and the pre-sorted kernels split them into 16 slices."""

import numpy as np
import pytest

from oracle import apply_top_k_top_p as oracle_apply
from oracle import apply_top_k_top_p_with_sorted as oracle_sorted
from oracle import sample_top_k_top_p as oracle_sample
from oracle import sorted_survivors as oracle_survivors
from tests.gpu_util import gpu_apply, gpu_with_sorted, k_dev, need_gpu, say, to_dev
from tests.parity import ParityReport, compare, compare_samples, compare_survivors
from workloads.synth import f32_to_bits, random_rows, stable_ascending_sort

pytestmark = pytest.mark.gpu

V_MAX = 1 << 20


def _params(dtype, B):
    k = np.array([1, 3000, 0], np.int32)[:B]
    p = f32_to_bits(np.array([0.9, 0.5, 0.99], np.float32)[:B], dtype)
    mp = f32_to_bits(np.array([0.05, 0.2, 0.01], np.float32)[:B], dtype)
    return k, p, mp


@pytest.mark.parametrize("dtype,V", [("bf16", V_MAX), ("f32", V_MAX), ("f16", V_MAX - 1)])
def test_apply_max_rows(dtype, V):
    need_gpu()
    B = 3
    total = ParityReport()
    for kind in ("normal", "ties"):
        xb = random_rows(2100 + V % 5, B, V, dtype, kind=kind, scale=3.0)
        k, p, mp = _params(dtype, B)
        for pp, kk, mm in ((p, k, None), (None, k, None), (p, None, None), (p, k, mp)):
            got = gpu_apply(xb, dtype, pp, kk, mm)
            ref = oracle_apply(xb, dtype, pp, kk, min_p_bits=mm)
            rep = compare(got, xb, ref, dtype)
            assert rep.hard_mismatches == 0, (kind, pp is None, kk is None, mm is None, rep.details[:2])
            total.merge(rep)
    say(f"apply {dtype} V={V}: {total}")


@pytest.mark.parametrize("dtype,V", [("bf16", V_MAX), ("f32", V_MAX - 1)])
def test_with_sorted_max_rows(dtype, V):
    need_gpu()
    B = 3
    total = ParityReport()
    xb = random_rows(2200 + V % 5, B, V, dtype, kind="ties", scale=3.0)
    idx, sv = stable_ascending_sort(xb, dtype)
    k, p, mp = _params(dtype, B)
    for pp, kk, mm in ((p, k, None), (None, k, None), (p, None, None), (p, k, mp)):
        ref = oracle_sorted(sv, idx, dtype, pp, kk, logits_bits=xb, min_p_bits=mm)
        for use_logits in (True, False):
            got = gpu_with_sorted(sv, idx, dtype, pp, kk, xb if use_logits else None, min_p=mm)
            rep = compare(got, xb, ref, dtype)
            assert rep.hard_mismatches == 0, (pp is None, kk is None, mm is None, use_logits, rep.details[:2])
            total.merge(rep)
    say(f"with_sorted {dtype} V={V}: {total}")


def test_sample_and_survivors_max_rows():
    need_gpu()
    import torch
    import top_logits_filtering_amd as tk

    dtype, V, B = "bf16", V_MAX, 3
    xb = random_rows(2300, B, V, dtype, kind="gumbel", scale=4.0)
    k, p, _ = _params(dtype, B)
    q = np.random.default_rng(2301).exponential(1.0, size=(B, V)).astype(np.float32)
    qd = torch.from_numpy(q).cuda()
    for qq, qh in ((None, None), (qd, q)):
        sel = tk.sample_top_k_top_p(to_dev(xb, dtype), to_dev(p, dtype), k_dev(k), None, qq, 1e-6)
        torch.cuda.synchronize()
        ref = oracle_sample(xb, dtype, p, k, None, None if qh is None else qh.astype(np.float64), 1e-6)
        h, _, det = compare_samples(sel.cpu().numpy(), ref)
        assert h == 0, (qq is None, det[:3])
    pr, ix, cnt = tk.top_k_top_p_sorted_survivors(to_dev(xb, dtype), to_dev(p, dtype), k_dev(k), None, cap=512)
    torch.cuda.synchronize()
    ref = oracle_survivors(xb, dtype, p, k, None, 512)
    h, det = compare_survivors(pr.cpu().numpy().astype(np.float64), ix.cpu().numpy(), cnt.cpu().numpy(), ref)
    assert h == 0, det[:3]
    say("sample and survivors bf16 V=2^20: ok")


def test_many_short_rows():
    """More rows than one grid dimension of 65535 blocks would hold: one block
    per row (or per slice) over 70000 rows of 96 values, sampled rows against
    the oracle and properties on every row."""
    need_gpu()
    dtype, B, V = "bf16", 70000, 96
    xb = random_rows(2400, B, V, dtype, kind="ties", scale=2.0)
    rng = np.random.default_rng(2401)
    k = rng.integers(0, V + 2, size=B).astype(np.int32)
    p = f32_to_bits(rng.uniform(0.1, 1.0, size=B).astype(np.float32), dtype)
    got = gpu_apply(xb, dtype, p, k)
    rows = np.unique(np.concatenate([[0, 1, 65534, 65535, 65536, B - 1], rng.choice(B, 40, replace=False)]))
    ref = oracle_apply(xb[rows], dtype, p[rows], k[rows])
    rep = compare(got[rows], xb[rows], ref, dtype)
    assert rep.hard_mismatches == 0, rep.details[:2]
    neg = 0xFF80
    assert np.all((got == xb) | (got == neg)), "values other than input bits or -inf"
    assert (got != neg).any(axis=1).all(), "a row lost every position"
    idx, sv = stable_ascending_sort(xb[:20000], dtype)
    got_s = gpu_with_sorted(sv, idx, dtype, p[:20000], k[:20000], xb[:20000])
    assert np.array_equal(got_s, got[:20000]), "pre-sorted entry differs from the sorting entry"
    say(f"{B} rows of {V}: {rep}")


def test_rows_beyond_one_launch():
    """2^21 + 3 rows of two values: one launch takes at most 2^21 rows, so
    the batch is launched in two chunks. Every row is checked against the
    result the filter must give for k = 1 (the maximum and its ties), on the
    sorting entry, the pre-sorted entry, both sampling modes and the sorted
    survivors; rows around the chunk boundary also against the oracle."""
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    dtype, B, V = "f32", (1 << 21) + 3, 2
    rng = np.random.default_rng(2500)
    vals = np.round(rng.normal(0.0, 2.0, size=(B, V)), 1).astype(np.float32)  # some rows tie
    xb = vals.view(np.uint32)
    k = np.ones(B, np.int32)
    p = f32_to_bits(np.full(B, 0.5, np.float32), dtype)
    mx = vals.max(axis=1, keepdims=True)
    keep = vals == mx
    expect = np.where(keep, xb, np.uint32(0xFF800000))
    top = np.where(keep[:, 1], 1, 0)  # the maximum with the highest index
    got = gpu_apply(xb, dtype, None, k)
    assert np.array_equal(got, expect)
    rows = np.array([0, (1 << 21) - 2, (1 << 21) - 1, 1 << 21, (1 << 21) + 1, B - 1])
    rep = compare(got[rows], xb[rows], oracle_apply(xb[rows], dtype, p[rows], k[rows]), dtype)
    assert rep.hard_mismatches == 0, rep.details
    got_pk = gpu_apply(xb, dtype, p, k)
    rep = compare(got_pk[rows], xb[rows], oracle_apply(xb[rows], dtype, p[rows], k[rows]), dtype)
    assert rep.hard_mismatches == 0, rep.details
    idx, sv = stable_ascending_sort(xb, dtype)
    for logits in (xb, None):
        got_s = gpu_with_sorted(sv, idx, dtype, None, k, logits)
        assert np.array_equal(got_s, expect)
    x = to_dev(xb, dtype)
    q = torch.ones((B, V), dtype=torch.float32, device="cuda")
    for qq in (None, q):
        sel = tk.sample_top_k_top_p(x, None, k_dev(k), None, qq, 0.0)
        torch.cuda.synchronize()
        assert np.array_equal(sel.cpu().numpy(), top)
    pr, ix, cnt = tk.top_k_top_p_sorted_survivors(x, None, k_dev(k), None, cap=2)
    torch.cuda.synchronize()
    n = keep.sum(axis=1)
    assert np.array_equal(cnt.cpu().numpy(), n)
    ix = ix.cpu().numpy()
    assert np.array_equal(ix[:, 0], top)
    assert np.array_equal(ix[:, 1], np.where(n == 2, 0, -1))
    say(f"{B} rows of {V} in two launches: ok")
