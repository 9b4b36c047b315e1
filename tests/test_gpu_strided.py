"""Row-strided operands (views of wider buffers, e.g. a vocabulary padded to
a multiple of 64) through the _ex entry points, checked against the CPU
oracle on the un-padded rows; the result must also equal the dense call bit
for bit, and the padding must stay untouched (needs an MI355X). Row strides
that are not a multiple of 16 bytes take the streamed kernels."""

import numpy as np
import pytest

from oracle import apply_top_k_top_p as oracle_apply
from oracle import apply_top_k_top_p_with_sorted as oracle_sorted
from tests.gpu_util import SENTINEL, from_dev, k_dev, need_gpu, padded_dev, say, to_dev
from tests.parity import compare
from workloads.synth import random_min_p, random_params, random_rows, stable_ascending_sort

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,V,pad", [("bf16", 151936, 64), ("bf16", 151936, 1), ("bf16", 4099, 13),
                                         ("f32", 70001, 7), ("f32", 65536, 4), ("f16", 32000, 8),
                                         ("f16", 32000, 3), ("f32", 1, 3)])
def test_apply_strided(dtype, V, pad):
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    B = 6
    xb = random_rows(2100 + V + pad, B, V, dtype, kind="gumbel")
    k, p = random_params(2100 + V, B, V, dtype, k_lo=1, k_hi=min(V, 2000))
    mp = random_min_p(2100 + V, B, dtype)
    for min_p in (None, mp):
        dense = tk.apply_top_k_top_p(to_dev(xb, dtype), to_dev(p, dtype), k_dev(k), min_p=to_dev(min_p, dtype))
        torch.cuda.synchronize()
        _, xv = padded_dev(xb, dtype, V + pad, SENTINEL[dtype])
        obuf, ov = padded_dev(np.zeros_like(xb), dtype, V + pad + 5, SENTINEL[dtype])
        tk.apply_top_k_top_p(xv, to_dev(p, dtype), k_dev(k), out=ov, min_p=to_dev(min_p, dtype))
        torch.cuda.synchronize()
        got = from_dev(obuf, dtype)
        rep = compare(np.ascontiguousarray(got[:, :V]), xb, oracle_apply(xb, dtype, p, k, min_p_bits=min_p), dtype)
        assert rep.hard_mismatches == 0, (dtype, V, pad, min_p is None, rep.details[:2])
        assert np.array_equal(got[:, :V], from_dev(dense, dtype)), (dtype, V, pad, min_p is None)
        assert (got[:, V:] == SENTINEL[dtype]).all(), "padding was written"
        say(f"strided {dtype} V={V} pad={pad} min_p={min_p is not None}: {rep}")


@pytest.mark.parametrize("use_logits", [True, False])
@pytest.mark.parametrize("dtype,V", [("bf16", 70001), ("f32", 4099)])
def test_with_sorted_strided(use_logits, dtype, V):
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    B = 5
    xb = random_rows(2200 + V, B, V, dtype, kind="normal", scale=3.0)
    idx, sv = stable_ascending_sort(xb, dtype)
    k, p = random_params(2200, B, V, dtype, k_lo=1, k_hi=4096)
    mp = random_min_p(2200 + V, B, dtype)
    for min_p in (None, mp):
        dense = tk.apply_top_k_top_p_with_sorted(to_dev(sv, dtype), k_dev(idx), to_dev(p, dtype), k_dev(k),
                                                 to_dev(xb, dtype) if use_logits else None,
                                                 min_p=to_dev(min_p, dtype))
        torch.cuda.synchronize()
        _, svv = padded_dev(sv, dtype, V + 9, SENTINEL[dtype])
        ibuf = torch.from_numpy(np.full((B, V + 3), -7, np.int32)).cuda()
        ibuf[:, :V] = k_dev(idx)
        _, xv = padded_dev(xb, dtype, V + 64, SENTINEL[dtype])
        obuf, ov = padded_dev(np.zeros_like(xb), dtype, V + 1, SENTINEL[dtype])
        tk.apply_top_k_top_p_with_sorted(svv, ibuf[:, :V], to_dev(p, dtype), k_dev(k), xv if use_logits else None,
                                         out=ov, min_p=to_dev(min_p, dtype))
        torch.cuda.synchronize()
        got = from_dev(obuf, dtype)
        ref = oracle_sorted(sv, idx, dtype, p, k, logits_bits=xb, min_p_bits=min_p)
        rep = compare(np.ascontiguousarray(got[:, :V]), xb, ref, dtype)
        assert rep.hard_mismatches == 0, (dtype, V, use_logits, min_p is None, rep.details[:2])
        assert np.array_equal(got[:, :V], from_dev(dense, dtype))
        assert (got[:, V:] == SENTINEL[dtype]).all()
