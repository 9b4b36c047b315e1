"""Row-strided operands (views of wider buffers, e.g. a vocabulary padded to
a multiple of 64) through the _ex entry points: the result must equal the
dense call bit for bit, and the padding must stay untouched (needs an MI355X)."""

import numpy as np
import pytest

from tests.gpu_util import from_dev, k_dev, need_gpu, to_dev
from workloads.synth import f32_to_bits, random_min_p, random_params, random_rows, stable_ascending_sort

pytestmark = pytest.mark.gpu

SENTINEL = {"f32": 0x7FC00001, "f16": 0x7E01, "bf16": 0x7FC1}  # NaN patterns the filter never writes


def _padded(bits, dtype, ld, fill):
    """A [B, ld] device buffer holding bits in its first V columns, and the [B, V] view."""
    B, V = bits.shape
    full = np.full((B, ld), fill, dtype=bits.dtype)
    full[:, :V] = bits
    t = to_dev(full, dtype)
    return t, t[:, :V]


@pytest.mark.parametrize("dtype,V,pad", [("bf16", 151936, 64), ("bf16", 4099, 13), ("f32", 70001, 7),
                                         ("f16", 32000, 8), ("f32", 1, 3)])
def test_apply_strided_matches_dense(dtype, V, pad):
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    B = 6
    xb = random_rows(2100 + V, B, V, dtype, kind="gumbel")
    k, p = random_params(2100 + V, B, V, dtype, k_lo=1, k_hi=min(V, 2000))
    mp = random_min_p(2100 + V, B, dtype)
    for min_p in (None, mp):
        dense = tk.apply_top_k_top_p(to_dev(xb, dtype), to_dev(p, dtype), k_dev(k), min_p=to_dev(min_p, dtype))
        torch.cuda.synchronize()
        _, xv = _padded(xb, dtype, V + pad, SENTINEL[dtype])
        obuf, ov = _padded(np.zeros_like(xb), dtype, V + pad + 5, SENTINEL[dtype])
        tk.apply_top_k_top_p(xv, to_dev(p, dtype), k_dev(k), out=ov, min_p=to_dev(min_p, dtype))
        torch.cuda.synchronize()
        got = from_dev(obuf, dtype)
        assert np.array_equal(got[:, :V], from_dev(dense, dtype)), (dtype, V, pad, min_p is None)
        assert (got[:, V:] == SENTINEL[dtype]).all(), "padding was written"


@pytest.mark.parametrize("use_logits", [True, False])
def test_with_sorted_strided_matches_dense(use_logits):
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    dtype, B, V = "bf16", 5, 70001
    xb = random_rows(2200, B, V, dtype, kind="normal", scale=3.0)
    idx, sv = stable_ascending_sort(xb, dtype)
    k, p = random_params(2200, B, V, dtype, k_lo=1, k_hi=4096)
    dense = tk.apply_top_k_top_p_with_sorted(to_dev(sv, dtype), k_dev(idx), to_dev(p, dtype), k_dev(k),
                                             to_dev(xb, dtype) if use_logits else None)
    torch.cuda.synchronize()
    _, svv = _padded(sv, dtype, V + 9, SENTINEL[dtype])
    ibuf = torch.from_numpy(np.full((B, V + 3), -7, np.int32)).cuda()
    ibuf[:, :V] = k_dev(idx)
    _, xv = _padded(xb, dtype, V + 64, SENTINEL[dtype])
    obuf, ov = _padded(np.zeros_like(xb), dtype, V + 1, SENTINEL[dtype])
    tk.apply_top_k_top_p_with_sorted(svv, ibuf[:, :V], to_dev(p, dtype), k_dev(k), xv if use_logits else None,
                                     out=ov)
    torch.cuda.synchronize()
    got = from_dev(obuf, dtype)
    assert np.array_equal(got[:, :V], from_dev(dense, dtype))
    assert (got[:, V:] == SENTINEL[dtype]).all()
