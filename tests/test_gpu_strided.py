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


def _filled(shape, dtype):
    """A device buffer of the given shape holding the sentinel everywhere."""
    nt = np.uint32 if dtype == "f32" else np.uint16
    return to_dev(np.full(shape, SENTINEL[dtype], dtype=nt), dtype)


def _bits(t, dtype):
    return from_dev(t.contiguous(), dtype)


# (name, dtype, B, V): element-strided layouts of logits and out
ELEMENT_CASES = [("transposed", "bf16", 8, 70001), ("transposed", "f32", 5, 4099),
                 ("column_step", "f16", 6, 32000), ("column_step", "bf16", 3, 262144),
                 ("params_strided", "bf16", 7, 151936), ("rows_overlap", "f32", 6, 65536),
                 ("column_step", "f16", 1, 5000), ("transposed", "bf16", 9, 2),
                 ("transposed", "f32", 2, 1 << 20), ("column_step", "bf16", 2, (1 << 20) - 1)]


@pytest.mark.parametrize("policy", [0, 1])
@pytest.mark.parametrize("name,dtype,B,V", ELEMENT_CASES)
def test_apply_element_strided(name, dtype, B, V, policy):
    """Views with a non-unit element stride (a transposed [V, B] buffer, every
    second or third column of a wider one, parameters with strides 0, 2 and 3,
    input rows that share elements) through apply_top_k_top_p_strided: the
    oracle on the dense values decides, the row-contiguous call must give the
    same bits, and out's elements outside the view stay untouched."""
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    seed = 2300 + V + B
    xb = random_rows(seed, B, V, dtype, kind="gumbel")
    k, p = random_params(seed, B, V, dtype, k_lo=1, k_hi=min(V, 3000))
    mp = random_min_p(seed, B, dtype)
    if name == "rows_overlap":  # row b starts at element b * V / 2 of one buffer
        half = V // 2
        flat = random_rows(seed, 1, half * (B + 1), dtype, kind="gumbel")[0]
        xb = np.stack([flat[b * half:b * half + V] for b in range(B)])
    try:
        tk.set_plan_policy(policy)
        for min_p in (None, mp):
            dense = tk.apply_top_k_top_p(to_dev(xb, dtype), to_dev(p, dtype), k_dev(k), min_p=to_dev(min_p, dtype))
            pd, kd, md = to_dev(p, dtype), k_dev(k), to_dev(min_p, dtype)
            if name == "transposed":
                x = to_dev(np.ascontiguousarray(xb.T), dtype).t()
                obuf = _filled((V, B), dtype)
                out = obuf.t()
            elif name == "column_step":
                wide = np.zeros((B, 2 * V + 1), dtype=xb.dtype)
                wide[:, 1::2] = xb
                x = to_dev(wide, dtype)[:, 1::2]
                obuf = _filled((B, 3 * V), dtype)
                out = obuf[:, ::3]
            elif name == "params_strided":
                x = to_dev(xb, dtype)
                obuf = _filled((B, V), dtype)
                out = obuf
                pb = np.zeros(2 * B, dtype=p.dtype)
                pb[::2] = p
                kb = np.zeros(3 * B, dtype=np.int32)
                kb[::3] = k
                pd, kd = to_dev(pb, dtype)[::2], k_dev(kb)[::3]
                if min_p is not None:  # one value shared by every row (stride 0)
                    md = to_dev(min_p[:1], dtype).expand(B)
                    min_p = np.repeat(min_p[:1], B)
                    dense = tk.apply_top_k_top_p(to_dev(xb, dtype), to_dev(p, dtype), k_dev(k),
                                                 min_p=to_dev(min_p, dtype))
            else:  # rows_overlap
                x = to_dev(flat, dtype).as_strided((B, V), (V // 2, 1))
                obuf = _filled((B, V), dtype)
                out = obuf
            torch.cuda.synchronize()
            tk.apply_top_k_top_p(x, pd, kd, out=out, min_p=md)
            torch.cuda.synchronize()
            got = _bits(out, dtype)
            rep = compare(got, xb, oracle_apply(xb, dtype, p, k, min_p_bits=min_p), dtype)
            case = (name, dtype, B, V, policy, min_p is not None)
            assert rep.hard_mismatches == 0, (case, rep.details[:2])
            assert np.array_equal(got, from_dev(dense, dtype)), case
            whole = from_dev(obuf.contiguous(), dtype)
            assert int((whole != SENTINEL[dtype]).sum()) == B * V - int((got == SENTINEL[dtype]).sum()), case
            say(f"element-strided {case}: {rep}")
    finally:
        tk.set_plan_policy(0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_element_strided_single_column(dtype):
    """Rows of one element are copied through whatever the strides: one row,
    a logits row stride of 0 (one value expanded over the rows), and out as a
    column of a wider buffer."""
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    nt = np.uint32 if dtype == "f32" else np.uint16
    vals = random_rows(77, 1, 5, dtype, kind="normal")[0]
    p = to_dev(random_params(77, 5, 1, dtype)[1], dtype)
    # one row, transposed views of a [1, 1] buffer
    x1 = to_dev(vals[:1].reshape(1, 1), dtype).t()
    o1 = _filled((1, 1), dtype).t()
    tk.apply_top_k_top_p(x1, p[:1], None, out=o1)
    torch.cuda.synchronize()
    assert from_dev(o1.contiguous(), dtype)[0, 0] == vals[0]
    # one value expanded over 5 rows (row stride 0), out every third element of a [5, 3] buffer
    x = to_dev(vals[:1], dtype).reshape(1, 1).expand(5, 1)
    obuf = _filled((5, 3), dtype)
    tk.apply_top_k_top_p(x, p, None, out=obuf[:, 1:2])
    torch.cuda.synchronize()
    got = from_dev(obuf, dtype)
    assert (got[:, 1] == vals[0]).all()
    assert (got[:, [0, 2]] == nt(SENTINEL[dtype])).all()
    # rows of one element with a row stride of 2
    wide = to_dev(np.stack([vals, vals]).T.copy(), dtype)  # [5, 2]
    obuf = _filled((5, 2), dtype)
    tk.apply_top_k_top_p(wide[:, :1], p, None, out=obuf[:, 1:])
    torch.cuda.synchronize()
    got = from_dev(obuf, dtype)
    assert np.array_equal(got[:, 1], vals)
    assert (got[:, 0] == nt(SENTINEL[dtype])).all()
