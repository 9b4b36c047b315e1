"""A seeded sweep over random shapes, dtypes, value kinds, parameter mixes,
plan policies and every entry point, each case against the CPU oracle (needs
an MI355X). Row lengths are drawn from three ranges (short rows, rows held in
registers, streamed rows), so the cases cross every plan's branch points.
About a third of the filter cases pass row-strided views (each operand in a
buffer padded by 1-70 elements per row, so most row strides are not a
multiple of 16 bytes), and the padding must stay untouched. Of the other
raw-logits filter cases about a fifth pass element-strided views: logits
transposed or every second column, out transposed or every third column,
and p, k and min_p with strides 2, 3 and 2; out's other elements must stay
untouched."""

import numpy as np
import pytest

from oracle import apply_top_k_top_p as o_apply
from oracle import apply_top_k_top_p_with_sorted as o_sorted
from oracle import sample_top_k_top_p as o_sample
from oracle import sorted_survivors as o_surv
from tests.gpu_util import SENTINEL, from_dev, gpu_apply, gpu_with_sorted, k_dev, need_gpu, padded_dev, say, to_dev
from tests.parity import compare, compare_samples, compare_survivors
from workloads.synth import random_min_p, random_params, random_rows, stable_ascending_sort

pytestmark = pytest.mark.gpu

KINDS = ("normal", "ties", "gumbel", "spikes", "const", "zeros")


def _case(rng):
    dtype = str(rng.choice(["f32", "f16", "bf16"]))
    band = int(rng.integers(0, 3))
    V = int([rng.integers(2, 300), rng.integers(300, 20000), rng.integers(20000, 300000)][band])
    B = int(rng.integers(1, 5))
    kind = str(rng.choice(KINDS))
    seed = int(rng.integers(1, 1 << 30))
    xb = random_rows(seed, B, V, dtype, kind=kind, scale=float(rng.choice([0.5, 2.0, 4.0])))
    k, p = random_params(seed, B, V, dtype, k_lo=-1, k_hi=min(V + 2, 5000))
    mp = random_min_p(seed, B, dtype, specials=True) if rng.random() < 0.4 else None
    pp = p if rng.random() < 0.8 else None
    kk = k if (pp is None or rng.random() < 0.7) else None
    return dtype, B, V, kind, seed, xb, kk, pp, mp


def strided_apply(xb, dtype, p, k, mp, pads):
    """The filter on row-strided views of padded buffers; returns the [B, V]
    result after checking that the padding is untouched."""
    import torch
    import top_logits_filtering_amd as tk

    B, V = xb.shape
    _, xv = padded_dev(xb, dtype, V + pads[0], SENTINEL[dtype])
    obuf, ov = padded_dev(np.zeros_like(xb), dtype, V + pads[1], SENTINEL[dtype])
    tk.apply_top_k_top_p(xv, to_dev(p, dtype), k_dev(k), out=ov, min_p=to_dev(mp, dtype))
    torch.cuda.synchronize()
    got = from_dev(obuf, dtype)
    assert (got[:, V:] == SENTINEL[dtype]).all(), "padding was written"
    return np.ascontiguousarray(got[:, :V])


def strided_sorted(sv, idx, dtype, p, k, logits, mp, pads):
    """The pre-sorted entry on row-strided views of padded buffers."""
    import torch
    import top_logits_filtering_amd as tk

    B, V = sv.shape
    _, svv = padded_dev(sv, dtype, V + pads[0], SENTINEL[dtype])
    ibuf = torch.from_numpy(np.full((B, V + pads[1]), -7, np.int32)).cuda()
    ibuf[:, :V] = k_dev(idx)
    xv = None if logits is None else padded_dev(logits, dtype, V + pads[2], SENTINEL[dtype])[1]
    obuf, ov = padded_dev(np.zeros_like(sv), dtype, V + pads[3], SENTINEL[dtype])
    tk.apply_top_k_top_p_with_sorted(svv, ibuf[:, :V], to_dev(p, dtype), k_dev(k), xv, out=ov,
                                     min_p=to_dev(mp, dtype))
    torch.cuda.synchronize()
    got = from_dev(obuf, dtype)
    assert (got[:, V:] == SENTINEL[dtype]).all(), "padding was written"
    return np.ascontiguousarray(got[:, :V])


def elem_apply(xb, dtype, p, k, mp, mode):
    """The filter on element-strided views (mode 0-3: logits transposed or
    every second column, out transposed or every third column); returns the
    [B, V] result after checking that out's other elements are untouched."""
    import torch
    import top_logits_filtering_amd as tk

    B, V = xb.shape
    nt = np.uint32 if dtype == "f32" else np.uint16
    if mode % 2 == 0:
        x = to_dev(np.ascontiguousarray(xb.T), dtype).t()
    else:
        wide = np.full((B, 2 * V), SENTINEL[dtype], nt)
        wide[:, ::2] = xb
        x = to_dev(wide, dtype)[:, ::2]
    if mode // 2 == 0:
        obuf = to_dev(np.full((V, B), SENTINEL[dtype], nt), dtype)
        out = obuf.t()
    else:
        obuf = to_dev(np.full((B, 3 * V), SENTINEL[dtype], nt), dtype)
        out = obuf[:, ::3]

    def spaced(a, step, conv):
        if a is None:
            return None
        buf = np.zeros(step * len(a), dtype=a.dtype)
        buf[::step] = a
        return conv(buf)[::step]

    pd = spaced(p, 2, lambda a: to_dev(a, dtype))
    kd = spaced(k, 3, k_dev)
    md = spaced(mp, 2, lambda a: to_dev(a, dtype))
    tk.apply_top_k_top_p(x, pd, kd, out=out, min_p=md)
    torch.cuda.synchronize()
    whole = from_dev(obuf, dtype)
    assert int((whole != SENTINEL[dtype]).sum()) == B * V, "an element outside the view was written"
    return from_dev(out.contiguous(), dtype)


@pytest.mark.parametrize("sweep_seed", [101, 202])
def test_random_sweep(sweep_seed):
    need_gpu()
    import torch
    import top_logits_filtering_amd as tk

    rng = np.random.default_rng(sweep_seed)
    counts = {}
    try:
        for _ in range(1500):
            dtype, B, V, kind, seed, xb, kk, pp, mp = _case(rng)
            policy = int(rng.choice([0, 0, 0, 1, 2]))
            tk.set_plan_policy(policy)
            entry = str(rng.choice(["apply", "sorted", "sample", "survivors"]))
            tag = (entry, dtype, B, V, kind, seed, policy, pp is not None, kk is not None, mp is not None)
            strided = entry in ("apply", "sorted") and rng.random() < 0.35
            pads = [int(v) for v in rng.integers(1, 71, size=4)] if strided else None
            elem = int(rng.integers(0, 4)) if entry == "apply" and not strided and rng.random() < 0.2 else None
            tag = tag + (pads, elem)
            if entry == "apply":
                if strided:
                    got = strided_apply(xb, dtype, pp, kk, mp, pads)
                elif elem is not None:
                    got = elem_apply(xb, dtype, pp, kk, mp, elem)
                else:
                    got = gpu_apply(xb, dtype, pp, kk, mp)
                rep = compare(got, xb, o_apply(xb, dtype, pp, kk, min_p_bits=mp), dtype)
                assert rep.hard_mismatches == 0, (tag, rep.details[:2])
            elif entry == "sorted":
                idx, sv = stable_ascending_sort(xb, dtype)
                logits = xb if rng.random() < 0.7 else None
                if strided:
                    got = strided_sorted(sv, idx, dtype, pp, kk, logits, mp, pads)
                else:
                    got = gpu_with_sorted(sv, idx, dtype, pp, kk, logits, min_p=mp)
                rep = compare(got, xb, o_sorted(sv, idx, dtype, pp, kk, logits_bits=xb, min_p_bits=mp), dtype)
                assert rep.hard_mismatches == 0, (tag, rep.details[:2])
            elif entry == "sample":
                q = rng.exponential(1.0, size=(B, V)).astype(np.float32) if rng.random() < 0.7 else None
                sel = tk.sample_top_k_top_p(to_dev(xb, dtype), to_dev(pp, dtype), k_dev(kk), to_dev(mp, dtype),
                                            None if q is None else torch.from_numpy(q).cuda(), 1e-6)
                torch.cuda.synchronize()
                ref = o_sample(xb, dtype, pp, kk, mp, None if q is None else q.astype(np.float64), 1e-6)
                h, _, det = compare_samples(sel.cpu().numpy(), ref)
                assert h == 0, (tag, det[:2])
            else:
                cap = int(rng.choice([1, 64, 1024]))
                pr, ix, cnt = tk.top_k_top_p_sorted_survivors(to_dev(xb, dtype), to_dev(pp, dtype), k_dev(kk),
                                                              to_dev(mp, dtype), cap=cap)
                torch.cuda.synchronize()
                h, det = compare_survivors(pr.cpu().numpy().astype(np.float64), ix.cpu().numpy(), cnt.cpu().numpy(),
                                           o_surv(xb, dtype, pp, kk, mp, cap))
                assert h == 0, (tag, det[:2])
            counts[entry] = counts.get(entry, 0) + 1
    finally:
        tk.set_plan_policy(0)
    say(f"random sweep {sweep_seed}: {counts}")
