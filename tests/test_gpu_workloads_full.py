"""Every row of every workload against the CPU oracle (needs an MI355X).

Each test runs a whole workload batch through the library in the launch
configuration the benchmark times (and, for the raw-logits workloads, under
the two forced plan policies as well), then compares every row with the
oracle on a pool of worker processes (tests/parity_pool.py). Per workload and
variant the counts of the comparison rule are printed and, when the
environment variable TOPKTOPP_REPORT_DIR names a directory, collected in
parity_full_workloads.json there: rows, positions, top-p and min-p band
positions, band mismatches and hard mismatches (which must be 0). For
workload 2 the report also counts the rows whose output would change if
1 - p were rounded to p's own dtype (the other reading of step 6, which the
oracle computes but the library does not follow).
"""

import json
import os

import numpy as np
import pytest

from tests.gpu_util import from_dev, k_dev, need_gpu, say, to_dev
from tests.parity_pool import run_batch
from workloads.synth import make_workload, min_p_for_workload

pytestmark = pytest.mark.gpu

POLICIES = {"auto": 0, "multipass": 1, "stream": 2}
ROWS_PER_JOB = {1: 1, 2: 4, 3: 4, 4: 16, 5: 2}
REPORT_NAME = "parity_full_workloads.json"


def _record(key, summary):
    """Prints one result and merges it into the report file (when asked for)."""
    say(f"{key}: {json.dumps({k: v for k, v in summary.items() if k != 'details'})}")
    d = os.environ.get("TOPKTOPP_REPORT_DIR")
    if not d:
        return
    os.makedirs(d, exist_ok=True)
    path = os.path.join(d, REPORT_NAME)
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data[key] = summary
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)


@pytest.fixture(scope="module")
def scratch(tmp_path_factory):
    return tmp_path_factory.mktemp("full_batches")


def _save(d, name, arr):
    path = str(d / f"{name}.npy")
    np.save(path, arr)
    return path


def _assert_clean(summary, what):
    assert summary["hard_mismatches"] == 0, (what, summary.get("details"))


@pytest.mark.parametrize("c", [1, 2, 3, 4])
def test_apply_every_row(c, scratch):
    """Workloads 1-4 on the sorting entry, every row, under every plan policy."""
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    wl = make_workload(c)
    say(f"workload {c}: B={wl.B} V={wl.V} {wl.dtype}")
    x, p, k = to_dev(wl.logits, wl.dtype), to_dev(wl.p, wl.dtype), k_dev(wl.k)
    outs = {}
    try:
        for name, pol in POLICIES.items():
            tk.set_plan_policy(pol)
            out = tk.apply_top_k_top_p(x, p, k)
            torch.cuda.synchronize()
            outs[name] = _save(scratch, f"apply{c}_{name}", from_dev(out, wl.dtype))
            del out
    finally:
        tk.set_plan_policy(0)
    del x
    res = run_batch(dict(kind="apply", config=c, outs=outs, r5=(c == 2)), wl.B, ROWS_PER_JOB[c])
    for name in POLICIES:
        _record(f"workload{c}/apply/{name}", res[name])
    if c == 2:
        _record("workload2/r5_dtype_reading", dict(rows=wl.B, rows_changed=res["r5_rows_changed"],
                                                  positions_changed=res["r5_positions_changed"]))
    for name in POLICIES:
        _assert_clean(res[name], (c, name))


@pytest.mark.parametrize("c", [3, 5])
def test_min_p_every_row(c, scratch):
    """The benchmark's min-p variants (min_p U[0.01, 0.2] per row), every row."""
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    wl = make_workload(c)
    mp = to_dev(min_p_for_workload(c, wl.B, wl.dtype), wl.dtype)
    p, k = to_dev(wl.p, wl.dtype), k_dev(wl.k)
    if wl.entry == "apply":
        out = tk.apply_top_k_top_p(to_dev(wl.logits, wl.dtype), p, k, min_p=mp)
        kind = "apply"
    else:
        out = tk.apply_top_k_top_p_with_sorted(to_dev(wl.sorted_value, wl.dtype), k_dev(wl.sorted_indices), p, k,
                                               to_dev(wl.logits, wl.dtype), min_p=mp)
        kind = "sorted"
    torch.cuda.synchronize()
    outs = {"auto": _save(scratch, f"minp{c}", from_dev(out, wl.dtype))}
    del out
    res = run_batch(dict(kind=kind, config=c, outs=outs, min_p=True), wl.B, ROWS_PER_JOB[c])
    _record(f"workload{c}/{kind}_min_p/auto", res["auto"])
    _assert_clean(res["auto"], c)


def test_with_sorted_every_row(scratch):
    """Workload 5 on the pre-sorted entry with and without logits, every row;
    both forms agree, and so does the sorting entry on the same logits."""
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    wl = make_workload(5)
    sv, si = to_dev(wl.sorted_value, wl.dtype), k_dev(wl.sorted_indices)
    p, k = to_dev(wl.p, wl.dtype), k_dev(wl.k)
    x = to_dev(wl.logits, wl.dtype)
    got = {}
    for name, logits in (("with_logits", x), ("without_logits", None)):
        out = tk.apply_top_k_top_p_with_sorted(sv, si, p, k, logits)
        torch.cuda.synchronize()
        got[name] = from_dev(out, wl.dtype)
    again = from_dev(tk.apply_top_k_top_p(x, p, k), wl.dtype)
    torch.cuda.synchronize()
    outs = {name: _save(scratch, f"sorted5_{name}", g) for name, g in got.items()}
    res = run_batch(dict(kind="sorted", config=5, outs=outs), wl.B, ROWS_PER_JOB[5])
    for name in outs:
        _record(f"workload5/sorted/{name}", res[name])
    for name in outs:
        _assert_clean(res[name], name)
    assert np.array_equal(got["with_logits"], got["without_logits"])
    assert np.array_equal(got["with_logits"], again)


def test_with_sorted_p_only_every_row(scratch):
    """Workload 5 with k absent (top-p alone, the benchmark's --p-only), with
    and without min-p, every row."""
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    wl = make_workload(5)
    sv, si, x = to_dev(wl.sorted_value, wl.dtype), k_dev(wl.sorted_indices), to_dev(wl.logits, wl.dtype)
    p = to_dev(wl.p, wl.dtype)
    mp = to_dev(min_p_for_workload(5, wl.B, wl.dtype), wl.dtype)
    for name, mm in (("p_only", None), ("p_only_min_p", mp)):
        out = tk.apply_top_k_top_p_with_sorted(sv, si, p, None, x, min_p=mm)
        torch.cuda.synchronize()
        path = _save(scratch, f"sorted5_{name}", from_dev(out, wl.dtype))
        del out
        res = run_batch(dict(kind="sorted", config=5, outs={"auto": path}, min_p=mm is not None, no_k=True), wl.B,
                        ROWS_PER_JOB[5])
        _record(f"workload5/sorted_{name}/auto", res["auto"])
        _assert_clean(res["auto"], name)


@pytest.mark.parametrize("variant", ["qsample", "qsample_min_p", "argmax"])
def test_sample_every_row(variant, scratch):
    """Workload 3 followed by sampling (QSample with q ~ Exp(1), eps 1e-6, or
    the argmax), every row."""
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    wl = make_workload(3)
    with_min_p = variant == "qsample_min_p"
    mp = min_p_for_workload(3, wl.B, wl.dtype) if with_min_p else None
    qpath = None
    qd = None
    if variant != "argmax":
        q = np.random.default_rng(0x5A4D).exponential(1.0, size=(wl.B, wl.V)).astype(np.float32)
        qpath = _save(scratch, "q3", q)
        qd = torch.from_numpy(q).cuda()
    sel = tk.sample_top_k_top_p(to_dev(wl.logits, wl.dtype), to_dev(wl.p, wl.dtype), k_dev(wl.k),
                                to_dev(mp, wl.dtype), qd, 1e-6)
    torch.cuda.synchronize()
    g = sel.cpu().numpy()
    assert ((g >= 0) & (g < wl.V)).all()
    outs = {"auto": _save(scratch, f"sample3_{variant}", g)}
    res = run_batch(dict(kind="sample", config=3, outs=outs, q=qpath, min_p=with_min_p), wl.B, ROWS_PER_JOB[3])
    _record(f"workload3/sample_{variant}/auto", res["auto"])
    _assert_clean(res["auto"], variant)


def test_survivors_every_row(scratch):
    """Workload 3's sorted survivors (capacity 1024), every row; the
    indices-only call gives the same indices and counts."""
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    wl = make_workload(3)
    x, p, k = to_dev(wl.logits, wl.dtype), to_dev(wl.p, wl.dtype), k_dev(wl.k)
    pr, ix, cn = tk.top_k_top_p_sorted_survivors(x, p, k, None, cap=1024)
    _, ix2, cn2 = tk.top_k_top_p_sorted_survivors(x, p, k, None, cap=1024, with_probs=False)
    torch.cuda.synchronize()
    assert torch.equal(ix, ix2) and torch.equal(cn, cn2)
    outs = {"auto": (_save(scratch, "surv3_p", pr.cpu().numpy()), _save(scratch, "surv3_i", ix.cpu().numpy()),
                     _save(scratch, "surv3_c", cn.cpu().numpy()))}
    res = run_batch(dict(kind="survivors", config=3, outs=outs, cap=1024), wl.B, ROWS_PER_JOB[3])
    _record("workload3/survivors_cap1024/auto", res["auto"])
    _assert_clean(res["auto"], "survivors")
