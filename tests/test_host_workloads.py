"""Host-side checks of the benchmark's inputs and bookkeeping (CPU only): the
synthetic workloads have the shapes, value distributions and parameter ranges
they are described with, are reproducible from their seeds, and the
algorithmic byte counts follow their closed forms; a request for more than
one GPU is refused before anything touches a GPU."""

import os
import subprocess
import sys

import numpy as np
import pytest

from workloads.synth import bits_to_f32, make_workload, split_modes, stable_ascending_sort

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("c,B,V,dtype", [(1, 4, 1000, "f32"), (2, 64, 32000, "f16"), (3, 256, 151936, "bf16"),
                                         (4, 1024, 128256, "f32"), (5, 128, 262144, "bf16")])
def test_workload_shapes_and_parameters(c, B, V, dtype):
    wl = make_workload(c, rows=range(3))  # three rows are enough for the value checks
    assert (wl.B, wl.V, wl.dtype) == (3, V, dtype)
    full = make_workload(c, rows=[B - 1])  # the last row exists
    assert full.B == 1
    k = make_workload(c, rows=range(min(B, 64))).k
    if c == 1:
        assert ((k >= 1) & (k <= 50)).all()
    elif c == 2:
        off = (k == 0) | (k >= V)
        assert ((k[~off] >= 1) & (k[~off] <= 200)).all()
    elif c in (3, 4):
        assert ((k >= 0) & (k <= 1024)).all()  # workload 3 passes k = 0 for its top-p-only rows
    else:
        assert ((k >= 1) & (k <= 4096)).all()
    x = bits_to_f32(wl.logits, dtype)
    assert np.isfinite(x).all()
    if c == 4:  # multiples of 0.25
        assert np.array_equal(x * 4, np.rint(x * 4))
    if c == 2:  # eight spikes at +12 per row
        assert ((x == 12.0).sum(axis=1) >= 8).all()


def test_workloads_are_reproducible():
    a = make_workload(2, rows=[5, 9])
    b = make_workload(2, rows=[9, 5])
    assert np.array_equal(a.logits[0], b.logits[1]) and np.array_equal(a.logits[1], b.logits[0])
    assert np.array_equal(a.p, b.p[::-1]) and np.array_equal(a.k, b.k[::-1])


def test_workload3_modes():
    wl = make_workload(3, rows=range(9))
    assert list(wl.modes) == [0, 1, 2] * 3
    p = bits_to_f32(wl.p, "bf16")
    assert (p[wl.modes == 0] == 1.0).all() and (wl.k[wl.modes == 1] == 0).all()
    parts = split_modes(wl)  # three calls with p or k truly absent
    assert sorted(np.concatenate([pos for pos, _, _ in parts]).tolist()) == list(range(9))
    assert [(pp is None, kk is None) for _, pp, kk in parts] == [(True, False), (False, True), (False, False)]
    # the k-only rows' k and the p-only rows' p are the drawn ones; joint rows keep both
    k_joint = parts[2][2]
    assert ((k_joint >= 1) & (k_joint <= 1024)).all()
    p_only = bits_to_f32(parts[1][1], "bf16")
    assert ((p_only >= 0.79) & (p_only <= 0.99)).all()


def test_workload5_sorted_view():
    wl = make_workload(5, rows=range(2))
    idx, sv = stable_ascending_sort(wl.logits, wl.dtype)
    assert np.array_equal(sv, wl.sorted_value) and np.array_equal(idx, wl.sorted_indices)
    x = bits_to_f32(wl.sorted_value, "bf16")
    assert (np.diff(x, axis=1) >= 0).all()
    assert all(np.array_equal(np.sort(r), np.arange(wl.V)) for r in wl.sorted_indices)


def test_algorithmic_bytes_closed_forms():
    sys.path.insert(0, ROOT)
    import bench

    w3 = make_workload(3, rows=range(256))
    assert bench.algorithmic_bytes(w3) == 2 * 256 * 151936 * 2 + 256 * (2 + 4)  # 155,584,000 for the bench line
    assert bench.algorithmic_bytes(w3, with_k=False) == 2 * 256 * 151936 * 2 + 256 * 2  # k absent (top-p only)
    w5 = make_workload(5, rows=range(128))
    kept = int(np.clip(w5.k, 0, w5.V).sum())
    assert bench.algorithmic_bytes(w5) == 2 * 128 * 262144 * 2 + 128 * (2 + 4) + kept * 2
    assert bench.algorithmic_bytes(w5, with_k=False) == 3 * 128 * 262144 * 2 + 128 * 2
    assert bench.algorithmic_bytes(w5, with_logits=False) == 128 * 262144 * 2 + kept * (2 + 4) + 128 * (2 + 4)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "--gpus 1" in r.stderr
