"""Streamed rows whose candidates sit in a few threads' vectors (needs an
MI355X). The streamed plan keeps each thread's two vectors of largest maximum
from its first traversal in shared memory and fetches only the other
candidate vectors again; these rows plant many candidate vectors in one
thread (kept and fetched ones mixed), candidates spread over many threads,
ties across the kept/fetched split, and a ragged row that takes the
element-wise traversal. Compared with the CPU oracle."""

import numpy as np
import pytest

from oracle import apply_top_k_top_p as oracle_apply
from tests.gpu_util import gpu_apply, need_gpu, say
from tests.parity import ParityReport, compare
from workloads.synth import bits_to_f32, f32_to_bits

pytestmark = pytest.mark.gpu

THREADS = 1024
PER_VEC = {"f32": 4, "f16": 8, "bf16": 8}


def _planted_rows(dtype, V, seed):
    """Three rows: one thread holding a run of large vectors across its layers,
    the top values spread one per thread, and large values tied across both."""
    rng = np.random.default_rng(seed)
    pv = PER_VEC[dtype]
    span = THREADS * pv
    layers = (V + span - 1) // span
    rows = np.empty((3, V), np.float32)
    for r in range(3):
        rows[r] = rng.normal(0.0, 1.0, V).astype(np.float32)

    def put(r, t, layer, vals):
        e0 = layer * span + t * pv
        n = min(pv, V - e0)
        if n > 0:
            rows[r, e0:e0 + n] = vals[:n]

    # row 0: thread 5 holds large distinct values in 12 of its layers, thread 900 in two
    for i in range(12):
        put(0, 5, i, 10.0 + 0.25 * i + 0.01 * np.arange(pv))
    put(0, 900, 3, np.full(pv, 12.5))
    put(0, 900, layers - 1, np.full(pv, 12.75))
    # row 1: one large value per thread in a random layer
    for t in range(THREADS):
        layer = int(rng.integers(0, layers))
        e0 = layer * span + t * pv + int(rng.integers(0, pv))
        if e0 < V:
            rows[1, e0] = 6.0 + 0.5 * rng.random()
    # row 2: the value 9.0 in every lane of thread 7's first 10 layers and once in 300 other threads
    for i in range(10):
        put(2, 7, i, np.full(pv, 9.0))
    for t in rng.choice(np.arange(8, THREADS), 300, replace=False):
        e0 = int(rng.integers(0, layers)) * span + int(t) * pv
        if e0 < V:
            rows[2, e0] = 9.0
    return f32_to_bits(rows, dtype)


@pytest.mark.parametrize("dtype,V", [("f32", 128256), ("bf16", 200000), ("f16", 200001)])
def test_streamed_rows_kept_vectors(dtype, V):
    need_gpu()
    xb = _planted_rows(dtype, V, 4100 + V % 7)
    assert np.all(np.isfinite(bits_to_f32(xb, dtype)))
    total = ParityReport()
    for kk in ([1, 1, 1], [20, 300, 45], [60, 1500, 330], [0, 0, 0]):
        k = np.array(kk, np.int32)
        for pv in (None, [0.9, 0.5, 0.99]):
            p = None if pv is None else f32_to_bits(np.array(pv, np.float32), dtype)
            if p is None and not k.any():
                continue
            got = gpu_apply(xb, dtype, p, k)
            ref = oracle_apply(xb, dtype, p, k)
            rep = compare(got, xb, ref, dtype)
            assert rep.hard_mismatches == 0, (kk, pv, rep.details[:2])
            total.merge(rep)
    say(f"streamed planted rows {dtype} V={V}: {total}")
