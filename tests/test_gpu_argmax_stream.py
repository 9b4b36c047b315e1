"""Argmax sampling (no q, no filtered row) on rows long enough to be
streamed, which take a kernel of their own (needs an MI355X). The pick is the
top position of the stable order: the highest index holding the row maximum,
with -0 and +0 equal. Rows plant the maximum at several positions across
threads and layers, make the maximum a mix of -0 and +0, and use a ragged
length that takes the element-wise traversal. Compared with the CPU oracle."""

import numpy as np
import pytest

from oracle import sample_top_k_top_p as oracle_sample
from tests.gpu_util import k_dev, need_gpu, to_dev
from workloads.synth import f32_to_bits

pytestmark = pytest.mark.gpu


def _rows(V, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, 2.0, (4, V)).astype(np.float32)
    # row 0: the maximum at five spread positions
    for pos in rng.choice(V, 5, replace=False):
        x[0, pos] = 9.5
    # row 1: every value <= 0, the maximum zero with both signs
    x[1] = -np.abs(x[1]) - 0.5
    zeros = np.sort(rng.choice(V, 6, replace=False))
    x[1, zeros] = np.where(np.arange(6) % 2 == 0, np.float32(0.0), np.float32(-0.0))
    # row 2: the maximum in the last element only; row 3: in the first only
    x[2, V - 1] = 20.0
    x[3, 0] = 20.0
    return x


@pytest.mark.parametrize("dtype,V", [("f32", 128256), ("bf16", 200000), ("f16", 200001)])
def test_streamed_argmax(dtype, V):
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    xb = f32_to_bits(_rows(V, 4700 + V % 11), dtype)
    k = np.array([5, 0, 1, 3000], np.int32)
    p = f32_to_bits(np.array([0.9, 0.5, 1.0, 0.2], np.float32), dtype)
    for pp, kk in ((p, k), (None, k), (p, None)):
        sel = tk.sample_top_k_top_p(to_dev(xb, dtype), to_dev(pp, dtype), k_dev(kk), None, None, 0.0)
        torch.cuda.synchronize()
        got = sel.cpu().numpy().astype(np.int64)
        ref = oracle_sample(xb, dtype, pp, kk).selected
        assert np.array_equal(got, ref), (dtype, pp is None, kk is None, got, ref)
