"""Calls on several streams at once (needs an MI355X): the library keeps no
state between calls and no shared device memory, so concurrent calls on
different streams, on different inputs, each give their eager result."""

import numpy as np
import pytest

from tests.gpu_util import from_dev, k_dev, need_gpu, say, to_dev
from workloads.synth import make_workload

pytestmark = pytest.mark.gpu


def test_concurrent_streams():
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    batches = [make_workload(3, rows=range(16 * i, 16 * i + 16)) for i in range(4)]
    dt = batches[0].dtype
    ins = [(to_dev(w.logits, dt), to_dev(w.p, dt), k_dev(w.k)) for w in batches]
    expect = []
    for x, p, k in ins:
        expect.append(from_dev(tk.apply_top_k_top_p(x, p, k), dt))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in ins]  # default priority
    outs = [torch.empty_like(x) for x, _, _ in ins]
    for rep in range(3):
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        for s, (x, p, k), o in zip(streams, ins, outs):
            with torch.cuda.stream(s):
                for _ in range(5):  # several calls queued on each stream
                    tk.apply_top_k_top_p(x, p, k, out=o)
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, expect)):
            assert np.array_equal(from_dev(o, dt), e), (rep, i)
    # an explicit stream argument instead of the current stream
    o = torch.empty_like(ins[0][0])
    tk.apply_top_k_top_p(*ins[0], out=o, stream=streams[1])
    streams[1].synchronize()
    assert np.array_equal(from_dev(o, dt), expect[0])
    say("concurrent streams: every call matches its eager result")
