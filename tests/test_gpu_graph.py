"""Every entry point captured in a HIP graph (through torch's graph capture of
the current stream) and replayed (needs an MI355X). The library's calls only
enqueue kernels on the given stream, with no allocation and no host
synchronisation, so a captured call must give the eager result on every
replay, with other work on the device between replays, and must follow new
input data written in place."""

import numpy as np
import pytest

from tests.gpu_util import from_dev, k_dev, need_gpu, say, to_dev
from workloads.synth import make_workload, random_min_p, stable_ascending_sort

pytestmark = pytest.mark.gpu


def _capture(torch, fn):
    """fn() once on a side stream (warm-up), then captured into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_graph_replays_every_entry():
    torch = need_gpu()
    import top_logits_filtering_amd as tk

    wl = make_workload(3, rows=range(24))
    dt = wl.dtype
    x, p, k = to_dev(wl.logits, dt), to_dev(wl.p, dt), k_dev(wl.k)
    mp = to_dev(random_min_p(11, wl.B, dt, specials=False), dt)
    q = torch.from_numpy(np.random.default_rng(3).exponential(1.0, size=(wl.B, wl.V)).astype(np.float32)).cuda()
    idx, sv_bits = stable_ascending_sort(wl.logits, dt)
    sv, si = to_dev(sv_bits, dt), k_dev(idx)

    out = torch.empty_like(x)
    out_s = torch.empty_like(x)
    sel = torch.empty(wl.B, dtype=torch.int32, device="cuda")
    probs = torch.empty((wl.B, 256), dtype=torch.float32, device="cuda")
    ind = torch.empty((wl.B, 256), dtype=torch.int32, device="cuda")
    cnt = torch.empty(wl.B, dtype=torch.int32, device="cuda")

    def calls():
        tk.apply_top_k_top_p(x, p, k, out=out, min_p=mp)
        tk.apply_top_k_top_p_with_sorted(sv, si, p, k, x, out=out_s)
        tk.sample_top_k_top_p(x, p, k, None, q, 1e-6, selected=sel)
        tk.top_k_top_p_sorted_survivors(x, p, k, None, cap=256, out=(probs, ind, cnt))

    calls()
    torch.cuda.synchronize()
    eager = [from_dev(out, dt), from_dev(out_s, dt), sel.cpu().numpy(), probs.cpu().numpy(), ind.cpu().numpy(),
             cnt.cpu().numpy()]
    g = _capture(torch, calls)
    getters = [lambda: from_dev(out, dt), lambda: from_dev(out_s, dt), lambda: sel.cpu().numpy(),
               lambda: probs.cpu().numpy(), lambda: ind.cpu().numpy(), lambda: cnt.cpu().numpy()]

    def scribble_all():
        for t in (out, out_s, probs):
            t.fill_(0.5)
        for t in (sel, ind, cnt):
            t.fill_(-3)

    for r in range(3):
        scribble_all()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (get, e) in enumerate(zip(getters, eager)):
            assert np.array_equal(get(), e), (r, i)

    # new logits written in place: the replay follows them
    wl2 = make_workload(3, rows=range(24, 48))
    x.copy_(to_dev(wl2.logits, dt))
    idx2, sv2 = stable_ascending_sort(wl2.logits, dt)
    sv.copy_(to_dev(sv2, dt))
    si.copy_(k_dev(idx2))
    torch.cuda.synchronize()
    calls()
    torch.cuda.synchronize()
    eager2 = [get() for get in getters]
    scribble_all()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    for i, (get, e) in enumerate(zip(getters, eager2)):
        assert np.array_equal(get(), e), ("new data", i)
    assert not np.array_equal(eager2[0], eager[0])
    say("graph replays: every entry point matches its eager call")
