"""The GPU-vs-oracle comparison rule itself, exercised on the CPU with the
oracle's own output standing in for a GPU result."""

import numpy as np

from oracle import apply_top_k_top_p
from tests.parity import NEG_INF_WORD, compare
from workloads.synth import f32_to_bits, random_rows


def _case(min_p=True):
    dtype = "bf16"
    xb = random_rows(31, 6, 400, dtype, kind="normal")
    rng = np.random.default_rng(3)
    k = rng.integers(1, 399, size=6).astype(np.int32)
    p = f32_to_bits(rng.uniform(0.3, 0.95, size=6).astype(np.float32), dtype)
    mp = f32_to_bits(rng.uniform(0.01, 0.3, size=6).astype(np.float32), dtype) if min_p else None
    ref = apply_top_k_top_p(xb, dtype, p, k, min_p_bits=mp)
    return dtype, xb, ref


def test_oracle_output_passes():
    for min_p in (False, True):
        dtype, xb, ref = _case(min_p)
        rep = compare(ref.out.copy(), xb, ref, dtype)
        assert rep.hard_mismatches == 0 and rep.band_mismatches == 0


def test_flipped_survivor_is_caught():
    dtype, xb, ref = _case()
    g = ref.out.copy()
    b = 0
    kept = np.nonzero(g[b] != NEG_INF_WORD[dtype])[0]
    g[b, kept[0]] = NEG_INF_WORD[dtype]  # drop a survivor outside any band
    tr = ref.traces[b]
    j = int(np.nonzero(tr.sorted_indices == kept[0])[0][0])
    in_band = (tr.min_p_ratio is not None and abs(tr.min_p_ratio[j] - 1) <= 1e-5) or (
        abs(float(tr.probs_sum32[j]) - float(tr.t)) <= 1e-5)
    rep = compare(g, xb, ref, dtype)
    assert in_band or rep.hard_mismatches >= 1


def test_resurrected_min_p_position_is_caught():
    dtype, xb, ref = _case()
    for b, tr in enumerate(ref.traces):
        only_m = tr.min_p_mask & ~tr.top_k_mask & ~tr.top_p_mask & (np.abs(tr.min_p_ratio - 1) > 1e-5)
        if only_m.any():
            j = int(np.nonzero(only_m)[0][-1])
            g = ref.out.copy()
            g[b, tr.sorted_indices[j]] = xb[b, tr.sorted_indices[j]]
            assert compare(g, xb, ref, dtype).hard_mismatches >= 1
            return
    raise AssertionError("no row has a position masked by min-p alone")


def test_foreign_value_is_caught():
    dtype, xb, ref = _case(False)
    g = ref.out.copy()
    g[1, 5] = np.uint16(0x3F80)  # 1.0, neither the input bits nor -inf (unless equal)
    rep = compare(g, xb, ref, dtype)
    assert xb[1, 5] == 0x3F80 or rep.hard_mismatches >= 1


def test_sample_rule():
    from oracle import sample_top_k_top_p
    from tests.parity import compare_samples

    dtype = "bf16"
    xb = random_rows(37, 8, 300, dtype, kind="normal")
    rng = np.random.default_rng(5)
    k = rng.integers(5, 200, size=8).astype(np.int32)
    q = rng.exponential(1.0, size=(8, 300))
    res = sample_top_k_top_p(xb, dtype, None, k, None, q, 0.0)
    assert compare_samples(res.selected, res)[0] == 0
    bad = res.selected.copy()
    # a masked position (the row's minimum) is never an allowed pick
    bad[0] = int(res.filtered.traces[0].sorted_indices[0])
    assert compare_samples(bad, res)[0] == 1


def test_top_p_band_position_with_min_p():
    """With min-p on, a position top-p masks inside its band may still be kept:
    the oracle's min-p trace also marks the positions top-p masked, but those
    are top-p's decisions. A long row of equal values puts several positions in
    the top-p band (each holds 1/V < 1e-5 of the mass)."""
    dtype, V = "bf16", 200000
    xb = np.zeros((1, V), dtype=np.uint16)  # every value +0.0
    p = f32_to_bits(np.array([0.026], np.float32), dtype)
    mp = f32_to_bits(np.array([1e-3], np.float32), dtype)
    ref = apply_top_k_top_p(xb, dtype, p, None, min_p_bits=mp)
    tr = ref.traces[0]
    band = np.abs(tr.probs_sum32.astype(np.float64) - float(tr.t)) <= 1e-5
    masked_band = np.nonzero(band & tr.top_p_mask)[0]
    assert len(masked_band) > 0
    g = ref.out.copy()
    j = int(masked_band[-1])  # the band position just below the survivors: kept on the "GPU"
    g[0, tr.sorted_indices[j]] = xb[0, tr.sorted_indices[j]]
    rep = compare(g, xb, ref, dtype)
    assert rep.hard_mismatches == 0 and rep.band_mismatches == 1
    # outside the band the same change is still an error
    g = ref.out.copy()
    far = int(np.nonzero(tr.top_p_mask & ~band)[0][-1])
    g[0, tr.sorted_indices[far]] = xb[0, tr.sorted_indices[far]]
    assert compare(g, xb, ref, dtype).hard_mismatches >= 1


def test_worker_pool_on_oracle_outputs(tmp_path):
    """The whole-batch harness (tests/parity_pool.py) on the CPU: the
    oracle's own outputs for workloads 1 and 2 pass on every row, and a
    survivor dropped from one row is caught in that row."""
    from tests.parity_pool import run_batch
    from workloads.synth import make_workload

    for c, rows_per_job in ((1, 1), (2, 16)):
        wl = make_workload(c)
        ref = apply_top_k_top_p(wl.logits, wl.dtype, wl.p, wl.k, keep_traces=False).out
        good = str(tmp_path / f"good{c}.npy")
        np.save(good, ref)
        bad_out = ref.copy()
        b = wl.B - 1
        top = int(np.nonzero(bad_out[b] != NEG_INF_WORD[wl.dtype])[0][-1])
        bad_out[b, top] = NEG_INF_WORD[wl.dtype]
        bad = str(tmp_path / f"bad{c}.npy")
        np.save(bad, bad_out)
        res = run_batch(dict(kind="apply", config=c, outs={"good": good, "bad": bad}, r5=(c == 2)), wl.B,
                        rows_per_job)
        assert res["good"]["rows"] == wl.B and res["good"]["hard_mismatches"] == 0
        assert res["bad"]["hard_mismatches"] >= 1 and res["bad"]["details"][0]["row"] == b
        if c == 2:
            assert 0 <= res["r5_rows_changed"] <= wl.B
