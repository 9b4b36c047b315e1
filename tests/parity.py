"""GPU-vs-oracle comparison rule for the top-k / top-p filter.

Per row, with o the oracle output and its trace, and g the GPU output:
  1. every position the oracle masks by top-k is -inf in g (bit-exact);
  2. every position the oracle keeps holds the input bits in g, unless it is a
     band position;
  3. every position the oracle masks only by top-p or min-p is -inf in g,
     unless it is a band position of that stage;
  4. g holds nothing but input bits or the dtype's -inf pattern;
  5. g's survivors form a suffix of the stable ascending order.
A top-p band position is a sorted position j != V-1 whose oracle fp32
cumulative probability lies within ``tol`` (1e-5) of t = 1 - p. Summation order
on the GPU differs from the oracle's, so only there may the top-p decision
differ. A min-p band position is one whose oracle probability lies within a
relative ``tol`` of the min-p threshold: the GPU takes exp in fp32, so only
there may the min-p decision differ.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

NEG_INF_WORD = {"f32": 0xFF800000, "f16": 0xFC00, "bf16": 0xFF80}
BAND_TOL = 1e-5


@dataclass
class ParityReport:
    rows: int = 0
    positions: int = 0
    band_positions: int = 0
    band_mismatches: int = 0
    hard_mismatches: int = 0
    # the same split by stage: top-p band and min-p band (a position may be in both)
    band_positions_p: int = 0
    band_mismatches_p: int = 0
    band_positions_m: int = 0
    band_mismatches_m: int = 0
    details: list = field(default_factory=list)

    COUNTS = ("rows", "positions", "band_positions", "band_mismatches", "hard_mismatches", "band_positions_p",
              "band_mismatches_p", "band_positions_m", "band_mismatches_m")

    def merge(self, other: "ParityReport"):
        for name in self.COUNTS:
            setattr(self, name, getattr(self, name) + getattr(other, name))
        self.details.extend(other.details)
        return self

    def summary(self) -> dict:
        """The counts as a dict, with the first few mismatch details."""
        d = {name: getattr(self, name) for name in self.COUNTS}
        d["details"] = self.details[:3]
        return d

    def __str__(self):
        return (f"rows={self.rows} positions={self.positions} band={self.band_positions} "
                f"band_mismatches={self.band_mismatches} hard_mismatches={self.hard_mismatches}")


def compare_row(g_row, x_row, trace, dtype, tol=BAND_TOL, row_id=None) -> ParityReport:
    """Apply the rule to one row; x_row are the bits the kept values must equal."""
    rep = ParityReport(rows=1, positions=len(g_row))
    neg = np.asarray(NEG_INF_WORD[dtype], dtype=g_row.dtype)
    perm = trace.sorted_indices
    V = len(g_row)
    gs = g_row[perm]
    xs = x_row[perm]
    is_neg = gs == neg
    is_x = gs == xs
    mask_m = trace.min_p_mask if trace.min_p_mask is not None else np.zeros(V, dtype=bool)
    o_masked = trace.top_k_mask | trace.top_p_mask | mask_m
    # min-p's own decision, probability below the threshold: the oracle's
    # trace also marks every position top-p masked (their probability is set
    # aside), but those are top-p's decisions, and inside top-p's band the GPU
    # may keep them
    own_m = mask_m if trace.min_p_ratio is None else (trace.min_p_ratio < 1.0)
    band_p = np.zeros(V, dtype=bool)
    if trace.probs_sum32 is not None and trace.t is not None:
        band_p = np.abs(trace.probs_sum32.astype(np.float64) - np.float64(trace.t)) <= tol
        band_p[V - 1] = False
    band_m = np.zeros(V, dtype=bool)
    if trace.min_p_ratio is not None:
        band_m = np.abs(trace.min_p_ratio - 1.0) <= tol
        band_m[V - 1] = False
    # top-k decisions are exact: a position top-k masks is never a band position
    band_p &= ~trace.top_k_mask
    band_m &= ~trace.top_k_mask
    band = band_p | band_m
    ambiguous_val = xs == neg  # input already -inf: kept and masked look the same
    # a stage forces a mask where it masks outside its band, and allows a keep
    # where it keeps or is inside its band
    must_mask = trace.top_k_mask | (trace.top_p_mask & ~band_p) | (own_m & ~band_m)
    must_keep = ~trace.top_k_mask & ~(trace.top_p_mask | band_p) & ~(own_m | band_m)
    bad = ~(is_neg | is_x)  # rule 4
    bad |= must_mask & ~is_neg  # rules 1 and 3
    bad |= must_keep & ~is_x  # rule 2
    # rule 5: survivors are a suffix of the stable order
    kept = is_x & ~is_neg
    kept_or_amb = kept | ambiguous_val
    if kept.any():
        first = int(np.argmax(kept))
        if not kept_or_amb[first:].all():
            bad[first:] |= ~kept_or_amb[first:]
    n_bad = int(bad.sum())
    rep.hard_mismatches = n_bad
    rep.band_positions = int(band.sum())
    g_masked = is_neg & ~ambiguous_val
    differs = g_masked != (o_masked & ~ambiguous_val)
    rep.band_mismatches = int((band & differs).sum())
    rep.band_positions_p = int(band_p.sum())
    rep.band_mismatches_p = int((band_p & differs).sum())
    rep.band_positions_m = int(band_m.sum())
    rep.band_mismatches_m = int((band_m & differs).sum())
    if n_bad:
        js = np.nonzero(bad)[0][:5]
        rep.details.append(dict(row=row_id, sorted_positions=js.tolist(), orig=perm[js].tolist(),
                                g=gs[js].tolist(), x=xs[js].tolist(), maskK=trace.top_k_mask[js].tolist(),
                                maskP=trace.top_p_mask[js].tolist(), maskM=mask_m[js].tolist()))
    return rep


def compare(g, x_bits, oracle_result, dtype, tol=BAND_TOL, row_ids=None) -> ParityReport:
    """Apply the rule to every row of a batch."""
    rep = ParityReport()
    for b, tr in enumerate(oracle_result.traces):
        rid = b if row_ids is None else int(row_ids[b])
        rep.merge(compare_row(g[b], x_bits[b], tr, dtype, tol, rid))
    return rep


def compare_samples(g_sel, sample_result, tol=BAND_TOL):
    """Sampling rule: per row the GPU's pick equals the oracle's, unless the
    row is a near tie: the GPU's pick must then be an oracle survivor or a
    band position of top-p or min-p (kept or masked on the GPU within the
    tolerance), and its score (probability over q + eps, at its descending
    rank) must be within a relative ``tol`` of the best oracle survivor's.
    Returns (hard mismatches, near-tie mismatches, details)."""
    hard, soft, details = 0, 0, []
    for b, (o, tr) in enumerate(zip(sample_result.selected, sample_result.filtered.traces)):
        g = int(g_sel[b])
        if g == int(o):
            continue
        sc = sample_result.scores[b]
        raw = sample_result.raw_scores[b]
        ok = False
        if sc is not None and 0 <= g < len(tr.sorted_indices):
            V = len(tr.sorted_indices)
            pos = int(np.nonzero(tr.sorted_indices == g)[0][0])  # ascending position
            r = V - 1 - pos
            masked = tr.top_k_mask | tr.top_p_mask
            if tr.min_p_mask is not None:
                masked = masked | tr.min_p_mask
            band = np.zeros(V, dtype=bool)
            if tr.probs_sum32 is not None and tr.t is not None:
                band |= np.abs(tr.probs_sum32.astype(np.float64) - np.float64(tr.t)) <= tol
            if tr.min_p_ratio is not None:
                band |= np.abs(tr.min_p_ratio - 1.0) <= tol
            eligible = (not masked[pos]) or (band[pos] and not tr.top_k_mask[pos])
            best = float(sc.max())
            ok = eligible and raw[r] >= best * (1.0 - tol)
        if ok:
            soft += 1
        else:
            hard += 1
            details.append(dict(row=b, gpu=g, oracle=int(o)))
    return hard, soft, details


def compare_survivors(g_probs, g_idx, g_cnt, surv_result, tol=BAND_TOL):
    """Sorted-survivors rule, per row:
      * the GPU's count equals the oracle's, or differs only by band positions
        of top-p / min-p (which sit at the low end of the order);
      * ranks below both counts (and the capacity) hold the same original
        index, and probabilities within a relative ``tol`` (plus 1e-30);
      * ranks past the GPU's count hold -1 and 0.
    Returns (hard mismatches, details)."""
    hard, details = 0, []
    cap = g_idx.shape[1]
    for b, tr in enumerate(surv_result.filtered.traces):
        n_o, n_g = int(surv_result.counts[b]), int(g_cnt[b])
        masked = tr.top_k_mask | tr.top_p_mask
        if tr.min_p_mask is not None:
            masked = masked | tr.min_p_mask
        V = len(tr.sorted_indices)
        band = np.zeros(V, dtype=bool)
        if tr.probs_sum32 is not None and tr.t is not None:
            band |= np.abs(tr.probs_sum32.astype(np.float64) - np.float64(tr.t)) <= tol
        if tr.min_p_ratio is not None:
            band |= np.abs(tr.min_p_ratio - 1.0) <= tol
        band &= ~tr.top_k_mask
        nband = int(band.sum())
        bad = abs(n_o - n_g) > nband
        listed = min(n_g, cap)
        m = min(n_o, n_g, cap)
        bad |= not np.array_equal(g_idx[b, :m], surv_result.indices[b, :m])
        if g_probs is not None:
            o = surv_result.probs[b, :m]
            bad |= not np.all(np.abs(g_probs[b, :m] - o) <= tol * o + 1e-30)
        bad |= not (g_idx[b, listed:] == -1).all()
        if g_probs is not None:
            bad |= not (g_probs[b, listed:] == 0).all()
        if bad:
            hard += 1
            details.append(dict(row=b, n_oracle=n_o, n_gpu=n_g, band=nband))
    return hard, details
