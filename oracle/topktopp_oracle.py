"""CPU oracle for the top-k / top-p logits filter.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import or run this module. The product path
(the HIP library and its binding) never calls it, and it shares no code with
that path: not the key transform, not the dtype widening, not the -inf
constants, not the arithmetic.

What it follows. "AKP" below is the CANN ops-nn page "ApplyTopKTopPWithSorted
的 top-k/top-p 采样过滤原理与 aclnn 调用指南" (the filter's own description);
"TKS" is Ascend's "aclnnTopKTopPSampleV2" page. For each row the filter
(AKP §2, steps 1-8, and the PyTorch golden printed after them):

  0. sorts the row ascending with a stable sort (AKP §6.1: the aclnn entry sorts
     ascending and stable before calling the sorted-input operator);
  1. takes the k-th largest value, sortedValue[V - k], as the top-k threshold;
  2-3. masks (sets to -inf) every sorted value strictly below that threshold;
       k <= 0 or k >= V means no top-k (AKP §4 and the §5.2 parameter table);
  4. takes a softmax of what remains, in fp32 or wider (the golden casts to
     float32 before the softmax);
  5. forms the ascending cumulative sum, smallest probability first;
  6. masks every position whose cumulative sum is <= 1 - p, but never the last
     (largest) position;
  7. sets those positions to -inf;
  8. scatters the result back to the original vocabulary order through the
     sort permutation.

Readings adopted where the pages are garbled or silent (the comparison
operators were lost in the page text; the prose next to each step gives them):
  * top-k masks values strictly below the threshold (step 2 prose);
  * top-p masks cumsum <= 1 - p (step 6 prose; TKS agrees);
  * step 8 is a scatter out[perm[j]] = s[j]: the golden uses scatter_, and the
    gather as typeset would not restore the original order;
  * values compare as IEEE floats, so -0.0 and +0.0 are equal and keep their
    index order; kept outputs copy the input bits, so a kept -0.0 stays -0.0;
  * the softmax and cumsum are carried out in float64 here and the cumsum is
    then rounded to fp32 (the golden's tensor dtype), which keeps the oracle's
    own rounding far below the 1e-5 tolerance band used for comparisons;
  * t = 1 - p is an fp32 subtraction (p is widened exactly from its dtype).
    ``t_reading="dtype"`` rounds 1 - p to p's own dtype instead, the other
    plausible reading of the golden, kept only to count the rows on which the
    two readings disagree;
  * with pre-sorted input, ties follow the given positions; when the original
    logits are passed, kept values are read from them (AKP §3 parameter table).

Min-p (TKS, "minP sampling"), an optional third stage after top-k and top-p.
Its probabilities are those of step 4 (the softmax over the top-k survivors),
with the positions top-p masked set aside; the threshold is the largest of
them times min_p, and positions whose probability is strictly below it are
masked. min_p <= 0 skips the stage; min_p >= 1 keeps a single token with the
maximum value, read here as the last position of the stable ascending order
(the same tie rule as p = 0). min_p is stored in the logits dtype, like p.
Every stage only masks a prefix of the stable order, so the survivors of the
three stages together are the intersection of each stage's survivors.

Pins (tests/test_oracle.py) tie every step to something other than this code:
the worked example of AKP §7 (outputs derived by hand, stored in
tests/golden/), brute-force counting for top-k, the textbook nucleus
definition accumulated from the top for top-p, the logit-space form of min-p
(x - max >= ln(min_p)) evaluated by counting, and invariants. The exact fp32
cumsum values near 1 - p are parity unpinned: the pages print none, so the
GPU comparison tolerates differences only inside a 1e-5 band around 1 - p;
likewise min-p decisions only where a probability lies within a relative
1e-5 of the min-p threshold.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

# Bit patterns of -inf per dtype (AKP §6.3 lists them as kernel constants).
NEG_INF_BITS = {"f32": np.uint32(0xFF800000), "f16": np.uint16(0xFC00), "bf16": np.uint16(0xFF80)}
BITS_DTYPE = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}


def widen_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of each stored fp32 / fp16 / bf16 bit pattern."""
    if dtype == "f32":
        return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def one_minus_p(p_bits_b, dtype: str, t_reading: str = "fp32") -> np.float32:
    """t = 1 - p as the filter compares it (AKP §2 step 6)."""
    p32 = np.float32(widen_to_f64(np.asarray([p_bits_b]), dtype)[0])
    t = np.float32(np.float32(1.0) - p32)
    if t_reading == "fp32":
        return t
    if t_reading == "dtype":
        # round 1 - p to p's own storage dtype, then widen again
        if dtype == "f32":
            return t
        if dtype == "f16":
            return np.float32(np.float16(t))
        u = np.asarray([t], dtype=np.float32).view(np.uint32).astype(np.uint64)
        r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << np.uint32(16)
        return np.float32(r.view(np.float32)[0])
    raise ValueError(t_reading)


@dataclass
class RowTrace:
    """Intermediate results of one row, in sorted order (AKP §2 notation)."""

    sorted_indices: np.ndarray  # int64 [V]
    top_k_mask: np.ndarray  # bool [V]
    top_p_mask: np.ndarray  # bool [V]
    probs_sum32: Optional[np.ndarray]  # float32 [V] cumulative probability, or None
    t: Optional[np.float32]  # 1 - p as compared, or None
    min_p_mask: Optional[np.ndarray] = None  # bool [V], or None without min-p
    min_p_ratio: Optional[np.ndarray] = None  # float64 [V] probability / min-p threshold, or None


def filter_sorted_row(sorted_value: np.ndarray, k_b: Optional[int], p_bits_b, dtype: str,
                      t_reading: str = "fp32", min_p_bits_b=None):
    """Steps 1-7 of AKP §2 on one ascending row of float64 values, then min-p.

    Returns (top_k_mask, top_p_mask, probs_sum32, t, min_p_mask, min_p_ratio),
    all in sorted order; the last two are None without min-p.
    """
    V = sorted_value.shape[0]
    s = sorted_value.copy()

    # Steps 1-3: the k-th largest value sits at V - k in ascending order; values
    # strictly below it are masked. k outside [1, V-1] disables top-k.
    top_k_mask = np.zeros(V, dtype=bool)
    if k_b is not None and 1 <= int(k_b) <= V - 1:
        top_k_value = s[V - int(k_b)]
        top_k_mask = s < top_k_value
        s[top_k_mask] = -np.inf

    top_p_mask = np.zeros(V, dtype=bool)
    probs_sum32 = None
    t = None
    if p_bits_b is not None:
        # Step 4: softmax over what survived top-k. The largest value sits last.
        m = s[V - 1]
        if not np.isfinite(m):
            raise ValueError("row has no finite maximum (outside the filter's contract)")
        e = np.exp(s - m)  # exactly 0 for masked (-inf) entries
        Z = np.cumsum(e)[-1]  # sequential, ascending
        probs_value = e / Z
        # Step 5: cumulative sum starting from the smallest probability.
        probs_sum = np.cumsum(probs_value)
        probs_sum32 = probs_sum.astype(np.float32)
        # Step 6: mask cumsum <= 1 - p, never the last position.
        t = one_minus_p(p_bits_b, dtype, t_reading)
        top_p_mask = probs_sum32 <= t
        top_p_mask[V - 1] = False

    min_p_mask = None
    min_p_ratio = None
    if min_p_bits_b is not None:
        min_p_mask = np.zeros(V, dtype=bool)
        mp = widen_to_f64(np.asarray([min_p_bits_b]), dtype)[0]
        if mp >= 1.0:
            # a single token with the maximum value: the last sorted position
            min_p_mask[: V - 1] = True
        elif mp > 0.0:
            # probabilities of step 4 (softmax over the top-k survivors); the
            # positions top-p masked hold -inf, as after TKS's top-p stage
            m = s[V - 1]
            e = np.exp(s - m)
            probs = e / np.cumsum(e)[-1]
            sort_masked = np.where(top_p_mask, -np.inf, probs)
            threshold = sort_masked.max() * mp
            min_p_mask = sort_masked < threshold
            min_p_ratio = probs / threshold
        # min_p <= 0 (or NaN): the stage is skipped
    return top_k_mask, top_p_mask, probs_sum32, t, min_p_mask, min_p_ratio


@dataclass
class OracleResult:
    """Output bits plus per-row traces for the parity checker."""

    out: np.ndarray  # [B, V] bits in the logits dtype
    traces: list  # RowTrace per row (empty when traces were not requested)


def _check_args(dtype: str, p, k, min_p=None):
    if dtype not in NEG_INF_BITS:
        raise ValueError(f"unknown dtype {dtype!r}")
    if p is None and k is None and min_p is None:
        raise ValueError("p and k are both absent (at least one is required, AKP §4)")


def apply_top_k_top_p(logits_bits: np.ndarray, dtype: str, p_bits: Optional[np.ndarray] = None,
                      k: Optional[np.ndarray] = None, keep_traces: bool = True,
                      t_reading: str = "fp32", min_p_bits: Optional[np.ndarray] = None) -> OracleResult:
    """The aclnn entry: sort each row, then filter (AKP §6.1 call chain).

    logits_bits: [B, V] raw bits (uint32 for f32, uint16 for f16/bf16).
    p_bits: [B] bits in the same dtype, or None. k: [B] int32, or None.
    min_p_bits: [B] bits in the same dtype, or None (TKS min-p stage).
    """
    _check_args(dtype, p_bits, k, min_p_bits)
    logits_bits = np.asarray(logits_bits, dtype=BITS_DTYPE[dtype])
    B, V = logits_bits.shape
    out = np.empty_like(logits_bits)
    traces = []
    for b in range(B):
        row_bits = logits_bits[b]
        if V == 1:
            # A last dimension of 1 is copied through (AKP §6.1).
            out[b] = row_bits
            if keep_traces:
                traces.append(RowTrace(np.zeros(1, np.int64), np.zeros(1, bool), np.zeros(1, bool), None, None))
            continue
        x = widen_to_f64(row_bits, dtype)
        sorted_indices = np.argsort(x, kind="stable")  # ascending; equal values keep index order
        sorted_value = x[sorted_indices]
        kb = None if k is None else int(k[b])
        pb = None if p_bits is None else p_bits[b]
        mpb = None if min_p_bits is None else min_p_bits[b]
        top_k_mask, top_p_mask, probs_sum32, t, min_p_mask, min_p_ratio = filter_sorted_row(
            sorted_value, kb, pb, dtype, t_reading, mpb)
        masked = top_k_mask | top_p_mask
        if min_p_mask is not None:
            masked = masked | min_p_mask
        # Step 8: scatter back to the original order; kept entries are the input bits.
        sorted_bits = np.where(masked, NEG_INF_BITS[dtype], row_bits[sorted_indices])
        out[b, sorted_indices] = sorted_bits
        if keep_traces:
            traces.append(RowTrace(sorted_indices, top_k_mask, top_p_mask, probs_sum32, t, min_p_mask, min_p_ratio))
    return OracleResult(out, traces)


def apply_top_k_top_p_with_sorted(sorted_value_bits: np.ndarray, sorted_indices: np.ndarray, dtype: str,
                                  p_bits: Optional[np.ndarray] = None, k: Optional[np.ndarray] = None,
                                  logits_bits: Optional[np.ndarray] = None, keep_traces: bool = True,
                                  t_reading: str = "fp32",
                                  min_p_bits: Optional[np.ndarray] = None) -> OracleResult:
    """The sorted-input operator ApplyTopKTopPWithSorted (AKP §1, §3).

    sorted_value_bits must be ascending and sorted_indices the matching
    permutation; positions in the given order decide ties. If logits_bits is
    given, kept outputs are read from it in the original order. min_p_bits
    adds the TKS min-p stage, as in apply_top_k_top_p.
    """
    _check_args(dtype, p_bits, k, min_p_bits)
    sorted_value_bits = np.asarray(sorted_value_bits, dtype=BITS_DTYPE[dtype])
    B, V = sorted_value_bits.shape
    out = np.empty_like(sorted_value_bits)
    traces = []
    for b in range(B):
        perm = np.asarray(sorted_indices[b], dtype=np.int64)
        if V == 1:
            src = sorted_value_bits[b] if logits_bits is None else logits_bits[b]
            out[b] = src
            if keep_traces:
                traces.append(RowTrace(perm, np.zeros(1, bool), np.zeros(1, bool), None, None))
            continue
        s = widen_to_f64(sorted_value_bits[b], dtype)
        kb = None if k is None else int(k[b])
        pb = None if p_bits is None else p_bits[b]
        mpb = None if min_p_bits is None else min_p_bits[b]
        top_k_mask, top_p_mask, probs_sum32, t, min_p_mask, min_p_ratio = filter_sorted_row(
            s, kb, pb, dtype, t_reading, mpb)
        masked = top_k_mask | top_p_mask
        if min_p_mask is not None:
            masked = masked | min_p_mask
        if logits_bits is None:
            out[b, perm] = np.where(masked, NEG_INF_BITS[dtype], sorted_value_bits[b])
        else:
            keep = np.zeros(V, dtype=bool)
            keep[perm] = ~masked
            out[b] = np.where(keep, logits_bits[b], NEG_INF_BITS[dtype])
        if keep_traces:
            traces.append(RowTrace(perm, top_k_mask, top_p_mask, probs_sum32, t, min_p_mask, min_p_ratio))
    return OracleResult(out, traces)


@dataclass
class SampleResult:
    """Selected original index per row, with what the parity rule needs."""

    selected: np.ndarray  # int64 [B]
    filtered: OracleResult  # the filter's output and traces
    scores: list  # per row: float64 [V] score by descending rank (0 where the rank is masked), or None
    raw_scores: list  # per row: the same before the top-p / min-p masks (0 only where top-k masks), or None


def sample_top_k_top_p(logits_bits: np.ndarray, dtype: str, p_bits: Optional[np.ndarray] = None,
                       k: Optional[np.ndarray] = None, min_p_bits: Optional[np.ndarray] = None,
                       q: Optional[np.ndarray] = None, eps: float = 0.0, t_reading: str = "fp32") -> SampleResult:
    """Sampling after the filter, TKS "Subsequent processing".

    probs is the filter's result in descending order: the probabilities of
    step 4 (softmax over the top-k survivors) at the surviving positions, zero
    elsewhere. Descending order is read as the reverse of the stable ascending
    sort, so among equal values the higher original index comes first.
      * None mode (q is None): the index of ArgMax(probs), the first maximum:
        the maximum value with the highest original index.
      * QSample (q [B, V] float): probsOpt = probs / (q[b, :qCnt] + eps), where
        q's entry r pairs with descending rank r, and the index of the first
        maximum of probsOpt. qCnt counts the positions min-p keeps (every
        position when min-p is skipped); positions masked by any stage have
        zero probability and cannot win, so the ranks that matter are those
        of the survivors, 0 .. n_s - 1.
    """
    res = apply_top_k_top_p(logits_bits, dtype, p_bits, k, keep_traces=True, t_reading=t_reading,
                            min_p_bits=min_p_bits)
    B, V = np.asarray(logits_bits).shape
    selected = np.zeros(B, dtype=np.int64)
    scores = []
    raw_scores = []
    for b in range(B):
        tr = res.traces[b]
        perm = tr.sorted_indices  # ascending
        if V == 1:
            selected[b] = 0
            scores.append(None)
            raw_scores.append(None)
            continue
        masked = tr.top_k_mask | tr.top_p_mask
        if tr.min_p_mask is not None:
            masked = masked | tr.min_p_mask
        desc = perm[::-1]  # descending rank r -> original index
        kept_desc = ~masked[::-1]
        if q is None:
            selected[b] = int(desc[0])
            scores.append(None)
            raw_scores.append(None)
            continue
        x = widen_to_f64(np.asarray(logits_bits)[b], dtype)[desc]
        # step 4 probabilities: softmax over the top-k survivors
        xk = np.where(tr.top_k_mask[::-1], -np.inf, x)
        e = np.exp(xk - xk[0])
        step4 = e / e.sum()
        probs = np.where(kept_desc, step4, 0.0)
        qb = np.asarray(q[b], dtype=np.float64)
        score = probs / (qb + float(eps))
        score = np.where(kept_desc, score, 0.0)
        r = int(np.argmax(score))  # first maximum
        selected[b] = int(desc[r])
        scores.append(score)
        raw_scores.append(step4 / (qb + float(eps)))
    return SampleResult(selected, res, scores, raw_scores)


@dataclass
class SurvivorsResult:
    """The survivors of each row in descending order (TKS intermediate output)."""

    probs: np.ndarray  # float64 [B, cap]: step-4 probabilities, 0 after the survivors
    indices: np.ndarray  # int64 [B, cap]: original indices, -1 after the survivors
    counts: np.ndarray  # int64 [B]
    filtered: OracleResult


def sorted_survivors(logits_bits: np.ndarray, dtype: str, p_bits: Optional[np.ndarray] = None,
                     k: Optional[np.ndarray] = None, min_p_bits: Optional[np.ndarray] = None, cap: int = 1,
                     t_reading: str = "fp32") -> SurvivorsResult:
    """TKS "Intermediate result output": logitsSortMasked and logitsIdx, the
    filtered probabilities in descending order with their original indices,
    cut to the survivors (the masked tail, zeros in TKS, is not listed).
    The probabilities are those of step 4: the softmax over the top-k
    survivors. Descending order is the reverse of the stable ascending sort."""
    res = apply_top_k_top_p(logits_bits, dtype, p_bits, k, keep_traces=True, t_reading=t_reading,
                            min_p_bits=min_p_bits)
    B, V = np.asarray(logits_bits).shape
    probs = np.zeros((B, cap), dtype=np.float64)
    indices = np.full((B, cap), -1, dtype=np.int64)
    counts = np.zeros(B, dtype=np.int64)
    for b in range(B):
        tr = res.traces[b]
        masked = tr.top_k_mask | tr.top_p_mask
        if tr.min_p_mask is not None:
            masked = masked | tr.min_p_mask
        desc = tr.sorted_indices[::-1]
        kept_desc = ~masked[::-1]
        n = int(kept_desc.sum())  # a prefix of the descending order
        counts[b] = n
        x = widen_to_f64(np.asarray(logits_bits)[b], dtype)[desc]
        xk = np.where(tr.top_k_mask[::-1], -np.inf, x)
        e = np.exp(xk - xk[0])
        step4 = e / e.sum()
        m = min(n, cap)
        probs[b, :m] = step4[:m]
        indices[b, :m] = desc[:m]
    return SurvivorsResult(probs, indices, counts, res)
