"""CPU oracle for the top-k / top-p logits filter: Python binding of the C++17
oracle in topktopp_oracle.cpp.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import or run this module. The product path
(the HIP library and its binding) never calls it, and the oracle shares no
code with that path.

The computation itself (AKP §2 steps 1-8 on a stable ascending ranking, the
min-p stage and the sampling stage of aclnnTopKTopPSampleV2, and every reading
taken where the pages are silent) is in topktopp_oracle.cpp and documented
there. This module only allocates arrays, calls the library one batch at a
time, and hands back the output bits together with per-row traces (in
ascending rank order) that the GPU comparison rule needs. The library is
built by oracle/build_oracle.py (g++) on first use when it is missing.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "topktopp_oracle.cpp")
LIB_PATH = os.path.join(HERE, "liboracle_topktopp.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
BITS_DTYPE = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}
# Bit patterns of -inf per dtype, for callers that inspect outputs.
NEG_INF_BITS = {"f32": np.uint32(0xFF800000), "f16": np.uint16(0xFC00), "bf16": np.uint16(0xFF80)}
T_READING = {"fp32": 0, "dtype": 1}


class _Trace(ctypes.Structure):
    _fields_ = [
        ("order", ctypes.c_void_p),
        ("masked_k", ctypes.c_void_p),
        ("masked_p", ctypes.c_void_p),
        ("masked_m", ctypes.c_void_p),
        ("cum32", ctypes.c_void_p),
        ("ratio_m", ctypes.c_void_p),
        ("prob", ctypes.c_void_p),
        ("t", ctypes.c_void_p),
        ("p_active", ctypes.c_void_p),
        ("ratio_valid", ctypes.c_void_p),
    ]


@dataclass
class RowTrace:
    """Intermediate results of one row, by ascending rank (AKP §2 notation)."""

    sorted_indices: np.ndarray  # int64 [V]: original index at each rank
    top_k_mask: np.ndarray  # bool [V]
    top_p_mask: np.ndarray  # bool [V]
    probs_sum32: Optional[np.ndarray]  # float32 [V] cumulative probability, or None without top-p
    t: Optional[np.float32]  # 1 - p as compared, or None
    min_p_mask: Optional[np.ndarray] = None  # bool [V], or None without min-p
    min_p_ratio: Optional[np.ndarray] = None  # float64 [V] probability / min-p threshold, or None


@dataclass
class OracleResult:
    """Output bits plus per-row traces for the parity checker."""

    out: np.ndarray  # [B, V] bits in the logits dtype
    traces: list  # RowTrace per row (empty when traces were not requested)


@dataclass
class SampleResult:
    """Selected original index per row, with what the parity rule needs."""

    selected: np.ndarray  # int64 [B]
    filtered: OracleResult  # the filter's output and traces
    scores: list  # per row: float64 [V] score by descending rank (0 where the rank is masked), or None
    raw_scores: list  # per row: the same before the top-p / min-p masks (0 only where top-k masks), or None


@dataclass
class SurvivorsResult:
    """The survivors of each row in descending order (TKS intermediate output)."""

    probs: np.ndarray  # float64 [B, cap]: step-4 probabilities, 0 after the survivors
    indices: np.ndarray  # int64 [B, cap]: original indices, -1 after the survivors
    counts: np.ndarray  # int64 [B]
    filtered: OracleResult


def _ptr(a):
    return None if a is None else a.ctypes.data


class Oracle:
    """The oracle library at `path` (a planted-mistake copy in the tests)."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            if path != LIB_PATH:
                raise FileNotFoundError(path)
            from oracle.build_oracle import build_oracle

            build_oracle()
        lib = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        tp = ctypes.POINTER(_Trace)
        lib.oracle_apply.argtypes = [vp, i32, i64, i64, vp, vp, vp, i32, vp, tp]
        lib.oracle_with_sorted.argtypes = [vp, vp, i32, i64, i64, vp, vp, vp, vp, i32, vp, tp]
        lib.oracle_sample.argtypes = [vp, i32, i64, i64, vp, vp, vp, vp, ctypes.c_double, i32, vp, vp, vp, vp, tp]
        lib.oracle_survivors.argtypes = [vp, i32, i64, i64, vp, vp, vp, i64, i32, vp, vp, vp, vp, tp]
        for f in (lib.oracle_apply, lib.oracle_with_sorted, lib.oracle_sample, lib.oracle_survivors):
            f.restype = i32
        lib.oracle_one_minus_p.argtypes = [ctypes.c_uint32, i32, i32]
        lib.oracle_one_minus_p.restype = ctypes.c_float
        self.lib = lib

    # ---------------------------------------------------------------- helpers
    @staticmethod
    def _args(dtype, bits, p_bits, k, min_p_bits):
        if dtype not in DTYPE_CODE:
            raise ValueError(f"unknown dtype {dtype!r}")
        if p_bits is None and k is None and min_p_bits is None:
            raise ValueError("p and k are both absent (at least one is required, AKP §4)")
        bits = np.ascontiguousarray(bits, dtype=BITS_DTYPE[dtype])
        if bits.ndim != 2:
            raise ValueError("expected [B, V] bits")
        p = None if p_bits is None else np.ascontiguousarray(p_bits, dtype=BITS_DTYPE[dtype])
        kk = None if k is None else np.ascontiguousarray(k, dtype=np.int32)
        mp = None if min_p_bits is None else np.ascontiguousarray(min_p_bits, dtype=BITS_DTYPE[dtype])
        return bits, p, kk, mp

    @staticmethod
    def _trace_arrays(B, V, keep):
        if not keep:
            return None, None
        arr = dict(order=np.empty((B, V), np.int64), masked_k=np.empty((B, V), np.uint8),
                   masked_p=np.empty((B, V), np.uint8), masked_m=np.empty((B, V), np.uint8),
                   cum32=np.empty((B, V), np.float32), ratio_m=np.empty((B, V), np.float64),
                   t=np.empty(B, np.float32), p_active=np.empty(B, np.uint8), ratio_valid=np.empty(B, np.uint8))
        tr = _Trace(**{name: a.ctypes.data for name, a in arr.items()}, prob=None)
        return arr, tr

    @staticmethod
    def _traces(arr, B, with_min_p):
        if arr is None:
            return []
        out = []
        for b in range(B):
            p_on = bool(arr["p_active"][b])
            out.append(RowTrace(
                arr["order"][b], arr["masked_k"][b].view(bool), arr["masked_p"][b].view(bool),
                arr["cum32"][b] if p_on else None, np.float32(arr["t"][b]) if p_on else None,
                arr["masked_m"][b].view(bool) if with_min_p else None,
                arr["ratio_m"][b] if (with_min_p and arr["ratio_valid"][b]) else None))
        return out

    # ------------------------------------------------------------ the oracle
    def one_minus_p(self, p_bits_b, dtype: str, t_reading: str = "fp32") -> np.float32:
        """t = 1 - p as the filter compares it (AKP §2 step 6)."""
        return np.float32(self.lib.oracle_one_minus_p(int(p_bits_b), DTYPE_CODE[dtype], T_READING[t_reading]))

    def apply_top_k_top_p(self, logits_bits, dtype: str, p_bits=None, k=None, keep_traces: bool = True,
                          t_reading: str = "fp32", min_p_bits=None) -> OracleResult:
        """The aclnn entry: rank each row, then filter (AKP §6.1 call chain).

        logits_bits: [B, V] raw bits (uint32 for f32, uint16 for f16/bf16).
        p_bits, min_p_bits: [B] bits in the same dtype, or None. k: [B] int32, or None.
        """
        x, p, kk, mp = self._args(dtype, logits_bits, p_bits, k, min_p_bits)
        B, V = x.shape
        out = np.empty_like(x)
        arr, tr = self._trace_arrays(B, V, keep_traces)
        self.lib.oracle_apply(_ptr(x), DTYPE_CODE[dtype], B, V, _ptr(p), _ptr(kk), _ptr(mp), T_READING[t_reading],
                              _ptr(out), None if tr is None else ctypes.byref(tr))
        return OracleResult(out, self._traces(arr, B, mp is not None))

    def apply_top_k_top_p_with_sorted(self, sorted_value_bits, sorted_indices, dtype: str, p_bits=None, k=None,
                                      logits_bits=None, keep_traces: bool = True, t_reading: str = "fp32",
                                      min_p_bits=None) -> OracleResult:
        """The sorted-input operator ApplyTopKTopPWithSorted (AKP §1, §3):
        ranks are the given positions; with logits_bits, kept outputs are read
        from it in the original order."""
        sv, p, kk, mp = self._args(dtype, sorted_value_bits, p_bits, k, min_p_bits)
        B, V = sv.shape
        si = np.ascontiguousarray(sorted_indices, dtype=np.int64)
        xl = None if logits_bits is None else np.ascontiguousarray(logits_bits, dtype=BITS_DTYPE[dtype])
        out = np.empty_like(sv)
        arr, tr = self._trace_arrays(B, V, keep_traces)
        self.lib.oracle_with_sorted(_ptr(sv), _ptr(si), DTYPE_CODE[dtype], B, V, _ptr(p), _ptr(kk), _ptr(mp),
                                    _ptr(xl), T_READING[t_reading], _ptr(out),
                                    None if tr is None else ctypes.byref(tr))
        return OracleResult(out, self._traces(arr, B, mp is not None))

    def sample_top_k_top_p(self, logits_bits, dtype: str, p_bits=None, k=None, min_p_bits=None, q=None,
                           eps: float = 0.0, t_reading: str = "fp32") -> SampleResult:
        """Sampling after the filter (TKS "Subsequent processing"): the argmax
        without q, else QSample: the first maximum over descending ranks r of
        prob / (q[b, r] + eps). p, k and min_p may all be absent here."""
        if dtype not in DTYPE_CODE:
            raise ValueError(f"unknown dtype {dtype!r}")
        x = np.ascontiguousarray(logits_bits, dtype=BITS_DTYPE[dtype])
        B, V = x.shape
        p = None if p_bits is None else np.ascontiguousarray(p_bits, dtype=BITS_DTYPE[dtype])
        kk = None if k is None else np.ascontiguousarray(k, dtype=np.int32)
        mp = None if min_p_bits is None else np.ascontiguousarray(min_p_bits, dtype=BITS_DTYPE[dtype])
        qq = None if q is None else np.ascontiguousarray(q, dtype=np.float64)
        out = np.empty_like(x)
        sel = np.empty(B, np.int64)
        scores = None if qq is None else np.empty((B, V), np.float64)
        raw = None if qq is None else np.empty((B, V), np.float64)
        arr, tr = self._trace_arrays(B, V, True)
        self.lib.oracle_sample(_ptr(x), DTYPE_CODE[dtype], B, V, _ptr(p), _ptr(kk), _ptr(mp), _ptr(qq), float(eps),
                               T_READING[t_reading], _ptr(sel), _ptr(scores), _ptr(raw), _ptr(out), ctypes.byref(tr))
        res = OracleResult(out, self._traces(arr, B, mp is not None))
        none_rows = [None] * B
        if qq is None or V == 1:
            return SampleResult(sel, res, none_rows, none_rows)
        return SampleResult(sel, res, list(scores), list(raw))

    def sorted_survivors(self, logits_bits, dtype: str, p_bits=None, k=None, min_p_bits=None, cap: int = 1,
                         t_reading: str = "fp32") -> SurvivorsResult:
        """TKS "Intermediate result output" cut to the survivors: descending
        ranks with their step-4 probabilities and original indices."""
        if dtype not in DTYPE_CODE:
            raise ValueError(f"unknown dtype {dtype!r}")
        x = np.ascontiguousarray(logits_bits, dtype=BITS_DTYPE[dtype])
        B, V = x.shape
        p = None if p_bits is None else np.ascontiguousarray(p_bits, dtype=BITS_DTYPE[dtype])
        kk = None if k is None else np.ascontiguousarray(k, dtype=np.int32)
        mp = None if min_p_bits is None else np.ascontiguousarray(min_p_bits, dtype=BITS_DTYPE[dtype])
        out = np.empty_like(x)
        probs = np.empty((B, cap), np.float64)
        idx = np.empty((B, cap), np.int64)
        counts = np.empty(B, np.int64)
        arr, tr = self._trace_arrays(B, V, True)
        self.lib.oracle_survivors(_ptr(x), DTYPE_CODE[dtype], B, V, _ptr(p), _ptr(kk), _ptr(mp), int(cap),
                                  T_READING[t_reading], _ptr(probs), _ptr(idx), _ptr(counts), _ptr(out),
                                  ctypes.byref(tr))
        return SurvivorsResult(probs, idx, counts, OracleResult(out, self._traces(arr, B, mp is not None)))


_DEFAULT = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT


def one_minus_p(p_bits_b, dtype: str, t_reading: str = "fp32") -> np.float32:
    return default().one_minus_p(p_bits_b, dtype, t_reading)


def apply_top_k_top_p(logits_bits, dtype, p_bits=None, k=None, keep_traces=True, t_reading="fp32",
                      min_p_bits=None) -> OracleResult:
    return default().apply_top_k_top_p(logits_bits, dtype, p_bits, k, keep_traces, t_reading, min_p_bits)


def apply_top_k_top_p_with_sorted(sorted_value_bits, sorted_indices, dtype, p_bits=None, k=None, logits_bits=None,
                                  keep_traces=True, t_reading="fp32", min_p_bits=None) -> OracleResult:
    return default().apply_top_k_top_p_with_sorted(sorted_value_bits, sorted_indices, dtype, p_bits, k, logits_bits,
                                                   keep_traces, t_reading, min_p_bits)


def sample_top_k_top_p(logits_bits, dtype, p_bits=None, k=None, min_p_bits=None, q=None, eps=0.0,
                       t_reading="fp32") -> SampleResult:
    return default().sample_top_k_top_p(logits_bits, dtype, p_bits, k, min_p_bits, q, eps, t_reading)


def sorted_survivors(logits_bits, dtype, p_bits=None, k=None, min_p_bits=None, cap=1,
                     t_reading="fp32") -> SurvivorsResult:
    return default().sorted_survivors(logits_bits, dtype, p_bits, k, min_p_bits, cap, t_reading)
