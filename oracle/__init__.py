"""CPU oracle for the top-k / top-p logits filter (test infrastructure only).

A plain single-threaded C++17 implementation (topktopp_oracle.cpp) behind a
ctypes binding. Only the tests, the smoke check and the CPU baseline of the
benchmark may use this package. The HIP path never imports it.
"""

from .topktopp_oracle import (  # noqa: F401
    NEG_INF_BITS,
    Oracle,
    OracleResult,
    RowTrace,
    SampleResult,
    SurvivorsResult,
    apply_top_k_top_p,
    apply_top_k_top_p_with_sorted,
    one_minus_p,
    sample_top_k_top_p,
    sorted_survivors,
)
