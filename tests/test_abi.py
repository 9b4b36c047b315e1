"""The C ABI without a GPU: the library loads, exports what the header
declares, and rejects bad arguments on the host before touching HIP."""

import ctypes
import os
import re

import pytest

import top_logits_filtering_amd as tk
from top_logits_filtering_amd.binding import LIB_PATH

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "topktopp.h")

NULLPTR, INVALID = 1, 2
FAKE = 1 << 40  # a device-looking address; never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        from top_logits_filtering_amd.build import build

        build()
    return tk.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(tk.EXPORTED_SYMBOLS), names
    for n in names:
        assert hasattr(lib, n), n


def test_null_pointers(lib):
    f = lib.apply_top_k_top_p
    assert f(None, 0, 2, 8, FAKE, FAKE, FAKE, None) == NULLPTR
    assert "logits" in tk.last_error()
    assert f(FAKE, 0, 2, 8, FAKE, FAKE, None, None) == NULLPTR
    assert f(FAKE, 0, 2, 8, None, None, FAKE + (1 << 30), None) == NULLPTR
    assert "p and k" in tk.last_error()
    g = lib.apply_top_k_top_p_with_sorted
    assert g(None, FAKE, 0, 2, 8, FAKE, None, None, FAKE + (1 << 30), None) == NULLPTR
    assert g(FAKE, None, 0, 2, 8, FAKE, None, None, FAKE + (1 << 30), None) == NULLPTR
    assert g(FAKE, FAKE, 0, 2, 8, None, None, None, FAKE + (1 << 30), None) == NULLPTR


def test_min_p_entry_points(lib):
    f = lib.apply_top_k_top_p_min_p
    out = FAKE + (1 << 32)
    # min_p alone is enough; all three absent is not
    assert f(FAKE, 0, 2, 8, None, None, None, out, None) == NULLPTR
    assert "min_p" in tk.last_error()
    assert f(FAKE, 5, 2, 8, None, None, FAKE, out, None) == INVALID  # reaches the dtype check
    assert f(FAKE, 0, 2, 8, None, None, out + 4, out, None) == INVALID
    assert "overlap" in tk.last_error()
    g = lib.apply_top_k_top_p_min_p_with_sorted
    assert g(FAKE, FAKE, 0, 2, 8, None, None, None, None, out, None) == NULLPTR
    assert g(FAKE, FAKE, 7, 2, 8, None, None, FAKE, None, out, None) == INVALID
    assert g(None, None, 0, 0, 9, None, None, None, None, None, None) == 0


def test_invalid_dtype_and_shape(lib):
    f = lib.apply_top_k_top_p
    out = FAKE + (1 << 32)
    assert f(FAKE, 3, 2, 8, FAKE, None, out, None) == INVALID
    assert "dtype" in tk.last_error()
    assert f(FAKE, -1, 2, 8, FAKE, None, out, None) == INVALID
    assert f(FAKE, 0, -1, 8, FAKE, None, out, None) == INVALID
    assert f(FAKE, 0, 2, -8, FAKE, None, out, None) == INVALID
    assert f(FAKE, 2, 2, (1 << 20) + 1, FAKE, None, out, None) == INVALID
    assert "maximum" in tk.last_error()
    assert f(FAKE, 0, 1 << 31, 8, FAKE, None, out, None) == INVALID  # more rows than 2^31 - 1
    assert "rows" in tk.last_error()
    g = lib.apply_top_k_top_p_with_sorted
    assert g(FAKE, FAKE, 0, 1 << 31, 8, FAKE, None, None, out, None) == INVALID
    h = lib.sample_top_k_top_p
    assert h(FAKE, 0, 1 << 31, 8, None, None, None, None, 0.0, None, out, None) == INVALID
    s = lib.top_k_top_p_sorted_survivors
    assert s(FAKE, 0, 1 << 31, 8, None, None, None, 4, None, out, out + (1 << 20), None) == INVALID


def test_overlap_rejected(lib):
    f = lib.apply_top_k_top_p
    assert f(FAKE, 2, 4, 100, FAKE + (1 << 32), None, FAKE + 64, None) == INVALID
    assert "overlap" in tk.last_error()


def test_empty_is_ok_without_launch(lib):
    f = lib.apply_top_k_top_p
    assert f(FAKE, 1, 0, 100, None, FAKE + 8, FAKE + (1 << 32), None) == 0
    assert f(FAKE, 1, 5, 0, None, FAKE + 8, FAKE + (1 << 32), None) == 0
    assert tk.last_error() == ""
    # empty buffers may be NULL (torch hands out NULL for empty tensors)
    assert f(None, 2, 0, 151936, None, None, None, None) == 0
    assert lib.apply_top_k_top_p_with_sorted(None, None, 0, 7, 0, None, None, None, None, None) == 0
    assert f(None, 9, 0, 4, None, None, None, None) == INVALID


def test_plan_policy_roundtrip(lib):
    prev = tk.set_plan_policy(1)
    assert tk.set_plan_policy(prev) == 1
    assert lib.topktopp_set_plan_policy(7) == -1
    with pytest.raises(ValueError):
        tk.set_plan_policy(9)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="no fallback"):
        tk.load_library(str(tmp_path / "nope.so"))


def test_strided_entry_points_check_strides(lib):
    f = lib.apply_top_k_top_p_ex
    out = FAKE + (1 << 32)
    assert f(FAKE, 7, 0, 2, 8, FAKE, None, None, out, 8, None) == INVALID  # ld_logits < V
    assert "stride" in tk.last_error()
    assert f(FAKE, 8, 0, 2, 8, FAKE, None, None, out, 4, None) == INVALID  # ld_out < V
    assert f(FAKE, 1 << 32, 0, 2, 8, FAKE, None, None, out, 8, None) == INVALID
    assert "maximum" in tk.last_error()
    # the strided extent of out reaches into logits: [out, out + (2-1)*1000*4 + 8*4)
    assert f(out + 2000, 8, 0, 2, 8, FAKE, None, None, out, 1000, None) == INVALID
    assert "overlap" in tk.last_error()
    assert f(FAKE, 8, 0, 2, 8, None, None, None, out, 8, None) == NULLPTR
    g = lib.apply_top_k_top_p_with_sorted_ex
    assert g(FAKE, 8, FAKE + (1 << 34), 6, 0, 2, 8, FAKE, None, None, None, 0, out, 8, None) == INVALID
    assert "sorted_indices" in tk.last_error()
    # ld_logits is not checked when logits is NULL
    assert g(None, 8, FAKE, 8, 0, 0, 8, None, None, None, None, 0, None, 8, None) == 0


def test_element_strided_entry_point_checks(lib):
    """apply_top_k_top_p_strided: stride ranges, an out layout that gives
    every position its own element, span overlaps, and the usual order of
    checks (pointers, dtype, shape)."""
    f = lib.apply_top_k_top_p_strided
    out = FAKE + (1 << 36)

    def call(x=FAKE, xr=8, xc=1, dt=0, B=2, V=8, p=FAKE, ps=1, k=None, ks=1, mp=None, ms=1, o=out, orr=8, oc=1):
        return f(x, xr, xc, dt, B, V, p, ps, k, ks, mp, ms, o, orr, oc, None)

    assert call(x=None) == NULLPTR
    assert call(o=None) == NULLPTR
    assert call(p=None) == NULLPTR and "min_p" in tk.last_error()
    assert call(dt=3) == INVALID and "dtype" in tk.last_error()
    assert call(V=(1 << 20) + 1) == INVALID
    assert call(xc=-1) == INVALID and "logits_col_stride" in tk.last_error()
    assert call(xr=(1 << 31) + 1) == INVALID and "logits_row_stride" in tk.last_error()
    assert call(ps=-2) == INVALID and "p_stride" in tk.last_error()
    assert call(k=FAKE + (1 << 34), ks=-1) == INVALID and "k_stride" in tk.last_error()
    assert call(mp=FAKE + (1 << 35), ms=-1) == INVALID and "min_p_stride" in tk.last_error()
    assert call(orr=0, oc=1) == INVALID and "out_row_stride" in tk.last_error()
    assert call(oc=0) == INVALID and "out_col_stride" in tk.last_error()
    # out strides that map two positions to one element: (b, v) -> 3b + v
    assert call(orr=3, oc=1) == INVALID and "map two positions" in tk.last_error()
    assert call(B=3, orr=2, oc=5) == INVALID  # 3 rows in steps of 2 overrun the column stride 5
    # strides of NULL operands and along extents of 1 are ignored (each call
    # still fails at a later check, so nothing is launched)
    assert call(k=None, ks=-5, orr=3) == INVALID and "map two positions" in tk.last_error()
    assert call(B=1, xr=-3, orr=0, oc=0) == INVALID and "out_col_stride" in tk.last_error()
    assert call(V=1, xc=-3, oc=0, orr=0) == INVALID and "out_row_stride" in tk.last_error()
    # the span of out, [out, out + 64), reaches the span of logits
    assert call(x=out + 32, xr=1, xc=4, orr=1, oc=2) == INVALID and "overlap" in tk.last_error()
    # p with stride 0 (one value for every row) sitting inside out
    assert call(p=out + 4, ps=0) == INVALID and "overlap" in tk.last_error()
    assert call(B=0, x=None, o=None, p=None) == 0  # empty


def test_sample_entry_point_checks(lib):
    f = lib.sample_top_k_top_p
    sel = FAKE + (1 << 36)
    assert f(None, 0, 2, 8, None, None, None, None, 0.0, None, sel, None) == NULLPTR
    assert "logits" in tk.last_error()
    assert f(FAKE, 0, 2, 8, None, None, None, None, 0.0, None, None, None) == NULLPTR
    assert "selected" in tk.last_error()
    assert f(FAKE, 4, 2, 8, None, None, None, None, 0.0, None, sel, None) == INVALID
    assert f(FAKE, 0, 2, 8, None, None, None, None, -1.0, None, sel, None) == INVALID
    assert "eps" in tk.last_error()
    assert f(FAKE, 0, 2, 8, None, None, None, None, float("nan"), None, sel, None) == INVALID
    assert f(FAKE, 0, 2, 8, None, None, None, None, 0.0, None, FAKE + 8, None) == INVALID  # selected inside logits
    assert "overlap" in tk.last_error()
    assert f(None, 1, 0, 8, None, None, None, None, 0.0, None, None, None) == 0  # empty


def test_survivors_entry_point_checks(lib):
    f = lib.top_k_top_p_sorted_survivors
    o1, o2, o3 = FAKE + (1 << 36), FAKE + (1 << 37), FAKE + (1 << 38)
    assert f(FAKE, 0, 2, 8, None, None, None, 4, o1, None, o3, None) == NULLPTR
    assert "indices" in tk.last_error()
    assert f(FAKE, 0, 2, 8, None, None, None, 4, o1, o2, None, None) == NULLPTR
    assert f(FAKE, 0, 2, 8, None, None, None, 0, o1, o2, o3, None) == INVALID
    assert "cap" in tk.last_error()
    assert f(FAKE, 0, 2, 8, None, None, None, 4, o1, o1 + 8, o3, None) == INVALID  # probs and indices overlap
    assert f(FAKE, 0, 2, 8, None, None, None, 4, None, FAKE + 4, o3, None) == INVALID  # indices inside logits
    assert f(None, 1, 0, 8, None, None, None, 4, None, None, None, None) == 0


def test_build_rejects_spilling_kernels():
    """The build reads the compiler's resource report and fails on any kernel
    that uses scratch (a register spill)."""
    from top_logits_filtering_amd.build import _spills

    report = "\n".join([
        "a.hip:1:1: remark: Function Name: _ZN3tkp4goodE [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     VGPRs: 64 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark: Function Name: _ZN3tkp5spillE [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert _spills(report) == [("_ZN3tkp5spillE", 12)]
    assert _spills(report.replace(": 12 ", ": 0 ")) == []


def test_binding_view_routing():
    """Which views the binding passes to the row-strided entry points (rows
    contiguous and disjoint) and which to the element-strided one; tensor
    metadata only, so CPU tensors serve."""
    import torch

    from top_logits_filtering_amd.binding import _rows_contiguous

    base = torch.zeros(6, 40)
    assert _rows_contiguous(base)
    assert _rows_contiguous(base[:, :33])  # padded rows
    assert not _rows_contiguous(torch.zeros(40, 6).t())  # transposed
    assert not _rows_contiguous(base[:, ::2])  # every second column
    assert not _rows_contiguous(base.flatten().as_strided((6, 20), (10, 1)))  # rows share elements
    assert _rows_contiguous(torch.zeros(40, 1).t())  # one row: its stride plays no part
    assert _rows_contiguous(torch.zeros(6, 1)[:, :1])  # one column


def test_binding_rejects_mismatched_operands():
    """The binding checks every operand's dtype and shape against the logits
    before anything reaches the library (a short p or a narrower out would
    otherwise be read or written past its end), then that all live on the
    GPU; tensor metadata only, so CPU tensors serve."""
    import pytest
    import torch

    import top_logits_filtering_amd as tk

    B, V = 3, 10
    x = torch.zeros(B, V, dtype=torch.bfloat16)
    p = torch.full((B,), 0.9, dtype=torch.bfloat16)
    k = torch.ones(B, dtype=torch.int32)
    bad = [
        (TypeError, dict(p=p.float())),
        (ValueError, dict(p=torch.ones(B + 1, dtype=torch.bfloat16))),
        (TypeError, dict(k=k.long())),
        (ValueError, dict(k=torch.ones(B, 1, dtype=torch.int32))),
        (TypeError, dict(min_p=p.half())),
        (TypeError, dict(out=torch.zeros(B, V, dtype=torch.float16))),
        (ValueError, dict(out=torch.zeros(B, V + 1, dtype=torch.bfloat16))),
    ]
    for err, kw in bad:
        args = dict(p=p, k=k)
        args.update(kw)
        with pytest.raises(err):
            tk.apply_top_k_top_p(x, **args)
    with pytest.raises(ValueError, match="GPU"):
        tk.apply_top_k_top_p(x, p, k)

    idx = torch.zeros(B, V, dtype=torch.int32)
    with pytest.raises(TypeError):
        tk.apply_top_k_top_p_with_sorted(x, idx.long(), p, k)
    with pytest.raises(TypeError):
        tk.apply_top_k_top_p_with_sorted(x, idx, p, k, logits=x.half())
    with pytest.raises(ValueError):
        tk.apply_top_k_top_p_with_sorted(x, idx[:, :5], p, k)

    with pytest.raises(TypeError):
        tk.sample_top_k_top_p(x, p, k, selected=torch.zeros(B, dtype=torch.int64))
    with pytest.raises(TypeError):
        tk.sample_top_k_top_p(x, p, k, out=torch.zeros(B, V, dtype=torch.float32))
    with pytest.raises(ValueError):
        tk.sample_top_k_top_p(x, p[:2], k)

    cap = 4
    good = (torch.zeros(B, cap), torch.zeros(B, cap, dtype=torch.int32), torch.zeros(B, dtype=torch.int32))
    with pytest.raises(TypeError):
        tk.top_k_top_p_sorted_survivors(x, p, k, cap=cap, out=(good[0].double(), good[1], good[2]))
    with pytest.raises(ValueError):
        tk.top_k_top_p_sorted_survivors(x, p, k, cap=cap, out=(good[0], good[1], good[2][:2]))
    with pytest.raises(ValueError, match="GPU"):
        tk.top_k_top_p_sorted_survivors(x, p, k, cap=cap, out=good)
