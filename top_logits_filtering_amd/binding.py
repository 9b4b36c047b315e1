"""ctypes binding of libtopktopp (include/topktopp.h).

Argument marshalling only: tensors are turned into device pointers and the
current HIP stream, and every step of the filter runs in the library's HIP
kernels. If the library has not been built this module raises instead of
falling back to anything else.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libtopktopp.so")

TOPKTOPP_F32, TOPKTOPP_F16, TOPKTOPP_BF16 = 0, 1, 2
STATUS_NAMES = {0: "OK", 1: "ERR_NULLPTR", 2: "ERR_INVALID", 3: "ERR_RUNTIME"}
EXPORTED_SYMBOLS = (
    "apply_top_k_top_p",
    "apply_top_k_top_p_ex",
    "apply_top_k_top_p_min_p",
    "apply_top_k_top_p_min_p_with_sorted",
    "apply_top_k_top_p_strided",
    "apply_top_k_top_p_with_sorted",
    "apply_top_k_top_p_with_sorted_ex",
    "sample_top_k_top_p",
    "top_k_top_p_sorted_survivors",
    "topktopp_last_error",
    "topktopp_set_plan_policy",
)

_lib = None


class TopKTopPError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libtopktopp.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build it first (python -m top_logits_filtering_amd.build); "
            "there is no fallback implementation"
        )
    lib = ctypes.CDLL(p)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.apply_top_k_top_p.argtypes = [vp, i32, i64, i64, vp, vp, vp, vp]
    lib.apply_top_k_top_p.restype = i32
    lib.apply_top_k_top_p_with_sorted.argtypes = [vp, vp, i32, i64, i64, vp, vp, vp, vp, vp]
    lib.apply_top_k_top_p_with_sorted.restype = i32
    lib.apply_top_k_top_p_min_p.argtypes = [vp, i32, i64, i64, vp, vp, vp, vp, vp]
    lib.apply_top_k_top_p_min_p.restype = i32
    lib.apply_top_k_top_p_min_p_with_sorted.argtypes = [vp, vp, i32, i64, i64, vp, vp, vp, vp, vp, vp]
    lib.apply_top_k_top_p_min_p_with_sorted.restype = i32
    lib.apply_top_k_top_p_ex.argtypes = [vp, i64, i32, i64, i64, vp, vp, vp, vp, i64, vp]
    lib.apply_top_k_top_p_ex.restype = i32
    lib.apply_top_k_top_p_with_sorted_ex.argtypes = [vp, i64, vp, i64, i32, i64, i64, vp, vp, vp, vp, i64, vp, i64, vp]
    lib.apply_top_k_top_p_with_sorted_ex.restype = i32
    lib.apply_top_k_top_p_strided.argtypes = [vp, i64, i64, i32, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, i64, vp]
    lib.apply_top_k_top_p_strided.restype = i32
    lib.sample_top_k_top_p.argtypes = [vp, i32, i64, i64, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp]
    lib.sample_top_k_top_p.restype = i32
    lib.top_k_top_p_sorted_survivors.argtypes = [vp, i32, i64, i64, vp, vp, vp, i64, vp, vp, vp, vp]
    lib.top_k_top_p_sorted_survivors.restype = i32
    lib.topktopp_last_error.argtypes = []
    lib.topktopp_last_error.restype = ctypes.c_char_p
    lib.topktopp_set_plan_policy.argtypes = [i32]
    lib.topktopp_set_plan_policy.restype = i32
    if path is None:
        _lib = lib
    return lib


def last_error() -> str:
    return load_library().topktopp_last_error().decode()


def set_plan_policy(policy: int) -> int:
    """0 auto (candidate plan), 1 multi-pass plan, 2 candidate plan re-reading global memory."""
    prev = load_library().topktopp_set_plan_policy(int(policy))
    if prev < 0:
        raise ValueError(f"unknown plan policy {policy}")
    return prev


_DTYPE_CODES = None


def _dtype_code(t) -> int:
    global _DTYPE_CODES
    if _DTYPE_CODES is None:
        import torch

        _DTYPE_CODES = {torch.float32: TOPKTOPP_F32, torch.float16: TOPKTOPP_F16, torch.bfloat16: TOPKTOPP_BF16}
    code = _DTYPE_CODES.get(t.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return code


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _rows(t):
    """(pointer, row stride in elements) of a 2-D tensor whose rows are
    contiguous; None for None."""
    if t is None:
        return None, 0
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if t.dim() != 2:
        raise ValueError("expected a 2-D [B, V] tensor")
    B, V = t.shape
    if V > 1 and t.stride(1) != 1:
        raise ValueError("rows must be contiguous (stride 1 along the last dimension)")
    ld = t.stride(0) if B > 1 else V
    return t.data_ptr(), ld


def _rows_contiguous(t) -> bool:
    """Rows contiguous and disjoint: a view the row-strided entry points take."""
    B, V = t.shape
    return (V <= 1 or t.stride(1) == 1) and (B <= 1 or t.stride(0) >= V)


def _entries(t, B):
    """(pointer, stride in elements) of a [B] parameter vector of any stride;
    (None, 0) for None."""
    if t is None:
        return None, 0
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if t.dim() != 1 or t.shape[0] != B:
        raise ValueError(f"expected a 1-D tensor of {B} entries, got shape {tuple(t.shape)}")
    return t.data_ptr(), t.stride(0)


def _check_vector(t, B, dtype, name):
    """A per-row parameter or output: None, or a 1-D tensor of B entries of `dtype`."""
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 1 or t.shape[0] != B:
        raise ValueError(f"{name} must be a 1-D tensor of {B} entries, got shape {tuple(t.shape)}")


def _check_matrix(t, shape, dtype, name):
    """None, or a 2-D tensor of `shape` and `dtype`."""
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2 or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be [{shape[0]}, {shape[1]}], got shape {tuple(t.shape)}")


def _check_params(B, dtype, p, k, min_p):
    """p and min_p [B] in the logits dtype, k [B] int32 (each optional)."""
    import torch

    _check_vector(p, B, dtype, "p")
    _check_vector(k, B, torch.int32, "k")
    _check_vector(min_p, B, dtype, "min_p")


def _check_device(device, *tensors):
    """Every given tensor on the GPU, on `device`."""
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if t.device != device:
            raise ValueError(f"tensors must share one device: {t.device} and {device}")


def _stream(stream, device) -> int:
    """The HIP stream handle to launch on: the given one, else torch's current
    stream of the tensors' device."""
    if stream is None:
        import torch

        return torch._C._cuda_getCurrentRawStream(device.index)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int):
    if status != 0:
        raise TopKTopPError(status, last_error())


def apply_top_k_top_p(logits, p=None, k=None, out=None, stream=None, min_p=None):
    """Filter raw logits [B, V]; p [B] (logits dtype), k [B] (int32) and min_p
    [B] (logits dtype, the min-p stage) are optional. Every operand may be a
    strided view: row-strided ones (rows contiguous, e.g. a slice of a padded
    vocabulary) take the vector kernels, any other view (a transpose, a
    column step, parameters with a stride) the element-wise strided kernel."""
    import torch

    lib = load_library()
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D [B, V]")
    B, V = logits.shape
    if out is None:
        out = torch.empty((B, V), dtype=logits.dtype, device=logits.device)
    _check_matrix(out, (B, V), logits.dtype, "out")
    _check_params(B, logits.dtype, p, k, min_p)
    _check_device(logits.device, logits, out, p, k, min_p)
    st = _stream(stream, logits.device)
    params = [t for t in (p, k, min_p) if t is not None]
    if not (_rows_contiguous(logits) and _rows_contiguous(out) and all(t.is_contiguous() for t in params)):
        if not (logits.is_cuda and out.is_cuda):
            raise ValueError("tensors must live on the GPU")
        (pp, ps), (kp, ks), (mp, ms) = _entries(p, B), _entries(k, B), _entries(min_p, B)
        status = lib.apply_top_k_top_p_strided(logits.data_ptr(), logits.stride(0), logits.stride(1),
                                               _dtype_code(logits), B, V, pp, ps, kp, ks, mp, ms, out.data_ptr(),
                                               out.stride(0), out.stride(1), st)
        _check(status)
        return out
    (xp, ldx), (op, ldo) = _rows(logits), _rows(out)
    if ldx != V or ldo != V:
        status = lib.apply_top_k_top_p_ex(xp, ldx, _dtype_code(logits), B, V, _ptr(p), _ptr(k), _ptr(min_p), op, ldo,
                                          st)
    elif min_p is None:
        status = lib.apply_top_k_top_p(xp, _dtype_code(logits), B, V, _ptr(p), _ptr(k), op, st)
    else:
        status = lib.apply_top_k_top_p_min_p(xp, _dtype_code(logits), B, V, _ptr(p), _ptr(k), _ptr(min_p), op, st)
    _check(status)
    return out


def apply_top_k_top_p_with_sorted(sorted_value, sorted_indices, p=None, k=None, logits=None, out=None,
                                  stream=None, min_p=None):
    """Filter pre-sorted rows (ascending sorted_value, int32 sorted_indices);
    min_p [B] (logits dtype) adds the min-p stage."""
    import torch

    lib = load_library()
    if sorted_value.dim() != 2:
        raise ValueError("sorted_value must be 2-D [B, V]")
    B, V = sorted_value.shape
    if out is None:
        out = torch.empty((B, V), dtype=sorted_value.dtype, device=sorted_value.device)
    _check_matrix(sorted_indices, (B, V), torch.int32, "sorted_indices")
    _check_matrix(logits, (B, V), sorted_value.dtype, "logits")
    _check_matrix(out, (B, V), sorted_value.dtype, "out")
    _check_params(B, sorted_value.dtype, p, k, min_p)
    _check_device(sorted_value.device, sorted_value, sorted_indices, logits, out, p, k, min_p)
    st = _stream(stream, sorted_value.device)
    (sp, lds), (ip, ldi), (xp, ldx), (op, ldo) = _rows(sorted_value), _rows(sorted_indices), _rows(logits), _rows(out)
    if lds != V or ldi != V or ldo != V or (logits is not None and ldx != V):
        status = lib.apply_top_k_top_p_with_sorted_ex(
            sp, lds, ip, ldi, _dtype_code(sorted_value), B, V, _ptr(p), _ptr(k), _ptr(min_p), xp, ldx, op, ldo, st
        )
    elif min_p is None:
        status = lib.apply_top_k_top_p_with_sorted(
            _ptr(sorted_value), _ptr(sorted_indices), _dtype_code(sorted_value), B, V, _ptr(p), _ptr(k),
            _ptr(logits), _ptr(out), st
        )
    else:
        status = lib.apply_top_k_top_p_min_p_with_sorted(
            _ptr(sorted_value), _ptr(sorted_indices), _dtype_code(sorted_value), B, V, _ptr(p), _ptr(k),
            _ptr(min_p), _ptr(logits), _ptr(out), st
        )
    _check(status)
    return out


def sample_top_k_top_p(logits, p=None, k=None, min_p=None, q=None, eps=0.0, out=None, selected=None, stream=None):
    """Filter logits [B, V] and pick one index per row (int32 [B], returned).

    q [B, V] float32 by descending survivor rank (QSample), or None (the
    argmax). out, if given, receives the filtered logits; otherwise the rows
    are only read."""
    import torch

    lib = load_library()
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D [B, V]")
    B, V = logits.shape
    if q is not None and (q.dtype != torch.float32 or tuple(q.shape) != (B, V)):
        raise ValueError("q must be float32 [B, V]")
    if selected is None:
        selected = torch.empty((B,), dtype=torch.int32, device=logits.device)
    _check_matrix(out, (B, V), logits.dtype, "out")
    _check_vector(selected, B, torch.int32, "selected")
    _check_params(B, logits.dtype, p, k, min_p)
    _check_device(logits.device, logits, p, k, min_p, q, out, selected)
    status = lib.sample_top_k_top_p(
        _ptr(logits), _dtype_code(logits), B, V, _ptr(p), _ptr(k), _ptr(min_p), _ptr(q), float(eps), _ptr(out),
        _ptr(selected), _stream(stream, logits.device)
    )
    _check(status)
    return selected


def top_k_top_p_sorted_survivors(logits, p=None, k=None, min_p=None, cap=1024, with_probs=True, stream=None,
                                 out=None):
    """The filter's survivors in descending order: (probs [B, cap] float32 or
    None, indices [B, cap] int32, counts [B] int32). Ranks past a row's
    survivors hold probability 0 and index -1. ``out`` may give the three
    buffers (probs may be None); they are then filled and returned."""
    import torch

    lib = load_library()
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D [B, V]")
    B, V = logits.shape
    dev = logits.device
    if out is not None:
        probs, indices, counts = out
        if (tuple(indices.shape) != (B, cap) or tuple(counts.shape) != (B,)
                or (probs is not None and tuple(probs.shape) != (B, cap))):
            raise ValueError("out buffers must be probs [B, cap], indices [B, cap], counts [B]")
    else:
        probs = torch.empty((B, cap), dtype=torch.float32, device=dev) if with_probs else None
        indices = torch.empty((B, cap), dtype=torch.int32, device=dev)
        counts = torch.empty((B,), dtype=torch.int32, device=dev)
    _check_matrix(probs, (B, cap), torch.float32, "probs")
    _check_matrix(indices, (B, cap), torch.int32, "indices")
    _check_vector(counts, B, torch.int32, "counts")
    _check_params(B, logits.dtype, p, k, min_p)
    _check_device(dev, logits, p, k, min_p, probs, indices, counts)
    status = lib.top_k_top_p_sorted_survivors(
        _ptr(logits), _dtype_code(logits), B, V, _ptr(p), _ptr(k), _ptr(min_p), int(cap), _ptr(probs), _ptr(indices),
        _ptr(counts), _stream(stream, dev)
    )
    _check(status)
    return probs, indices, counts
