"""Helpers for GPU tests: move raw bit arrays to device tensors and back, and
call the library through its binding (the C ABI)."""

from __future__ import annotations

import sys

import numpy as np

TORCH_VIEW = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def need_gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import top_logits_filtering_amd as tk

    tk.load_library()  # raises if libtopktopp.so is missing: no fallback
    return torch


def to_dev(bits, dtype):
    import torch

    if bits is None:
        return None
    bits = np.ascontiguousarray(bits)
    if dtype == "f32":
        t = torch.from_numpy(bits.view(np.int32))
    else:
        t = torch.from_numpy(bits.view(np.int16))
    return t.cuda().view(getattr(torch, TORCH_VIEW[dtype]))


def k_dev(k):
    import torch

    return None if k is None else torch.from_numpy(np.ascontiguousarray(k, dtype=np.int32)).cuda()


def from_dev(t, dtype):
    import torch

    if dtype == "f32":
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def gpu_apply(bits, dtype, p=None, k=None, min_p=None):
    import torch
    import top_logits_filtering_amd as tk

    x = to_dev(bits, dtype)
    out = tk.apply_top_k_top_p(x, to_dev(p, dtype), k_dev(k), min_p=to_dev(min_p, dtype))
    torch.cuda.synchronize()
    return from_dev(out, dtype)


def gpu_with_sorted(sv, si, dtype, p=None, k=None, logits=None, min_p=None):
    import torch
    import top_logits_filtering_amd as tk

    out = tk.apply_top_k_top_p_with_sorted(
        to_dev(sv, dtype), k_dev(si), to_dev(p, dtype), k_dev(k), to_dev(logits, dtype), min_p=to_dev(min_p, dtype)
    )
    torch.cuda.synchronize()
    return from_dev(out, dtype)


# NaN patterns the filter never writes: they mark padding that must stay untouched
SENTINEL = {"f32": 0x7FC00001, "f16": 0x7E01, "bf16": 0x7FC1}


def padded_dev(bits, dtype, ld, fill):
    """A [B, ld] device buffer holding bits in its first V columns (fill in
    the rest), and its [B, V] row-strided view."""
    B, V = bits.shape
    full = np.full((B, ld), fill, dtype=bits.dtype)
    full[:, :V] = bits
    t = to_dev(full, dtype)
    return t, t[:, :V]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
