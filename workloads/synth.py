"""Seeded synthetic workloads for the top-k / top-p logits filter.

Every array here is drawn from numpy's PCG64 generator seeded through
``numpy.random.SeedSequence``. Row ``b`` of workload ``c`` draws its values
from the entropy ``[seed_c, b]`` and the per-row parameters (k, p, spike
positions) from ``[seed_c, 2**32 - 1]``, so any subset of rows can be rebuilt
without drawing the rest. ``seed_c = 0x746F706B + c``.

Values are stored as raw bit patterns in the logits dtype:
``uint32`` for fp32, ``uint16`` for fp16 and bf16. p is stored in the logits
dtype as well, because the filter's parameter table gives p the dtype of the
logits (ApplyTopKTopPWithSorted page, section 3 parameter table). k is int32.

The five workloads mirror the shapes and value distributions the filter is
measured on: a small joint case, a 32k-vocab fp16 case with spikes and
disabled top-k rows, the 151936-vocab bf16 mixed-mode case, a 128256-vocab
fp32 tie-stress case, and a 262144-vocab bf16 pre-sorted case.

Nothing here computes any part of the filter.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

SEED_BASE = 0x746F706B
PARAM_STREAM = 2**32 - 1

DTYPES = ("f32", "f16", "bf16")


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16, nearest-even, and return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # finite values stay below 0xFF800000, so the uint32 sum cannot wrap
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored bit patterns to fp32 (input preparation only)."""
    if dtype == "f32":
        return np.ascontiguousarray(bits, dtype=np.uint32).view(np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def f32_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Store fp32 values in ``dtype``, rounding to nearest-even, as raw bits."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy().view(np.uint32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass
class Workload:
    """One batch of filter inputs, as raw bits in the logits dtype."""

    name: str
    entry: str  # "apply" or "with_sorted"
    dtype: str
    B: int
    V: int
    logits: np.ndarray  # [B, V] bits
    p: Optional[np.ndarray]  # [B] bits in dtype, or None
    k: Optional[np.ndarray]  # [B] int32, or None
    rows: np.ndarray  # global row numbers the arrays hold
    sorted_value: Optional[np.ndarray] = None  # [B, V] bits (with_sorted only)
    sorted_indices: Optional[np.ndarray] = None  # [B, V] int32 (with_sorted only)
    modes: Optional[np.ndarray] = None  # per row: 0 k only, 1 p only, 2 joint
    meta: dict = field(default_factory=dict)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


def _row_rng(seed: int, b: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, int(b)])))


def _param_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, PARAM_STREAM])))


WORKLOAD_SPECS = {
    1: dict(name="joint_fp32_B4_V1000", entry="apply", dtype="f32", B=4, V=1000),
    2: dict(name="spikes_fp16_B64_V32000", entry="apply", dtype="f16", B=64, V=32000),
    3: dict(name="mixed_bf16_B256_V151936", entry="apply", dtype="bf16", B=256, V=151936),
    4: dict(name="ties_fp32_B1024_V128256", entry="apply", dtype="f32", B=1024, V=128256),
    5: dict(name="sorted_bf16_B128_V262144", entry="with_sorted", dtype="bf16", B=128, V=262144),
}


def _row_values(c: int, seed: int, b: int, V: int, spikes: Optional[np.ndarray]) -> np.ndarray:
    rng = _row_rng(seed, b)
    if c == 1:
        return rng.normal(0.0, 2.0, V).astype(np.float32)
    if c == 2:
        x = rng.normal(0.0, 3.0, V)
        x[spikes] = 12.0
        return x.astype(np.float32)
    if c == 3:
        return (4.0 * rng.gumbel(0.0, 1.0, V)).astype(np.float32)
    if c == 4:
        # N(0, 2) snapped to multiples of 0.25 with round-half-even; rint keeps
        # the sign of values that round to zero, so -0.0 occurs next to +0.0.
        return (np.rint(rng.normal(0.0, 2.0, V) * 4.0) / 4.0).astype(np.float32)
    if c == 5:
        return rng.normal(0.0, 3.0, V).astype(np.float32)
    raise ValueError(c)


def make_workload(c: int, rows: Optional[Sequence[int]] = None, timed_modes: bool = True) -> Workload:
    """Build workload ``c`` (1..5), optionally only the listed rows.

    For workload 3 the rows cycle through three modes by ``b % 3``: 0 top-k
    only, 1 top-p only, 2 joint. With ``timed_modes`` both tensors are passed
    in one call, with k = 0 for top-p-only rows (k <= 0 disables top-k) and
    p = 1.0 for top-k-only rows (t = 1 - p = 0 masks only zero-probability
    positions). :func:`split_modes` rebuilds the same rows as three calls with
    truly absent p or k.
    """
    cfg = WORKLOAD_SPECS[c]
    B, V, dtype = cfg["B"], cfg["V"], cfg["dtype"]
    seed = SEED_BASE + c
    prng = _param_rng(seed)
    all_rows = np.arange(B)
    sel = all_rows if rows is None else np.asarray(list(rows), dtype=np.int64)

    spikes_all = None
    modes = None
    if c == 1:
        k = prng.integers(1, 50, size=B, endpoint=True)
        p = prng.uniform(0.5, 0.95, size=B)
    elif c == 2:
        off = prng.uniform(size=B) < 0.25
        off_val = prng.choice(np.array([0, V, V + 5]), size=B)
        k_on = prng.integers(1, 200, size=B, endpoint=True)
        k = np.where(off, off_val, k_on)
        p = prng.uniform(0.1, 1.0, size=B)
        spikes_all = [prng.choice(V, size=8, replace=False) for _ in range(B)]
    elif c == 3:
        k = prng.integers(1, 1024, size=B, endpoint=True)
        p = prng.uniform(0.8, 0.99, size=B)
        modes = all_rows % 3
        if timed_modes:
            k = np.where(modes == 1, 0, k)
            p = np.where(modes == 0, 1.0, p)
    elif c == 4:
        k = prng.integers(1, 1024, size=B, endpoint=True)
        p = prng.uniform(0.05, 0.95, size=B)
    elif c == 5:
        k = prng.integers(1, 4096, size=B, endpoint=True)
        p = prng.uniform(0.5, 0.99, size=B)
    else:
        raise ValueError(c)

    vals = np.empty((len(sel), V), dtype=np.float32)
    for i, b in enumerate(sel):
        vals[i] = _row_values(c, seed, int(b), V, None if spikes_all is None else spikes_all[b])
    logits = f32_to_bits(vals, dtype)
    del vals

    wl = Workload(
        name=cfg["name"],
        entry=cfg["entry"],
        dtype=dtype,
        B=len(sel),
        V=V,
        logits=logits,
        p=f32_to_bits(p[sel].astype(np.float32), dtype),
        k=k[sel].astype(np.int32),
        rows=sel,
        modes=None if modes is None else modes[sel],
        meta=dict(config=c, seed=seed),
    )
    if cfg["entry"] == "with_sorted":
        wl.sorted_indices, wl.sorted_value = stable_ascending_sort(logits, dtype)
    return wl


def stable_ascending_sort(logits_bits: np.ndarray, dtype: str):
    """Caller-side preparation of pre-sorted input: a stable ascending sort.

    Equal values (including -0.0 and +0.0, which compare equal) keep their
    original index order. Returns (sorted_indices int32, sorted_value bits).
    """
    x = bits_to_f32(logits_bits, dtype).reshape(logits_bits.shape)
    idx = np.argsort(x, axis=-1, kind="stable").astype(np.int32)
    sv = np.take_along_axis(logits_bits, idx.astype(np.int64), axis=-1)
    return idx, sv


def split_modes(wl: Workload):
    """Split a workload-3 batch into three calls with truly absent p or k.

    Returns a list of (row positions, p bits or None, k or None).
    """
    assert wl.modes is not None
    full = make_workload(wl.meta["config"], rows=wl.rows, timed_modes=False)
    out = []
    for mode in (0, 1, 2):
        pos = np.nonzero(wl.modes == mode)[0]
        if len(pos) == 0:
            continue
        p = None if mode == 0 else full.p[pos]
        k = None if mode == 1 else full.k[pos]
        out.append((pos, p, k))
    return out


def random_rows(
    seed: int,
    B: int,
    V: int,
    dtype: str,
    kind: str = "normal",
    scale: float = 2.0,
) -> np.ndarray:
    """Small random logits for tests, returned as bits in ``dtype``.

    kinds: ``normal`` N(0, scale); ``ties`` N(0, scale) snapped to multiples of
    0.5 (many equal values, both signs of zero); ``gumbel`` scale*Gumbel(0,1);
    ``const`` every value equal; ``zeros`` a random mix of +0.0 and -0.0;
    ``spikes`` normal plus a few positions set to the same large value;
    ``wide`` normal with a few very negative values and -inf entries.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([0x5EED, seed])))
    if kind == "normal":
        x = rng.normal(0.0, scale, (B, V))
    elif kind == "ties":
        x = np.rint(rng.normal(0.0, scale, (B, V)) * 2.0) / 2.0
    elif kind == "gumbel":
        x = scale * rng.gumbel(0.0, 1.0, (B, V))
    elif kind == "const":
        x = np.full((B, V), float(np.round(rng.normal(0.0, scale), 2)))
    elif kind == "zeros":
        x = np.where(rng.uniform(size=(B, V)) < 0.5, 0.0, -0.0)
    elif kind == "spikes":
        x = rng.normal(0.0, scale, (B, V))
        for b in range(B):
            pos = rng.choice(V, size=min(V, 4), replace=False)
            x[b, pos] = 6.0 * scale
    elif kind == "wide":
        x = rng.normal(0.0, scale, (B, V))
        for b in range(B):
            n = max(1, V // 16)
            pos = rng.choice(V, size=n, replace=False)
            x[b, pos[: n // 2]] = -np.inf
            x[b, pos[n // 2 :]] = -200.0 * scale
            x[b, rng.integers(V)] = 3.0 * scale  # keep a finite maximum
    else:
        raise ValueError(kind)
    return f32_to_bits(x.astype(np.float32), dtype)


def random_params(seed: int, B: int, V: int, dtype: str, k_lo: int = -2, k_hi: Optional[int] = None,
                  p_lo: float = 0.0, p_hi: float = 1.0):
    """Random per-row k (int32, may be out of range on purpose) and p bits."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([0xA11CE, seed])))
    k_hi = V + 2 if k_hi is None else k_hi
    k = rng.integers(k_lo, k_hi, size=B, endpoint=True).astype(np.int32)
    p = rng.uniform(p_lo, p_hi, size=B).astype(np.float32)
    return k, f32_to_bits(p, dtype)


# Seed stream of the min-p values (a stream of its own, so adding min-p to a
# workload leaves its logits, k and p unchanged).
MIN_P_STREAM = 2**32 - 2


def min_p_for_workload(c: int, B: int, dtype: str, lo: float = 0.01, hi: float = 0.2) -> np.ndarray:
    """Per-row min_p bits for workload c: uniform in [lo, hi], stored in the
    logits dtype like p (the typical range of min-p sampling settings)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_BASE + c, MIN_P_STREAM])))
    return f32_to_bits(rng.uniform(lo, hi, size=B).astype(np.float32), dtype)


def random_min_p(seed: int, B: int, dtype: str, specials: bool = True) -> np.ndarray:
    """Random per-row min_p bits: log-uniform in [1e-6, 1), with every 7th row
    set to a special value (0, negative, 1, above 1, or tiny) when asked."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([0x3199, seed])))
    v = np.exp(rng.uniform(np.log(1e-6), 0.0, size=B)).astype(np.float32)
    if specials:
        v[::7] = rng.choice(np.array([0.0, -0.5, 1.0, 2.0, 1e-30], np.float32), size=len(v[::7]))
    return f32_to_bits(v, dtype)
