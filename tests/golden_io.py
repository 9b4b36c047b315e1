"""Reader for the hand-derived cases in tests/golden/hand_cases.txt."""

from __future__ import annotations

import os
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from workloads.synth import f32_to_bits

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NEG_INF_WORD = {"f32": 0xFF800000, "f16": 0xFC00, "bf16": 0xFF80}


@dataclass
class HandCase:
    name: str
    dtype: str
    x: np.ndarray  # bits [B, V]
    p: Optional[np.ndarray]  # bits [B]
    k: Optional[np.ndarray]  # int32 [B]
    expect: np.ndarray  # bits [B, V]
    min_p: Optional[np.ndarray] = None  # bits [B], cases of min_p_cases.txt and sample_cases.txt
    q: Optional[np.ndarray] = None  # float64 [B, V] by descending rank (sample_cases.txt)
    eps: float = 0.0
    expect_idx: Optional[np.ndarray] = None  # int64 [B] (sample_cases.txt) or [B, cap] (survivor_cases.txt)
    cap: int = 0
    expect_probs: Optional[np.ndarray] = None  # float64 [B, cap] (survivor_cases.txt)
    expect_count: Optional[np.ndarray] = None  # int64 [B] (survivor_cases.txt)


def _parse_values(tokens, dtype):
    vals = []
    for t in tokens:
        if t == "-inf":
            vals.append(-np.inf)
        elif t == "-0":
            vals.append(-0.0)
        else:
            vals.append(float(t))
    return f32_to_bits(np.array(vals, dtype=np.float32), dtype)


def load_hand_cases(path: Optional[str] = None) -> List[HandCase]:
    path = path if path is None or os.path.isabs(path) else os.path.join(GOLDEN_DIR, path)
    path = path or os.path.join(GOLDEN_DIR, "hand_cases.txt")
    cases = []
    cur = None
    with open(path) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            head, *rest = line.split()
            if head == "case":
                cur = dict(name=rest[0], dtype=rest[1], x=[], p=None, k=None, min_p=None, expect=[], q=[],
                           eps=0.0, expect_idx=None, cap=0, idx_rows=[], prob_rows=[], counts=[])
                cases.append(cur)
            elif head == "x":
                cur["x"].append(_parse_values(rest, cur["dtype"]))
            elif head == "expect":
                cur["expect"].append(_parse_values(rest, cur["dtype"]))
            elif head == "p":
                cur["p"] = None if rest == ["none"] else _parse_values(rest, cur["dtype"])
            elif head == "q":
                if rest != ["none"]:
                    cur["q"].append(np.array([float(v) for v in rest], dtype=np.float64))
            elif head == "eps":
                cur["eps"] = float(rest[0])
            elif head == "expect_idx":
                cur["expect_idx"] = np.array([int(v) for v in rest], dtype=np.int64)
                cur["idx_rows"].append(cur["expect_idx"])
            elif head == "cap":
                cur["cap"] = int(rest[0])
            elif head == "expect_probs":
                cur["prob_rows"].append(np.array([float(v) for v in rest], dtype=np.float64))
            elif head == "expect_count":
                cur["counts"].append(int(rest[0]))
            elif head == "min_p":
                cur["min_p"] = None if rest == ["none"] else _parse_values(rest, cur["dtype"])
            elif head == "k":
                cur["k"] = None if rest == ["none"] else np.array([int(v) for v in rest], dtype=np.int32)
            else:
                raise ValueError(f"bad golden line: {line}")
    return [
        HandCase(c["name"], c["dtype"], np.stack(c["x"]), c["p"], c["k"],
                 np.stack(c["expect"]) if c["expect"] else None, c["min_p"],
                 np.stack(c["q"]) if c["q"] else None, c["eps"],
                 np.stack(c["idx_rows"]) if c["cap"] else c["expect_idx"], c["cap"],
                 np.stack(c["prob_rows"]) if c["prob_rows"] else None,
                 np.array(c["counts"], dtype=np.int64) if c["counts"] else None)
        for c in cases
    ]
