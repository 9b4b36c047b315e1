"""Whole-batch oracle comparisons in worker processes.

The GPU tests run a full workload batch through the library once, save the
outputs to .npy files, and hand row chunks to a pool of worker processes.
Each worker rebuilds its rows of the seeded workload (make_workload draws
every row from its own seed), runs the CPU oracle on them and applies the
comparison rule of tests/parity.py to the saved GPU rows. Only small
reports travel back. Workers are started with "spawn": they never touch the
GPU, and they do not inherit the parent's HIP state.

A job is a dict:
  kind      "apply", "sorted", "sample" or "survivors"
  config    workload number (1..5)
  lo, hi    row range
  outs      {label: path of the saved GPU output(s)}
  min_p     True: the workload's min-p column (min_p_for_workload)
  logits    "sorted" only: whether logits were passed
  q         "sample" only: path of the saved q matrix, or None (argmax)
  cap       "survivors" only
  no_k      True: the call passed no k
"""

from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

EPS = 1e-6


def pool_size() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _inputs(job):
    from workloads.synth import make_workload, min_p_for_workload

    wl = make_workload(job["config"], rows=range(job["lo"], job["hi"]))
    mp_bits = None
    if job.get("min_p"):
        mp_bits = min_p_for_workload(job["config"], job["B"], wl.dtype)[job["lo"]:job["hi"]]
    return wl, mp_bits


def run_job(job):
    """One row chunk: the oracle and the comparison rule. Returns
    {label: summary dict} (plus the R5 count for apply jobs that ask)."""
    from oracle import apply_top_k_top_p, apply_top_k_top_p_with_sorted, sample_top_k_top_p, sorted_survivors
    from tests.parity import compare, compare_samples, compare_survivors

    wl, mp_bits = _inputs(job)
    if job.get("no_k"):
        wl.k = None
    lo, hi = job["lo"], job["hi"]
    res = {}
    if job["kind"] in ("apply", "sorted"):
        if job["kind"] == "apply":
            ref = apply_top_k_top_p(wl.logits, wl.dtype, wl.p, wl.k, min_p_bits=mp_bits)
        else:
            ref = apply_top_k_top_p_with_sorted(wl.sorted_value, wl.sorted_indices, wl.dtype, wl.p, wl.k,
                                                logits_bits=wl.logits, min_p_bits=mp_bits)
        for label, path in job["outs"].items():
            g = np.load(path, mmap_mode="r")[lo:hi]
            rep = compare(np.asarray(g), wl.logits, ref, wl.dtype, row_ids=wl.rows)
            res[label] = rep.summary()
        if job.get("r5"):
            # rows whose output changes when 1 - p is rounded to p's dtype
            alt = apply_top_k_top_p(wl.logits, wl.dtype, wl.p, wl.k, keep_traces=False, t_reading="dtype",
                                    min_p_bits=mp_bits).out
            res["r5_rows_changed"] = int((alt != ref.out).any(axis=1).sum())
            res["r5_positions_changed"] = int((alt != ref.out).sum())
    elif job["kind"] == "sample":
        q = None
        if job["q"] is not None:
            q = np.asarray(np.load(job["q"], mmap_mode="r")[lo:hi], dtype=np.float64)
        ref = sample_top_k_top_p(wl.logits, wl.dtype, wl.p, wl.k, mp_bits, q, EPS)
        for label, path in job["outs"].items():
            g = np.asarray(np.load(path, mmap_mode="r")[lo:hi])
            hard, soft, det = compare_samples(g, ref)
            res[label] = dict(rows=hi - lo, hard_mismatches=hard, near_tie_picks=soft,
                              details=[dict(d, row=d["row"] + lo) for d in det[:3]])
    elif job["kind"] == "survivors":
        ref = sorted_survivors(wl.logits, wl.dtype, wl.p, wl.k, mp_bits, job["cap"])
        for label, (pp, ip, cp) in job["outs"].items():
            gp = None if pp is None else np.asarray(np.load(pp, mmap_mode="r")[lo:hi], dtype=np.float64)
            gi = np.asarray(np.load(ip, mmap_mode="r")[lo:hi])
            gc = np.asarray(np.load(cp, mmap_mode="r")[lo:hi])
            hard, det = compare_survivors(gp, gi, gc, ref)
            res[label] = dict(rows=hi - lo, hard_mismatches=hard,
                              details=[dict(d, row=d["row"] + lo) for d in det[:3]])
    else:
        raise ValueError(job["kind"])
    return res


def _merge(parts):
    """Sum the per-chunk summaries of each label."""
    out = {}
    for part in parts:
        for label, s in part.items():
            if not isinstance(s, dict):
                out[label] = out.get(label, 0) + s
                continue
            acc = out.setdefault(label, {})
            for key, v in s.items():
                if key == "details":
                    acc.setdefault("details", []).extend(v)
                else:
                    acc[key] = acc.get(key, 0) + v
    for s in out.values():
        if isinstance(s, dict) and "details" in s:
            s["details"] = s["details"][:5]
    return out


def run_batch(base_job, B, rows_per_job, timeout_s=600.0):
    """Runs base_job over rows [0, B) in chunks on the worker pool; returns
    the merged summaries. A worker that dies raises BrokenProcessPool, and a
    batch that takes longer than timeout_s raises TimeoutError."""
    jobs = [dict(base_job, lo=lo, hi=min(B, lo + rows_per_job), B=B) for lo in range(0, B, rows_per_job)]
    with ProcessPoolExecutor(max_workers=min(pool_size(), len(jobs)), mp_context=mp.get_context("spawn")) as ex:
        parts = list(ex.map(run_job, jobs, timeout=timeout_s))
    return _merge(parts)
