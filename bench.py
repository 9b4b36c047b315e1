#!/usr/bin/env python3
"""Throughput of the top-k / top-p logits filter on one MI355X.

A step is one call of the filter over a whole batch of synthetic input; the
default batch is 256 rows of 151936 bf16 logits (4 * Gumbel(0,1)) with the
rows cycling through top-k only, top-p only and joint modes. Inputs are
resident in HBM before timing starts. Four input/output buffer sets are
rotated so the 256 MB Infinity Cache cannot hold the working set between
steps.

Prints one JSON line: rows/s (value), the dominant kernel's achieved HBM
bandwidth against the 8 TB/s peak (roofline), and the CPU oracle timed on a
bounded sample of the same rows (cpu_baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1..5] [--min-p]

--min-p adds the min-p stage (aclnnTopKTopPSampleV2, "minP sampling") with a
per-row min_p drawn uniformly from [0.01, 0.2] to the chosen workload.
--no-logits runs the pre-sorted workload without logits (the output is
scattered through sorted_indices). --p-only passes no k (top-p alone).
--sample runs the filter followed by sampling (aclnnTopKTopPSampleV2
"Subsequent processing", QSample with q drawn i.i.d. from Exp(1), eps 1e-6)
and writes one index per row instead of the filtered logits; --sample-none
uses the argmax mode instead. --survivors returns each row's survivors in
descending order with their probabilities and original indices (capacity
1024 per row) instead of the filtered logits. --wide-top-p P replaces the
rows by N(0,3) rows and runs top-p only with p = P: rows that keep thousands
of survivors, beyond the candidate list. --topk-only K runs top-k only with
k = K on every row.
"""

import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "rows/s and HBM GB/s (% roofline), top-k/top-p filter B=256 V=151936 bf16"
HBM_PEAK_GBS = 8000.0
TORCH_VIEW = {"f32": ("int32", "float32"), "f16": ("int16", "float16"), "bf16": ("int16", "bfloat16")}
WORKLOAD_TEXT = {
    1: "apply_top_k_top_p joint, B=4 V=1000 fp32 N(0,2)",
    2: "apply_top_k_top_p, B=64 V=32000 fp16 N(0,3)+8 spikes, k off w.p. 0.25",
    3: "apply_top_k_top_p mixed modes (k only / p only / joint by row), B=256 V=151936 bf16 4*Gumbel",
    4: "apply_top_k_top_p tie stress, B=1024 V=128256 fp32 N(0,2) snapped to 0.25",
    5: "apply_top_k_top_p_with_sorted with logits, B=128 V=262144 bf16 N(0,3)",
}


# HBM bytes per launch of the filter kernel on workload 3, from the FETCH_SIZE
# and WRITE_SIZE counter passes (scaled by a plain copy's readings), together
# with a digest of the kernel sources they were taken on.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_apply_regs_kernel_bf16_B256_V151936.md")


def kernel_source_digest():
    """sha256 over the code of the library's kernel sources and build script,
    with C/C++ comments and whitespace removed (a comment edit does not change
    the kernel)."""
    pkg = os.path.join(ROOT, "top_logits_filtering_amd")
    names = sorted(os.path.join("csrc", n) for n in os.listdir(os.path.join(pkg, "csrc"))) + ["build.py"]
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(pkg, n), "rb") as f:
            text = f.read()
        if not n.endswith(".py"):
            text = re.sub(rb"/\*.*?\*/", b"", text, flags=re.S)
            text = re.sub(rb"//[^\n]*", b"", text)
        h.update(n.encode() + b"\0" + b"".join(text.split()) + b"\0")
    return h.hexdigest()


def measured_traffic(args):
    """Counter-measured HBM bytes per launch, or None when no counters were
    taken for this workload or the kernel sources changed since."""
    if (args.workload != 3 or args.policy != 0 or args.copy_calibration or args.min_p or args.no_logits
            or args.p_only or args.wide_top_p is not None or args.topk_only is not None or args.sample
            or args.sample_none or args.survivors
            or not os.path.exists(TRAFFIC_PROFILE)):
        return None
    text = open(TRAFFIC_PROFILE).read()
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not (m_bytes and m_hash) or m_hash.group(1) != kernel_source_digest():
        return None
    return int(m_bytes.group(1))


def dev(bits, dtype):
    import torch

    if bits is None:
        return None
    iv, fv = TORCH_VIEW[dtype]
    return torch.from_numpy(np.ascontiguousarray(bits).view(getattr(np, iv))).cuda().view(getattr(torch, fv))


def sample_bytes(wl, with_min_p, survivors, with_q):
    """Minimal HBM bytes of one sampling call: read every logit once, read p
    and k (and min_p), read q at each row's survivor ranks, write one int32
    per row."""
    s = wl.elem_bytes
    return wl.B * (wl.V * s + s + 4 + (s if with_min_p else 0) + 4) + (4 * survivors if with_q else 0)


def survivor_bytes(wl, with_min_p, cap):
    """Minimal HBM bytes of one sorted-survivors call: read every logit once,
    read p and k (and min_p), write cap probabilities and indices and one
    count per row."""
    s = wl.elem_bytes
    return wl.B * (wl.V * s + s + 4 + (s if with_min_p else 0) + 8 * cap + 4)


def algorithmic_bytes(wl, with_min_p=False, with_logits=True, with_k=True):
    """Minimal HBM bytes of one call: read every logit once, write every output
    once, read p and k (and min_p); the pre-sorted entry also reads at least
    the k largest sorted values of each row (every sorted value without k:
    Z sums the whole row). Without logits the pre-sorted entry writes every
    output once and reads the survivors' values and indices, at least
    min(k, V) per row."""
    s = wl.elem_bytes
    kept = int(np.clip(wl.k, 0, wl.V).sum()) if with_k else wl.B * wl.V
    params = wl.B * (s + (4 if with_k else 0) + (s if with_min_p else 0))
    if wl.entry == "with_sorted" and not with_logits:
        return wl.B * wl.V * s + kept * (s + 4) + params
    total = 2 * wl.B * wl.V * s + params
    if wl.entry == "with_sorted":
        total += kept * s
    return total


# The CPU oracle job of this run, set before worker processes are forked.
_CPU_JOB = None


def _oracle_chunk(lo):
    """Runs the oracle, as it stands, on rows lo .. lo+7 of the workload (its
    sampling stage or sorted-survivors output too when the GPU computes
    them); returns the number of rows done."""
    from oracle import apply_top_k_top_p, apply_top_k_top_p_with_sorted, sample_top_k_top_p, sorted_survivors

    wl, min_p, sample_q, sample_none, survivors_cap = _CPU_JOB
    r = slice(lo, min(wl.B, lo + 8))
    mp = None if min_p is None else min_p[r]
    kk = None if wl.k is None else wl.k[r]
    if survivors_cap:
        sorted_survivors(wl.logits[r], wl.dtype, wl.p[r], kk, mp, survivors_cap)
    elif sample_q is not None or sample_none:
        sample_top_k_top_p(wl.logits[r], wl.dtype, wl.p[r], kk, mp,
                           None if sample_q is None else sample_q[r], 1e-6)
    elif wl.entry == "apply":
        apply_top_k_top_p(wl.logits[r], wl.dtype, wl.p[r], kk, keep_traces=False, min_p_bits=mp)
    else:
        apply_top_k_top_p_with_sorted(wl.sorted_value[r], wl.sorted_indices[r], wl.dtype, wl.p[r], kk,
                                      logits_bits=wl.logits[r], keep_traces=False, min_p_bits=mp)
    return r.stop - r.start


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s=12.0, min_p=None, sample_q=None, sample_none=False, survivors_cap=0):
    """The CPU oracle on one thread, over the workload's rows in order (8 at a
    time, wrapping), for about budget_s seconds. Also sets the job that
    cpu_baseline_parallel runs."""
    global _CPU_JOB
    _CPU_JOB = (wl, min_p, sample_q, sample_none, survivors_cap)
    done = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) < budget_s:
        done += _oracle_chunk(done % wl.B)
    dt = time.perf_counter() - t0
    return {
        "value": round(done / dt, 3),
        "unit": "rows/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done} rows (the workload's rows in order, wrapping after {wl.B}), the C++17 oracle "
                  f"(double-precision softmax, std::stable_sort ranking), one thread, {dt:.1f} s",
        "cpu": cpu_model(),
    }


def cpu_baseline_parallel(wl, rate1, budget_s=12.0):
    """The same oracle job on every host core (at most 16: one GPU's share of
    the host), one process per core over disjoint 8-row chunks, sized from the
    one-thread rate to take about budget_s seconds. Must run before the GPU is
    initialised: the workers are forked from this process."""
    import multiprocessing as mp

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))
    chunks = max(cores, int(rate1 * cores * budget_s / 8))
    starts = [(8 * i) % wl.B for i in range(chunks)]
    ctx = mp.get_context("fork")
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_chunk, starts[:cores])  # workers imported and warm
        t0 = time.perf_counter()
        done = sum(pool.map(_oracle_chunk, starts, chunksize=1))
        dt = time.perf_counter() - t0
    return {
        "value": round(done / dt, 3),
        "unit": "rows/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{done} rows in 8-row chunks over {cores} worker processes (one per core), the same C++17 "
                  f"oracle, {dt:.1f} s",
        "cpu": cpu_model(),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--sets", type=int, default=4, help="rotating input/output buffer sets")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds for the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--policy", type=int, default=0, help="plan policy: 0 auto, 1 general, 2 registers")
    ap.add_argument("--min-p", action="store_true", help="add a per-row min_p in [0.01, 0.2] (the min-p stage)")
    ap.add_argument("--no-logits", action="store_true", help="pre-sorted workload without logits (scattered output)")
    ap.add_argument("--p-only", action="store_true",
                    help="top-p only: the workload's p with k absent (NULL), e.g. the pre-sorted top-p batch")
    ap.add_argument("--wide-top-p", type=float, default=None, metavar="P",
                    help="the workload's rows replaced by N(0,3) rows (thousands of top-p survivors each), top-p "
                         "only with p = P on every row: the rows that overflow the candidate list")
    ap.add_argument("--topk-only", type=int, default=None, metavar="K",
                    help="top-k only with k = K on every row (p = 1): large k shows where the candidate bound "
                         "stops and the multi-pass plan takes over")
    ap.add_argument("--sample", action="store_true", help="filter then sample one index per row (QSample)")
    ap.add_argument("--sample-none", action="store_true", help="filter then take the argmax index per row")
    ap.add_argument("--survivors", action="store_true",
                    help="sorted survivors (probabilities, indices, counts; capacity 1024) instead of the filtered row")
    ap.add_argument("--warm", action="store_true",
                    help="also time back-to-back calls on one buffer set (warm caches), reported apart")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain device-to-device copy of the logits instead of the filter (the reference "
                         "kernel whose HBM counters scale the filter's)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this filter is row-parallel and is built and measured on a "
              "single MI355X; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    from workloads.synth import f32_to_bits, make_workload, min_p_for_workload, random_rows

    wl = make_workload(args.workload)
    dt = wl.dtype
    if args.wide_top_p is not None:
        if wl.entry != "apply":
            print("--wide-top-p applies to the raw-logits workloads (1-4)", file=sys.stderr)
            sys.exit(2)
        wl.logits = random_rows(0x71DE, wl.B, wl.V, dt, kind="normal", scale=3.0)
        wl.p = f32_to_bits(np.full(wl.B, args.wide_top_p, np.float32), dt)
        wl.k = None
    if args.p_only:
        wl.k = None
    if args.topk_only is not None:  # p = 1 on every row: no top-p
        wl.k = np.full(wl.B, args.topk_only, np.int32)
        wl.p = f32_to_bits(np.ones(wl.B, np.float32), dt)
    mp_bits = min_p_for_workload(args.workload, wl.B, dt) if args.min_p else None
    sampling = args.sample or args.sample_none
    if (sampling or args.survivors) and wl.entry != "apply":
        print("--sample and --survivors apply to the raw-logits workloads (1-4)", file=sys.stderr)
        sys.exit(2)
    cap = 1024
    q_host = None
    if args.sample:
        rng = np.random.default_rng(0x5A4D)
        q_host = rng.exponential(1.0, size=(wl.B, wl.V)).astype(np.float32)

    # The CPU oracle first, before anything touches the GPU (its parallel leg
    # forks worker processes).
    baselines = None
    if not (args.copy_calibration or args.no_cpu_baseline):
        one = cpu_baseline(wl, args.cpu_budget, mp_bits, None if q_host is None else q_host.astype(np.float64),
                           args.sample_none, cap if args.survivors else 0)
        baselines = (one, cpu_baseline_parallel(wl, one["value"], args.cpu_budget))

    import torch

    import top_logits_filtering_amd as tk

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    tk.load_library()
    tk.set_plan_policy(args.policy)
    p = dev(wl.p, dt)
    k = None if wl.k is None else torch.from_numpy(wl.k).cuda()
    mp = dev(mp_bits, dt)
    surv_out = None
    if args.survivors:
        surv_out = (torch.empty((wl.B, cap), dtype=torch.float32, device="cuda"),
                    torch.empty((wl.B, cap), dtype=torch.int32, device="cuda"),
                    torch.empty((wl.B,), dtype=torch.int32, device="cuda"))
    q = None
    if args.sample:
        q = torch.from_numpy(q_host).cuda()
    selected = torch.empty((wl.B,), dtype=torch.int32, device="cuda")
    sets = []
    for _ in range(max(1, args.sets)):
        if wl.entry == "apply":
            x = dev(wl.logits, dt)
            sets.append((x, torch.empty_like(x)))
        else:
            x = dev(wl.logits, dt)
            sets.append((x, torch.empty_like(x), dev(wl.sorted_value, dt),
                         torch.from_numpy(wl.sorted_indices).cuda()))

    def step(i):
        st = sets[i % len(sets)]
        if args.copy_calibration:
            st[1].copy_(st[0])
        elif sampling:
            tk.sample_top_k_top_p(st[0], p, k, mp, q, 1e-6, out=None, selected=selected)
        elif args.survivors:
            tk.top_k_top_p_sorted_survivors(st[0], p, k, mp, cap=cap, out=surv_out)
        elif wl.entry == "apply":
            tk.apply_top_k_top_p(st[0], p, k, out=st[1], min_p=mp)
        else:
            tk.apply_top_k_top_p_with_sorted(st[2], st[3], p, k, logits=None if args.no_logits else st[0], out=st[1],
                                             min_p=mp)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The library launches on torch's current stream; the two events bracket
    # the K launches on that same stream.
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kernel_ms = ev0.elapsed_time(ev1) / args.steps

    # Outside the timed region: each call between its own pair of events
    # (rotating buffer sets), for the latency spread of a single call; with
    # --warm also back-to-back calls on one buffer set (inputs partly cached).
    n_single = 50
    singles = []
    for i in range(n_single):
        a = torch.cuda.Event(enable_timing=True)
        z = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step(i)
        z.record(stream)
        z.synchronize()
        singles.append(a.elapsed_time(z) * 1e3)
    torch.cuda.synchronize()
    warm_us = None
    if args.warm:
        wa = torch.cuda.Event(enable_timing=True)
        wz = torch.cuda.Event(enable_timing=True)
        wa.record(stream)
        for _ in range(n_single):
            step(0)
        wz.record(stream)
        torch.cuda.synchronize()
        warm_us = round(wa.elapsed_time(wz) * 1e3 / n_single, 3)
    p10, p50, p90 = np.percentile(np.array(singles), [10, 50, 90])
    if args.copy_calibration:
        nbytes = 2 * wl.B * wl.V * wl.elem_bytes
    elif sampling:
        survivors = 0
        if args.sample:  # q is read at each survivor's rank: count the survivors once (outside the timing)
            ref = torch.empty_like(sets[0][0])
            tk.apply_top_k_top_p(sets[0][0], p, k, out=ref, min_p=mp)
            survivors = int((ref.float() != float("-inf")).sum().item())
        nbytes = sample_bytes(wl, args.min_p, survivors, args.sample)
    elif args.survivors:
        nbytes = survivor_bytes(wl, args.min_p, cap)
    else:
        nbytes = algorithmic_bytes(wl, args.min_p, not args.no_logits, wl.k is not None)
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    rows_per_s = wl.B / (ms_per_step * 1e-3)

    line = {
        "metric": METRIC,
        "value": round(rows_per_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {
            "workload": (WORKLOAD_TEXT[args.workload] if args.wide_top_p is None else
                         f"apply_top_k_top_p, B={wl.B} V={wl.V} {dt} N(0,3) (thousands of top-p survivors per row)")
                        + (", min-p U[0.01,0.2] per row" if args.min_p else "")
                        + (", without logits" if args.no_logits and wl.entry == "with_sorted" else "")
                        + (", top-p only (k absent)" if args.p_only else "")
                        + (f", top-p only with p = {args.wide_top_p} on every row" if args.wide_top_p is not None else "")
                        + (f", top-k only with k = {args.topk_only} on every row" if args.topk_only is not None else "")
                        + (", then QSample (q ~ Exp(1), eps 1e-6), one index per row" if args.sample else "")
                        + (", then argmax, one index per row" if args.sample_none else "")
                        + (", sorted survivors (probabilities and indices, capacity 1024 per row)"
                           if args.survivors else ""),
            "B": wl.B,
            "V": wl.V,
            "buffer_sets": len(sets),
            "plan_policy": args.policy,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(args),
            "kernel_us": round(kernel_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": nbytes,
        },
    }
    line["latency"] = {
        "per_call_us": {"p10": round(float(p10), 3), "median": round(float(p50), 3), "p90": round(float(p90), 3),
                        "calls": n_single},
        "warm_same_buffer_us": warm_us,
        "note": "per_call_us: one call between its own events, rotating buffer sets; warm_same_buffer_us "
                "(--warm): back-to-back calls on one buffer set, inputs partly cached; both outside the timed region",
    }
    if args.copy_calibration:
        line["metric"] = "device copy of the logits (HBM counter calibration)"
        line["value"] = round(nbytes / (ms_per_step * 1e-3) / 1e9, 1)
        line["unit"] = "GB/s"
        line["config"]["workload"] = "torch copy_ of " + WORKLOAD_TEXT[args.workload]
    elif baselines is not None:
        line["cpu_baseline"], line["cpu_baseline_parallel"] = baselines
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
