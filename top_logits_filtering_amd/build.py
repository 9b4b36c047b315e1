"""Build libtopktopp.so in-tree with hipcc for gfx950.

Usage: ``python -m top_logits_filtering_amd.build`` (or ``build()`` from
Python). Every call recompiles every source. The library lands next to this
file as ``libtopktopp.so``; object files go to ``_build/``.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libtopktopp.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["api.cpp", "apply_f32.hip", "apply_f16.hip", "apply_bf16.hip", "sorted_kernels.hip", "util_kernels.hip"]

ARCH = "gfx950"
COMMON_FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no NaN handling in min/max (NaN inputs are outside the filter's contract)
    "-fno-honor-nans",
    "-I", os.path.join(REPO_ROOT, "include"),
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libtopktopp")
    return path


# Every kernel must fit its registers: a spill goes to scratch memory, whose
# accesses wait behind the row loads in flight. The compiler's resource report
# is read after each compile and any kernel with scratch fails the build.
RESOURCE_FLAG = "-Rpass-analysis=kernel-resource-usage"


def _spills(report: str) -> list:
    """(kernel, bytes per lane) for every kernel of a resource report that uses scratch."""
    found, name = [], None
    for line in report.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name is not None and int(m.group(1)) > 0:
            found.append((name, int(m.group(1))))
    return found


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, RESOURCE_FLAG, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "not a recognized feature for this target"
    lines = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    msg = "\n".join(l for l in lines if RESOURCE_FLAG not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    spills = _spills("\n".join(lines))
    if spills:
        raise RuntimeError(f"kernels in {src} spill registers to scratch: " +
                           ", ".join(f"{n} ({b} B/lane)" for n, b in spills))
    if verbose and msg.strip():
        print(msg, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libtopktopp.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 6)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
