"""Builds the CPU oracle library (test infrastructure) with the host C++
compiler: ``python -m oracle.build_oracle``. Every call recompiles.

The oracle is plain single-threaded C++17; nothing of the HIP library is
compiled or linked into it.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "topktopp_oracle.cpp")
LIB_PATH = os.path.join(HERE, "liboracle_topktopp.so")
FLAGS = ["-O2", "-std=c++17", "-Wall", "-Wextra", "-shared", "-fPIC"]


def compile_oracle(source: str, lib_path: str, opt: str = "-O2") -> str:
    """Compiles one oracle source (the oracle, or a copy with a planted
    mistake in the tests) into a shared library at lib_path."""
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        raise RuntimeError("no host C++ compiler (g++) found to build the oracle")
    tmp = lib_path + ".tmp%d" % os.getpid()
    cmd = [cxx, *[f if f != "-O2" else opt for f in FLAGS], source, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


def build_oracle() -> str:
    return compile_oracle(SOURCE, LIB_PATH)


if __name__ == "__main__":
    print(build_oracle())
    sys.exit(0)
