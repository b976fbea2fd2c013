"""Builds the plain C++ oracle (oracle/cpp/oracle.cpp) into oracle/liboracle_c.so with the
host compiler: -O2, no fast-math, no fused multiply-add contraction, OpenMP over output rows.

    python -m oracle.cbuild

Test infrastructure only (see ``oracle/__init__.py``)."""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cpp", "oracle.cpp")
LIB = os.path.join(HERE, "liboracle_c.so")
CXX = os.environ.get("CXX_ORACLE", shutil.which("g++") or "g++")
FLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-Wall"]


def build(verbose: bool = True) -> str:
    tmp = LIB + ".tmp"
    r = subprocess.run([CXX, *FLAGS, SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{r.stderr}")
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
