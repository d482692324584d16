"""Compile the CPU oracle (plain C, float64) into oracle/libtfp8_oracle.so with gcc.

Test infrastructure only: the product library never links this file's output."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libtfp8_oracle.so")


def build(verbose: bool = False, src: str | None = None, out: str | None = None) -> str:
    """Compile `src` (default: tfp8_oracle.c) into the shared library `out` (default: LIB)."""
    src = src or os.path.join(HERE, "tfp8_oracle.c")
    out = out or LIB
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-I", HERE, "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
