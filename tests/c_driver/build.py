"""Build tests/c_driver/tfp8_c_driver: a plain C99 program that calls libtfp8.so through
include/tfp8.h (the C ABI as a C caller sees it).  Needs the library built first."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "tfp8_c_driver.c")
EXE = os.path.join(HERE, "tfp8_c_driver")
LIBDIR = os.path.join(ROOT, "fp8_compression_tensor_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    tmp = EXE + ".tmp"
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-isystem", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-o", tmp, SRC, "-L", LIBDIR, "-ltfp8", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           # both found at run time without LD_LIBRARY_PATH, wherever the tree is copied
           "-Wl,-rpath,$ORIGIN/../../fp8_compression_tensor_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed ({r.returncode}):\n{r.stderr}")
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
